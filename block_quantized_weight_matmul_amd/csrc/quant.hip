// quant.hip -- the GPU quantizer fp32 -> blocks (the step before the path).
//
// The pages quantize random weights to each type before timing (candle pull
// request "Metal: 64-token tile for the quantized matrix-matrix kernel",
// section "Numbers") and print no quantizer; this library's closed-form
// readings are documented with qmm_quantize in qmm.h.  One thread per block,
// every step in fp64 on the exact fp32 inputs, in the documented order: fp64
// division and the fp16 roundings below are correctly rounded, so the bytes are
// fully determined by the inputs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode.hpp"
#include "internal.hpp"

namespace qmm {
namespace {

// fp16 bits nearest to v (ties to even), from the binary64 value directly (no
// intermediate fp32 rounding).
__device__ u16 f16_rne(double v) {
  const u16 sign = (__double_as_longlong(v) < 0) ? 0x8000 : 0;
  const double a = fabs(v);
  if (a != a) return 0x7E00;
  if (a >= 65520.0) return sign | 0x7C00;  // rounds past the largest finite fp16
  if (a < 0x1p-14) return sign | static_cast<u16>(rint(a * 0x1p24));  // subnormal (1024: the least normal)
  int e;
  frexp(a, &e);                                // a in [2^(e-1), 2^e)
  double m = rint(ldexp(a, 11 - e));           // 11 significant bits, in [1024, 2048]
  int E = e - 1;
  if (m >= 2048.0) { m = 1024.0; ++E; }
  return sign | static_cast<u16>((E + 15) << 10) | static_cast<u16>(static_cast<int>(m) - 1024);
}

__device__ double f16_val(u16 h) { return static_cast<double>(__builtin_bit_cast(_Float16, h)); }

// least fp16 >= v, greatest fp16 <= v
__device__ u16 f16_up(double v) {
  u16 h = f16_rne(v);
  if (f16_val(h) < v) h = (h == 0x0000 || h == 0x8000) ? 0x0001 : ((h & 0x8000) ? h - 1 : h + 1);
  return h;
}
__device__ u16 f16_down(double v) {
  u16 h = f16_rne(v);
  if (f16_val(h) > v) h = (h == 0x0000 || h == 0x8000) ? 0x8001 : ((h & 0x8000) ? h + 1 : h - 1);
  return h;
}

// extremes in index order: the first of equal values wins (this decides the sign
// of zero results: -0 and +0 compare equal)
__device__ void take_min(double& m, double v) { if (v < m) m = v; }
__device__ void take_max(double& m, double v) { if (v > m) m = v; }

__device__ double rha(double v) { return v != 0.0 ? copysign(floor(fabs(v) + 0.5), v) : 0.0; }
__device__ double divz(double a, double b) { return b != 0.0 ? a / b : 0.0; }
__device__ double clampd(double v, double lo, double hi) { return v < lo ? lo : (v > hi ? hi : v); }

__device__ void put16(u8* o, u16 h) { o[0] = static_cast<u8>(h & 0xFF); o[1] = static_cast<u8>(h >> 8); }

__device__ void quant_q4_0(const float* w, u8* o) {
  double ws = w[0];
  for (int i = 1; i < 32; ++i)
    if (fabs(static_cast<double>(w[i])) > fabs(ws)) ws = w[i];
  const u16 hd = f16_rne(ws / -8.0);
  const double d = f16_val(hd);
  put16(o, hd);
  for (int i = 0; i < 16; ++i) {
    int q[2];
    for (int h = 0; h < 2; ++h)
      q[h] = d == 0.0 ? 8 : static_cast<int>(clampd(floor(w[i + 16 * h] / d + 8.5), 0.0, 15.0));
    o[2 + i] = static_cast<u8>(q[0] | (q[1] << 4));
  }
}

__device__ void quant_q8_0(const float* w, u8* o) {
  double amax = fabs(static_cast<double>(w[0]));
  for (int i = 1; i < 32; ++i) take_max(amax, fabs(static_cast<double>(w[i])));
  const u16 hd = f16_rne(amax / 127.0);
  const double d = f16_val(hd);
  put16(o, hd);
  for (int i = 0; i < 32; ++i) {
    const int q = static_cast<int>(clampd(rha(divz(w[i], d)), -127.0, 127.0));
    o[2 + i] = static_cast<u8>(q & 0xFF);
  }
}

__device__ void quant_q4_k(const float* w, u8* o) {
  double lo[8], hi[8];
  double mneg = 0.0;
  for (int j = 0; j < 8; ++j) {
    double mn = w[32 * j], mx = w[32 * j];
    for (int i = 1; i < 32; ++i) {
      take_min(mn, static_cast<double>(w[32 * j + i]));
      take_max(mx, static_cast<double>(w[32 * j + i]));
    }
    lo[j] = mn < 0.0 ? mn : 0.0;
    hi[j] = mx;
    if (j == 0) mneg = -lo[0]; else take_max(mneg, -lo[j]);
  }
  const u16 hdm = f16_up(mneg / 63.0);
  const double dmin = f16_val(hdm);
  int m[8], sc[8];
  double span[8], top = 0.0;
  for (int j = 0; j < 8; ++j) {
    m[j] = static_cast<int>(clampd(ceil(divz(-lo[j], dmin)), 0.0, 63.0));
    span[j] = hi[j] + dmin * m[j];
    if (j == 0) top = span[0] / 15.0; else take_max(top, span[j] / 15.0);
  }
  const u16 hd = f16_up(top / 63.0);
  const double d = f16_val(hd);
  for (int j = 0; j < 8; ++j) sc[j] = static_cast<int>(clampd(ceil(divz(span[j], 15.0 * d)), 0.0, 63.0));
  put16(o, hd);
  put16(o + 2, hdm);
  // sixteen 6-bit fields (sc_0..7, m_0..7), field f at bit 6f of o[4..16)
  for (int i = 0; i < 12; ++i) o[4 + i] = 0;
  for (int f = 0; f < 16; ++f) {
    const int v = f < 8 ? sc[f] : m[f - 8];
    const int bit = 6 * f;
    o[4 + bit / 8] |= static_cast<u8>((v << (bit % 8)) & 0xFF);
    if (bit % 8 > 2) o[4 + bit / 8 + 1] |= static_cast<u8>(v >> (8 - bit % 8));
  }
  for (int p = 0; p < 4; ++p)
    for (int i = 0; i < 32; ++i) {
      int q[2];
      for (int h = 0; h < 2; ++h) {
        const int j = 2 * p + h;
        const double step = d * sc[j];
        q[h] = step == 0.0 ? 0
                           : static_cast<int>(clampd(rha((w[32 * j + i] + dmin * m[j]) / step), 0.0, 15.0));
      }
      o[16 + 32 * p + i] = static_cast<u8>(q[0] | (q[1] << 4));
    }
}

__device__ void quant_q6_k(const float* w, u8* o) {
  double a[16], amax = 0.0;
  for (int j = 0; j < 16; ++j) {
    double mx = fabs(static_cast<double>(w[16 * j]));
    for (int i = 1; i < 16; ++i) take_max(mx, fabs(static_cast<double>(w[16 * j + i])));
    a[j] = mx;
    if (j == 0) amax = mx; else take_max(amax, mx);
  }
  const u16 hd = f16_up(amax / 3937.0);
  const double d = f16_val(hd);
  put16(o, hd);
  int sc[16];
  for (int j = 0; j < 16; ++j) {
    sc[j] = static_cast<int>(clampd(ceil(divz(a[j], 31.0 * d)), 0.0, 127.0));
    o[2 + j] = static_cast<u8>(sc[j]);
  }
  auto code = [&](int i) {
    const int j = i >> 4;
    const double step = d * sc[j];
    return step == 0.0 ? 32 : static_cast<int>(clampd(rha(w[i] / step) + 32.0, 0.0, 63.0));
  };
  for (int i = 0; i < 128; ++i) o[18 + i] = static_cast<u8>((code(i) & 0xF) | ((code(i + 128) & 0xF) << 4));
  for (int i = 0; i < 64; ++i) {
    int v = 0;
    for (int b = 0; b < 4; ++b) v |= ((code(64 * b + i) >> 4) & 3) << (2 * b);
    o[146 + i] = static_cast<u8>(v);
  }
}

__device__ void quant_a4g64(const float* w, u8* o) {
  double mn = w[0], mx = w[0];
  for (int i = 1; i < 64; ++i) {
    take_min(mn, static_cast<double>(w[i]));
    take_max(mx, static_cast<double>(w[i]));
  }
  const u16 hb = f16_down(mn);
  const double bias = f16_val(hb);
  const u16 hs = f16_up((mx - bias) / 15.0);
  const double scale = f16_val(hs);
  put16(o, hs);
  put16(o + 2, hb);
  for (int i = 0; i < 32; ++i) {
    int q[2];
    for (int h = 0; h < 2; ++h)
      q[h] = scale == 0.0 ? 0 : static_cast<int>(clampd(rha((w[i + 32 * h] - bias) / scale), 0.0, 15.0));
    o[4 + i] = static_cast<u8>(q[0] | (q[1] << 4));
  }
}

// block b of the matrix: row b / nb, block b % nb of the row
template <int F>
__global__ __launch_bounds__(256) void k_quantize(const float* w, int64_t K, int64_t nb, int64_t blocks, u8* out) {
  constexpr int BW = FmtInfo<F>::BW, BB = FmtInfo<F>::BB;
  const int64_t b = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (b >= blocks) return;
  const int64_t r = b / nb, c = b - r * nb;
  const float* src = w + r * K + c * BW;
  u8* dst = out + b * BB;
  if constexpr (F == FMT_Q4_0) quant_q4_0(src, dst);
  if constexpr (F == FMT_Q8_0) quant_q8_0(src, dst);
  if constexpr (F == FMT_Q4_K) quant_q4_k(src, dst);
  if constexpr (F == FMT_Q6_K) quant_q6_k(src, dst);
  if constexpr (F == FMT_A4G64) quant_a4g64(src, dst);
}

}  // namespace

hipError_t launch_quantize(int fmt, const float* w, int64_t M, int64_t K, void* out, hipStream_t st) {
  static const int kBW[5] = {32, 32, 256, 256, 64};
  const int64_t nb = K / kBW[fmt];
  const int64_t blocks = M * nb;
  const int64_t grid = (blocks + 255) / 256;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  u8* o = static_cast<u8*>(out);
  switch (fmt) {
    case FMT_Q4_0: hipLaunchKernelGGL(k_quantize<FMT_Q4_0>, dim3(grid), dim3(256), 0, st, w, K, nb, blocks, o); break;
    case FMT_Q8_0: hipLaunchKernelGGL(k_quantize<FMT_Q8_0>, dim3(grid), dim3(256), 0, st, w, K, nb, blocks, o); break;
    case FMT_Q4_K: hipLaunchKernelGGL(k_quantize<FMT_Q4_K>, dim3(grid), dim3(256), 0, st, w, K, nb, blocks, o); break;
    case FMT_Q6_K: hipLaunchKernelGGL(k_quantize<FMT_Q6_K>, dim3(grid), dim3(256), 0, st, w, K, nb, blocks, o); break;
    case FMT_A4G64: hipLaunchKernelGGL(k_quantize<FMT_A4G64>, dim3(grid), dim3(256), 0, st, w, K, nb, blocks, o); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qmm
