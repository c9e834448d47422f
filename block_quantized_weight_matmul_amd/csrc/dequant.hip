// dequant.hip -- decode a whole matrix to fp32 (the exact dequantized weights) or
// to fp16 (round to nearest even of those: the values the matrix-matrix path
// stages in LDS).  One thread per 32-weight unit.
#include "decode.hpp"
#include "internal.hpp"

namespace qmm {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

template <int F>
__global__ __launch_bounds__(256) void k_dequant(const u8* W, u64 rb, int M, int nU, void* out, int out_f16) {
  const u64 idx = (u64)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (u64)M * nU) return;
  const int row = static_cast<int>(idx / nU);
  const int u = static_cast<int>(idx % nU);
  float w[32];
  decode_unit<F>(W, static_cast<u32>(row) * static_cast<u32>(rb), u, w);
  const u64 base = (u64)row * nU * 32 + 32ull * u;
  if (out_f16) {
    half8* p = reinterpret_cast<half8*>(reinterpret_cast<_Float16*>(out) + base);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half8 h;
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = static_cast<_Float16>(w[8 * j + e]);
      p[j] = h;
    }
  } else {
    float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + base);
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = make_float4(w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]);
  }
}

hipError_t launch_dequant(const MatDesc& m, int64_t expert, void* out, int out_f16, hipStream_t st) {
  const u8* W = m.blocks + static_cast<u64>(expert) * m.row_bytes * static_cast<u64>(m.M);
  const int nU = static_cast<int>(m.K / 32);
  const u64 units = static_cast<u64>(m.M) * nU;
  if ((units + 255) / 256 > 0x7FFFFFFFull) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>((units + 255) / 256));
  void (*k)(const u8*, u64, int, int, void*, int) = nullptr;
  switch (m.fmt) {
    case FMT_Q4_0: k = k_dequant<FMT_Q4_0>; break;
    case FMT_Q8_0: k = k_dequant<FMT_Q8_0>; break;
    case FMT_Q4_K: k = k_dequant<FMT_Q4_K>; break;
    case FMT_Q6_K: k = k_dequant<FMT_Q6_K>; break;
    case FMT_A4G64: k = k_dequant<FMT_A4G64>; break;
    case FMT_Q4_1: k = k_dequant<FMT_Q4_1>; break;
    case FMT_Q5_0: k = k_dequant<FMT_Q5_0>; break;
    case FMT_Q5_1: k = k_dequant<FMT_Q5_1>; break;
    case FMT_Q2_K: k = k_dequant<FMT_Q2_K>; break;
    case FMT_Q3_K: k = k_dequant<FMT_Q3_K>; break;
    case FMT_Q5_K: k = k_dequant<FMT_Q5_K>; break;
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(k, grid, dim3(256), 0, st, W, m.row_bytes, static_cast<int>(m.M), nU, out, out_f16);
  return hipGetLastError();
}

}  // namespace qmm
