// gemm.hip -- token-tiled matrix-matrix path on the gfx950 matrix cores.
//
// Candle pull request "Metal: 64-token tile for the quantized matrix-matrix
// kernel": a workgroup owns a tile of weight rows; on every step along K it
// reads those rows' blocks, dequantizes them once into LDS and multiplies them
// by the tokens of its tile (section "Why the tile sets the weight reuse"), so
// each weight is fetched and decoded once per token tile.  The tile is 32 or
// 64 tokens (section "What changes"), and the two tiles must give bit-identical
// outputs (section "Same results, bit for bit").
//
// Here: MT = 64 weight rows x T tokens per workgroup of 4 waves.  Per K step of
// KC = 128 weights, each thread decodes one 32-weight unit to fp32 (the exact
// dequantized value), rounds it to fp16 (nearest even) and writes it to LDS; the
// activation tile is staged as fp16 beside it.  Wave w then owns weight rows
// 16w .. 16w+15 and all T tokens: for each 32-deep slice it issues one
// v_mfma_f32_16x16x32_f16 per 16-token block, accumulating in fp32.
//
// Bit identity of the two tiles: an output (row r, token t) is always produced
// by the wave owning rows 16*floor((r % 64)/16), in the accumulator of token
// block floor((t % T)/16), at lane position (r % 16, t % 16), from the same
// LDS values, over the same K steps in the same order.  Only the number of
// token blocks per wave differs between T = 32 and T = 64.
#include <climits>

#include "decode.hpp"
#include "internal.hpp"

namespace qmm {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
  const u8* W;
  u64 row_bytes;
  int M, nU, K;
  const void* x;
  int x_f16;
  int N;
  float* y;
  int n_row_tiles;  // ceil(M / kMT); blockIdx.x = token_tile * n_row_tiles + row_tile
};

constexpr int kMT = 64;         // weight rows per workgroup
constexpr int kKC = 128;        // K per LDS stage (4 units)
constexpr int kKP = kKC + 8;    // padded LDS row length (halves)

__device__ __forceinline__ half8 cvt8(const float* f) {
  half8 h;
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = static_cast<_Float16>(f[e]);
  return h;
}

template <int F, int T>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 sW[kMT][kKP];
  __shared__ __attribute__((aligned(16))) _Float16 sX[T][kKP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row0 = (blockIdx.x % a.n_row_tiles) * kMT;
  const int tok0 = (blockIdx.x / a.n_row_tiles) * T;

  floatx4 acc[T / 16];
#pragma unroll
  for (int b = 0; b < T / 16; ++b) acc[b] = floatx4{0.f, 0.f, 0.f, 0.f};

  constexpr int kTPT = 256 / T;       // threads per token row of the activation tile
  constexpr int kHPT = kKC / kTPT;    // halves per thread (32 or 16)

  for (int u0 = 0; u0 < a.nU; u0 += kKC / 32) {
    // weights: thread -> (row tid/4, unit u0 + tid%4)
    {
      const int r = tid >> 2;
      const int uu = tid & 3;
      const int row = row0 + r;
      const int u = u0 + uu;
      half8* dst = reinterpret_cast<half8*>(&sW[r][32 * uu]);
      if (row < a.M && u < a.nU) {
        float w[32];
        decode_unit<F>(a.W, static_cast<u32>(row) * static_cast<u32>(a.row_bytes), u, w);
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j] = cvt8(&w[8 * j]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j] = half8{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
    // activations: thread -> (token tid/kTPT, halves [c*kHPT, (c+1)*kHPT))
    {
      const int t = tid / kTPT;
      const int c = tid % kTPT;
      const int tok = tok0 + t;
      const int kb = 32 * u0 + c * kHPT;
#pragma unroll
      for (int h = 0; h < kHPT / 8; ++h) {
        const int k = kb + 8 * h;
        half8 v = half8{0, 0, 0, 0, 0, 0, 0, 0};
        if (tok < a.N && k < a.K) {
          if (a.x_f16) {
            v = *reinterpret_cast<const half8*>(reinterpret_cast<const _Float16*>(a.x) + (u64)tok * a.K + k);
          } else {
            const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.x) + (u64)tok * a.K + k);
            const float4 f0 = p[0], f1 = p[1];
            const float f[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
            v = cvt8(f);
          }
        }
        *reinterpret_cast<half8*>(&sX[t][c * kHPT + 8 * h]) = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kKC / 32; ++ks) {
      const half8 A = *reinterpret_cast<const half8*>(&sW[16 * wave + (lane & 15)][32 * ks + 8 * (lane >> 4)]);
#pragma unroll
      for (int b = 0; b < T / 16; ++b) {
        const half8 B = *reinterpret_cast<const half8*>(&sX[16 * b + (lane & 15)][32 * ks + 8 * (lane >> 4)]);
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, acc[b], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // D[i][j] of a 16x16 block sits in lane j + 16*(i/4), element i%4.
#pragma unroll
  for (int b = 0; b < T / 16; ++b) {
    const int tok = tok0 + 16 * b + (lane & 15);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = row0 + 16 * wave + 4 * (lane >> 4) + v;
      if (tok < a.N && row < a.M) a.y[(u64)tok * a.M + row] = acc[b][v];
    }
  }
}

namespace {
typedef void (*GemmKernel)(GemmArgs);
template <int F>
GemmKernel pick(int T) {
  return T == 64 ? k_gemm<F, 64> : k_gemm<F, 32>;
}
}  // namespace

hipError_t launch_gemm(const MatDesc& m, const void* x, int x_f16, int64_t N, float* y, int tile,
                       hipStream_t st) {
  GemmArgs a{};
  a.W = m.blocks;
  a.row_bytes = m.row_bytes;
  a.M = static_cast<int>(m.M);
  a.nU = static_cast<int>(m.K / 32);
  a.K = static_cast<int>(m.K);
  a.x = x;
  a.x_f16 = x_f16;
  a.N = static_cast<int>(N);
  a.y = y;
  GemmKernel k = nullptr;
  switch (m.fmt) {
    case FMT_Q4_0: k = pick<FMT_Q4_0>(tile); break;
    case FMT_Q8_0: k = pick<FMT_Q8_0>(tile); break;
    case FMT_Q4_K: k = pick<FMT_Q4_K>(tile); break;
    case FMT_Q6_K: k = pick<FMT_Q6_K>(tile); break;
    case FMT_A4G64: k = pick<FMT_A4G64>(tile); break;
    default: return hipErrorInvalidValue;
  }
  a.n_row_tiles = static_cast<int>((m.M + kMT - 1) / kMT);
  const int64_t blocks = static_cast<int64_t>(a.n_row_tiles) * ((N + tile - 1) / tile);
  if (blocks > INT_MAX) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
  hipLaunchKernelGGL(k, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace qmm
