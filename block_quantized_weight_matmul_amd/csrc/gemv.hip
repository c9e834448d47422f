// gemv.hip -- matrix-vector paths: dense (1..32 tokens) and expert-indexed.
//
// Lane map.  A "row group" is LPR consecutive lanes of a 64-wide wavefront
// (LPR = 4..64) that share the rows of the group and split the row's 32-weight
// units between them: lane li takes units li, li+LPR, li+2*LPR, ...  The host
// picks LPR from K so that the units divide evenly over the lanes where
// possible -- at K = 512 (16 units) a row takes 16 lanes and a wave holds four
// rows, so no lane idles.  This is the idea of the llama.cpp pull request
// "metal : fix idle threads in mul_mv_iq3_xxs for ne00 < 1024" (section
// "Overview": several lanes per 32-weight chunk row set when there are fewer
// chunks than lanes), generalised: every (row, chunk) pair is computed once,
// and lanes beyond a row's last chunk add nothing (section "Additional
// information").  Each lane carries R rows at once so one load of a chunk of
// activations serves R rows.
//
// Token buckets.  The kernel is instantiated per token bucket NB (1, 2, 3, 4,
// 6, 8, 12, 16, 24, 32) so absent tokens get no registers -- the launch-shape
// idea of the tiny-llm pull request "perf: Optimize quantized matmul for small
// decode batches" (section "Summary"), on the token axis.
//
// Accuracy.  Each unit's 32 products are summed in a fresh fp32 chain, which is
// then added to the lane's accumulator; lanes of a row group are combined by a
// fixed butterfly (DPP within 16 lanes, then cross-row shuffles).  Every weight
// is the exact fp32 dequantized value.
#include <utility>

#include "decode.hpp"
#include "internal.hpp"

namespace qmm {

struct GemvArgs {
  const u8* W;          // block stream of expert 0
  u64 row_bytes;
  u64 expert_bytes;     // M * row_bytes
  int M, nU;            // rows; 32-weight units per row (K / 32)
  int lpr_log2;         // log2(lanes per row group)
  int R;                // rows per lane (must equal the template R)
  const void* x;
  int x_f16;
  int K;                // activation row length
  float* y;
  int N;                // tokens (dense)
  const int32_t* ids;   // expert-indexed mode
  int S, x_per_slot, E;
};

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}

// Sum over the 2^lg consecutive lanes of a row group; every lane of the group
// receives the same value (each step adds a pair of values in both orders,
// which IEEE addition makes identical).
__device__ __forceinline__ float group_sum(float v, int lg) {
  if (lg >= 1) v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
  if (lg >= 2) v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
  if (lg >= 3) v += dpp_mov<0x141>(v);   // row_half_mirror: quads of an 8-lane half
  if (lg >= 4) v += dpp_mov<0x140>(v);   // row_mirror: halves of a 16-lane row
  if (lg >= 5) v += __shfl_xor(v, 16);
  if (lg >= 6) v += __shfl_xor(v, 32);
  return v;
}

// 32 activations x[row][32u .. 32u+31] as fp32.
__device__ __forceinline__ void load_x32(const void* x, int x_f16, int row, int K, int u, float (&v)[32]) {
  if (x_f16) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const h8* p = reinterpret_cast<const h8*>(reinterpret_cast<const _Float16*>(x) + (u64)row * K + 32 * u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const h8 h = p[j];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[8 * j + e] = static_cast<float>(h[e]);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + (u64)row * K + 32 * u);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 f = p[j];
      v[4 * j] = f.x; v[4 * j + 1] = f.y; v[4 * j + 2] = f.z; v[4 * j + 3] = f.w;
    }
  }
}

__device__ __forceinline__ float dot32(const float (&w)[32], const float (&x)[32]) {
  float p = w[0] * x[0];
#pragma unroll
  for (int k = 1; k < 32; ++k) p = __builtin_fmaf(w[k], x[k], p);
  return p;
}

// One wave's share: this lane's row group owns rows row(i) = row_base + i*G + rg
// (i < R; G = row groups per wave), and lane li of the group takes units
// li, li+LPR, ...  Tokens t < ntok read activation row xrow[t] and write y row yrow[t].
template <int F, int NB, int R>
__device__ __forceinline__ void gemv_rows(const u8* W, u64 rb, int M, int nU, int lg, int row_base,
                                          const void* x, int x_f16, int K, const int (&xrow)[NB],
                                          const int (&yrow)[NB], int ntok, float* y) {
  const int lane = threadIdx.x & 63;
  const int LPR = 1 << lg;
  const int G = 64 >> lg;
  const int li = lane & (LPR - 1);
  const int rg = lane >> lg;
  int row[R];
  bool rv[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    row[i] = row_base + i * G + rg;
    rv[i] = row[i] < M;
  }
  float acc[R][NB];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int t = 0; t < NB; ++t) acc[i][t] = 0.0f;

  for (int u = li; u < nU; u += LPR) {
    // rows past M load row M-1 (in bounds); their sums are never stored
    typename Decoder<F>::Raw raw[R];
#pragma unroll
    for (int i = 0; i < R; ++i) Decoder<F>::load(W, (u64)(rv[i] ? row[i] : M - 1) * rb, u, raw[i]);
    if constexpr (NB <= 4) {
      // activations of every token in registers; decode one row at a time
      float xv[NB][32];
#pragma unroll
      for (int t = 0; t < NB; ++t)
        if (t < ntok) load_x32(x, x_f16, xrow[t], K, u, xv[t]);
#pragma unroll
      for (int i = 0; i < R; ++i) {
        Unit o;
        Decoder<F>::unpack(raw[i], o);
        float w[32];
#pragma unroll
        for (int k = 0; k < 32; ++k) w[k] = unit_weight(o, k);
#pragma unroll
        for (int t = 0; t < NB; ++t)
          if (t < ntok) acc[i][t] += dot32(w, xv[t]);
      }
    } else {
      // decoded weights of every row in registers; one token's activations at a time
      float w[R][32];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        Unit o;
        Decoder<F>::unpack(raw[i], o);
#pragma unroll
        for (int k = 0; k < 32; ++k) w[i][k] = unit_weight(o, k);
      }
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        if (t < ntok) {
          float xv[32];
          load_x32(x, x_f16, xrow[t], K, u, xv);
#pragma unroll
          for (int i = 0; i < R; ++i) acc[i][t] += dot32(w[i], xv);
        }
      }
    }
  }

#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      if (t < ntok) {
        const float v = group_sum(acc[i][t], lg);
        if (li == 0 && rv[i]) y[(u64)yrow[t] * M + row[i]] = v;
      }
    }
}

template <int F, int NB, int R>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs a) {
  const int wave = threadIdx.x >> 6;
  const int waves = blockDim.x >> 6;
  const int G = 64 >> a.lpr_log2;
  const int row_base = (blockIdx.x * waves + wave) * (G * R);
  int xrow[NB], yrow[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) xrow[t] = yrow[t] = t;
  gemv_rows<F, NB, R>(a.W, a.row_bytes, a.M, a.nU, a.lpr_log2, row_base, a.x, a.x_f16, a.K, xrow, yrow,
                      a.N, a.y);
}

// Expert-indexed: blockIdx.y = rank k of the expert among the distinct valid ids
// of this call (ascending), blockIdx.x = row tile.  Each workgroup builds, in LDS,
// the presence bitmap of the ids, finds its expert and the (token, slot) pairs
// routed to it, and streams that expert's rows of its tile once per NB pairs.
constexpr int kIdBitmapWords = static_cast<int>(kMaxExperts / 32);
constexpr int kIdMaxPairs = static_cast<int>(kMaxGemvTokens * kMaxSlots);

template <int F, int NB, int R>
__global__ __launch_bounds__(256) void k_gemv_id(GemvArgs a) {
  __shared__ u32 s_bits[kIdBitmapWords];
  __shared__ int s_cnt[256];
  __shared__ int s_pairs[kIdMaxPairs];
  __shared__ int s_expert, s_npairs;

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int P = a.N * a.S;
  const int nwords = (a.E + 31) >> 5;
  const int wave = threadIdx.x >> 6;
  const int waves = blockDim.x >> 6;
  const int G = 64 >> a.lpr_log2;
  const int rows_per_wg = waves * G * R;
  const int row_tile0 = blockIdx.x * rows_per_wg;

  for (int w = tid; w < nwords; w += nthr) s_bits[w] = 0u;
  if (tid == 0) { s_expert = -1; s_npairs = 0; }
  __syncthreads();
  for (int p = tid; p < P; p += nthr) {
    const int e = a.ids[p];
    if (e >= 0 && e < a.E) atomicOr(&s_bits[e >> 5], 1u << (e & 31));
  }
  __syncthreads();

  // k-th set bit: thread t counts words [t*wpt, (t+1)*wpt), then an exclusive scan.
  const int k = blockIdx.y;
  const int wpt = (nwords + nthr - 1) / nthr;
  int cnt = 0;
  for (int w = tid * wpt; w < min(nwords, (tid + 1) * wpt); ++w) cnt += __popc(s_bits[w]);
  s_cnt[tid] = cnt;
  __syncthreads();
  for (int off = 1; off < nthr; off <<= 1) {
    const int v = tid >= off ? s_cnt[tid - off] : 0;
    __syncthreads();
    s_cnt[tid] += v;
    __syncthreads();
  }
  const int incl = s_cnt[tid];
  const int excl = incl - cnt;
  if (k >= excl && k < incl) {
    int seen = excl;
    for (int w = tid * wpt; w < min(nwords, (tid + 1) * wpt); ++w) {
      u32 bits = s_bits[w];
      while (bits) {
        const int b = __ffs(bits) - 1;
        if (seen == k) s_expert = (w << 5) + b;
        ++seen;
        bits &= bits - 1u;
      }
    }
  }
  __syncthreads();
  const int e = s_expert;

  // Ids outside [0, E) have no matrix: their output rows are NaN (written by the
  // rank-0 workgroups, which exist for every row tile).
  if (blockIdx.y == 0) {
    const float qnan = __builtin_nanf("");
    const int rows = min(rows_per_wg, a.M - row_tile0);
    for (int p = 0; p < P; ++p) {
      const int id = a.ids[p];
      if (id < 0 || id >= a.E)
        for (int r = tid; r < rows; r += nthr) a.y[(u64)p * a.M + row_tile0 + r] = qnan;
    }
  }
  if (e < 0) return;  // uniform over the workgroup

  for (int p = tid; p < P; p += nthr)
    if (a.ids[p] == e) s_pairs[atomicAdd(&s_npairs, 1)] = p;
  __syncthreads();
  const int np = s_npairs;

  const u8* W = a.W + (u64)e * a.expert_bytes;
  const int row_base = row_tile0 + wave * (G * R);
  for (int c0 = 0; c0 < np; c0 += NB) {
    const int ntok = min(NB, np - c0);
    int xrow[NB], yrow[NB];
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const int p = t < ntok ? s_pairs[c0 + t] : 0;
      xrow[t] = a.x_per_slot ? p : p / a.S;
      yrow[t] = p;
    }
    gemv_rows<F, NB, R>(W, a.row_bytes, a.M, a.nU, a.lpr_log2, row_base, a.x, a.x_f16, a.K, xrow, yrow,
                        ntok, a.y);
  }
}

// ---------------------------------------------------------------------------------------------
// Host side: instance tables and launch-shape choice.

namespace {

constexpr int kBuckets[] = {1, 2, 3, 4, 6, 8, 12, 16, 24, 32};
constexpr int kNumBuckets = sizeof(kBuckets) / sizeof(kBuckets[0]);

int bucket_index(int n) {
  for (int i = 0; i < kNumBuckets; ++i)
    if (n <= kBuckets[i]) return i;
  return -1;
}

// Rows per lane for a token bucket: more rows share each activation load when
// activations sit in registers (NB <= 4); fewer rows keep registers in check above.
constexpr int rows_per_lane(int NB) { return NB <= 2 ? 4 : (NB <= 8 ? 2 : 1); }

typedef void (*GemvKernel)(GemvArgs);

template <int F, int BI>
constexpr GemvKernel dense_kernel() {
  return k_gemv<F, kBuckets[BI], rows_per_lane(kBuckets[BI])>;
}
template <int F, int BI>
constexpr GemvKernel id_kernel() {
  return k_gemv_id<F, kBuckets[BI], rows_per_lane(kBuckets[BI])>;
}

template <int F, int... BI>
constexpr void fill_dense(GemvKernel* t, std::integer_sequence<int, BI...>) {
  ((t[BI] = dense_kernel<F, BI>()), ...);
}
template <int F, int... BI>
constexpr void fill_id(GemvKernel* t, std::integer_sequence<int, BI...>) {
  ((t[BI] = id_kernel<F, BI>()), ...);
}

struct Tables {
  GemvKernel dense[5][kNumBuckets];
  GemvKernel id[5][kNumBuckets];
  Tables() {
    auto seq = std::make_integer_sequence<int, kNumBuckets>{};
    fill_dense<FMT_Q4_0>(dense[FMT_Q4_0], seq);
    fill_dense<FMT_Q8_0>(dense[FMT_Q8_0], seq);
    fill_dense<FMT_Q4_K>(dense[FMT_Q4_K], seq);
    fill_dense<FMT_Q6_K>(dense[FMT_Q6_K], seq);
    fill_dense<FMT_A4G64>(dense[FMT_A4G64], seq);
    fill_id<FMT_Q4_0>(id[FMT_Q4_0], seq);
    fill_id<FMT_Q8_0>(id[FMT_Q8_0], seq);
    fill_id<FMT_Q4_K>(id[FMT_Q4_K], seq);
    fill_id<FMT_Q6_K>(id[FMT_Q6_K], seq);
    fill_id<FMT_A4G64>(id[FMT_A4G64], seq);
  }
};

const Tables& tables() {
  static const Tables t;
  return t;
}

// Lanes per row group: the power of two in 4..64 that leaves the fewest lanes
// idle on the last pass over the row's units (ties go to the wider group).
int choose_lpr_log2(int nU) {
  int best = 6;
  long best_idle = 0, best_slots = 1;
  for (int lg = 6; lg >= 2; --lg) {
    const long L = 1L << lg;
    const long slots = ((nU + L - 1) / L) * L;
    const long idle = slots - nU;
    if (lg == 6 || idle * best_slots < best_idle * slots) {  // strictly fewer idle lanes (fraction)
      best = lg;
      best_idle = idle;
      best_slots = slots;
    }
  }
  return best;
}

struct Shape {
  int lg, R, waves, rows_per_wg;
};

Shape gemv_shape(int nU, int M, int NB) {
  Shape s;
  s.lg = choose_lpr_log2(nU);
  s.R = rows_per_lane(NB);
  const int rows_per_wave = (64 >> s.lg) * s.R;
  // up to 4 waves per workgroup while that still leaves >= 512 workgroups
  s.waves = 4;
  while (s.waves > 1 && (M + s.waves * rows_per_wave - 1) / (s.waves * rows_per_wave) < 512) s.waves >>= 1;
  s.rows_per_wg = s.waves * rows_per_wave;
  return s;
}

}  // namespace

hipError_t launch_gemv(const MatDesc& m, const void* x, int x_f16, int N, float* y, hipStream_t st) {
  const int bi = bucket_index(N);
  if (bi < 0) return hipErrorInvalidValue;
  const int nU = static_cast<int>(m.K / 32);
  const Shape s = gemv_shape(nU, static_cast<int>(m.M), kBuckets[bi]);
  GemvArgs a{};
  a.W = m.blocks;
  a.row_bytes = m.row_bytes;
  a.expert_bytes = m.row_bytes * static_cast<u64>(m.M);
  a.M = static_cast<int>(m.M);
  a.nU = nU;
  a.lpr_log2 = s.lg;
  a.R = s.R;
  a.x = x;
  a.x_f16 = x_f16;
  a.K = static_cast<int>(m.K);
  a.y = y;
  a.N = N;
  const dim3 grid((m.M + s.rows_per_wg - 1) / s.rows_per_wg);
  hipLaunchKernelGGL(tables().dense[m.fmt][bi], grid, dim3(64 * s.waves), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gemv_id(const MatDesc& m, const void* x, int x_f16, int N, int S, int x_per_slot,
                          const int32_t* ids, float* y, hipStream_t st) {
  // pairs per expert: at most N when a token's ids are distinct; larger counts
  // (duplicate ids) are processed in further passes of NB pairs
  const int bi = bucket_index(N < 8 ? N : 8);
  if (bi < 0) return hipErrorInvalidValue;
  const int nU = static_cast<int>(m.K / 32);
  Shape s = gemv_shape(nU, static_cast<int>(m.M), kBuckets[bi]);
  GemvArgs a{};
  a.W = m.blocks;
  a.row_bytes = m.row_bytes;
  a.expert_bytes = m.row_bytes * static_cast<u64>(m.M);
  a.M = static_cast<int>(m.M);
  a.nU = nU;
  a.lpr_log2 = s.lg;
  a.R = s.R;
  a.x = x;
  a.x_f16 = x_f16;
  a.K = static_cast<int>(m.K);
  a.y = y;
  a.N = N;
  a.ids = ids;
  a.S = S;
  a.x_per_slot = x_per_slot;
  a.E = static_cast<int>(m.n_experts);
  const int64_t P = static_cast<int64_t>(N) * S;
  const int ranks = static_cast<int>(P < m.n_experts ? P : m.n_experts);
  const dim3 grid((m.M + s.rows_per_wg - 1) / s.rows_per_wg, ranks);
  hipLaunchKernelGGL(tables().id[m.fmt][bi], grid, dim3(64 * s.waves), 0, st, a);
  return hipGetLastError();
}

}  // namespace qmm
