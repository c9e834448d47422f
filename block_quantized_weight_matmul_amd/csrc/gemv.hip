// gemv.hip -- matrix-vector paths: dense (1..32 tokens) and expert-indexed.
//
// Work items.  The unit of work is one "item": one row's 32-weight unit (one
// Q4_0/Q8_0 block, half an A4G64 group, a Q4_K sub-block, two Q6_K sub-blocks)
// against every token of the call.  A workgroup owns a contiguous slice of
// RW rows and spreads the slice's RW * (K/32) items over its threads, item
// index = row * units + unit, thread t taking items t, t + T, t + 2T, ...  So
// consecutive lanes read consecutive units of a row (coalesced; units that
// share code bytes are read by neighbouring lanes of one instruction), and no
// lane idles whatever K is: at K = 512 a wavefront covers four rows of 16
// units.  This is the idea of the llama.cpp pull request "metal : fix idle
// threads in mul_mv_iq3_xxs for ne00 < 1024" (section "Overview": when a row
// has fewer 32-weight chunks than lanes, lanes share the chunks of several
// rows), taken to its end: every (row, chunk) pair is computed exactly once
// (section "Additional information").
//
// Latency.  Grids hold one or two workgroups per CU, sized so each thread has
// at most four items; a thread issues the loads of all its items before it
// decodes the first, so a workgroup's weight bytes are in flight at once.
// Activations are staged in LDS once per workgroup (in K chunks when they do
// not fit) together with the sum of each 16-activation half: the only global
// loads of the item loop are weight bytes (global loads retire in order for
// s_waitcnt, so an activation load behind a weight prefetch would wait out the
// prefetch).
//
// Token buckets.  Kernels are instantiated per token bucket NB (1, 2, 3, 4, 6,
// 8, 12, 16, 24, 32) so absent tokens get no registers -- the launch-shape
// idea of the tiny-llm pull request "perf: Optimize quantized matmul for small
// decode batches" (section "Summary"), on the token axis.
//
// Arithmetic.  With w = a*q + b on each 16-weight half of a unit (one (a, b)
// pair per half; both halves share it except in Q6_K), an item's partial sum
// is a0*Sq0 + b0*Sx0 + a1*Sq1 + b1*Sx1 with Sq = sum q*x over the half (a fresh
// 16-term fp32 chain) and Sx the staged half sum: one conversion and one fma
// per weight and token.  Partials go to LDS; each output is then the sum of its
// row's partials in a fixed order (lane l adds units l, l+64, ...; then a
// butterfly over the wave), so results are deterministic and independent of
// the launch shape, and the dense and expert-indexed paths agree bit for bit.
#include <climits>
#include <type_traits>
#include <utility>

#include "decode.hpp"
#include "internal.hpp"

namespace qmm {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

struct GemvArgs {
  const u8* W;          // block stream of expert 0
  u64 row_bytes;
  u64 expert_bytes;     // M * row_bytes
  int M, nU, K;         // rows; 32-weight units per row (K / 32); activation row length
  int rows_per_wg;      // RW
  int chunk_units;      // units of activations staged in LDS at a time
  const void* x;
  int x_f16;
  float* y;
  int N;                // tokens (dense)
  const int32_t* ids;   // expert-indexed mode
  int S, x_per_slot, E;
  int tok_groups;       // multi-token kernel: token groups of threads
  int tok_pass;         // multi-token kernel: tokens staged per pass
};

// Matrices of one one-token launch: the same format and K, each with its own blocks,
// activations and outputs; matrix i takes workgroups first[i] .. first[i + 1] - 1.
struct GemvGroup {
  const u8* W[kGemvGroupMax];
  const void* x[kGemvGroupMax];
  float* y[kGemvGroupMax];
  int M[kGemvGroupMax];
  int first[kGemvGroupMax + 1];
  int n;
  int fmt_b;  // k_gemv1_pair: bit i set when matrix i is of its second format
};

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}

// Sum over the 64 lanes of a wave; every lane receives the same value (each step
// adds a pair of values in both orders, which IEEE addition makes identical).
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp_mov<0x141>(v);   // row_half_mirror: quads of an 8-lane half
  v += dpp_mov<0x140>(v);   // row_mirror: halves of a 16-lane row
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Token t of a call reads activation row tm.x(t) and writes output row tm.y(t):
// the identity for the dense path; for the expert-indexed path, t indexes the
// LDS list of (token, slot) pairs routed to the workgroup's expert.
struct TokMap {
  const int* pairs;  // LDS, or nullptr for the identity
  int S;             // slots per token
  int per_slot;      // activations per (token, slot) rather than per token
  __device__ __forceinline__ int x(int t) const {
    if (!pairs) return t;
    const int p = pairs[t];
    return per_slot ? p : p / S;
  }
  __device__ __forceinline__ int y(int t) const { return pairs ? pairs[t] : t; }
};

// LDS layout (floats).  Staged activations: token t, chunk unit uu at
// (t * KC + uu) * kXStride (4 pad floats per unit spread consecutive units over
// the LDS banks); their half sums at sx[(t * KC + uu) * 2 + h]; item partials at
// part[(t * RW + row) * nU + u].
constexpr int kXStride = 36;

__host__ __device__ constexpr int lds_floats(int NB, int KC, int RW, int nU) {
  return NB * KC * (kXStride + 2) + NB * RW * nU;
}

// The sum of 16 activations as a balanced pairwise tree: ((e0+e1)+(e2+e3)) for
// each group of four, then the groups pairwise.  Both staging routines form
// exactly this tree, so every path sees the same half sums.
__device__ __forceinline__ float sum4(float a, float b, float c, float d) { return (a + b) + (c + d); }
__device__ __forceinline__ float half_sum16(const float* p) {
  return (sum4(p[0], p[1], p[2], p[3]) + sum4(p[4], p[5], p[6], p[7])) +
         (sum4(p[8], p[9], p[10], p[11]) + sum4(p[12], p[13], p[14], p[15]));
}

// The activation chunk can instead pass through registers: x_load issues its
// global loads (kXRegs 16-byte slots per thread, 4 fp32 or 8 fp16 activations
// each; slot indices past the chunk are clamped, so the loads carry no branch)
// and x_put converts, writes them to LDS and forms the half sums with DPP.  A
// caller issues x_load before the weight loads: global loads retire in order for
// s_waitcnt, so the LDS store then waits for the activations only and the weight
// bytes stay in flight while they are staged.
constexpr int kXRegs = 8;
struct XRegs {
  uint4 v[kXRegs];
};

__device__ __forceinline__ int x_slots_per_unit(int x_f16) { return x_f16 ? 4 : 8; }

__device__ __forceinline__ bool x_fits_regs(int x_f16, int ntok, int cw) {
  return ntok * cw * x_slots_per_unit(x_f16) <= kXRegs * (int)blockDim.x;
}

__device__ __forceinline__ void x_load(const void* x, int x_f16, int K, const TokMap& tm, int ntok, int c0, int cw,
                                       XRegs& r, int base = 0) {
  const int spu = x_slots_per_unit(x_f16);
  const int es = x_f16 ? 2 : 4;
  const int per_tok = cw * spu;
  const int total = ntok * per_tok;
  const u8* xb = reinterpret_cast<const u8*>(x);
#pragma unroll
  for (int j = 0; j < kXRegs; ++j) {
    if (base + j * static_cast<int>(blockDim.x) < total) {  // uniform: slot rounds the chunk needs
      const int idx = min(base + static_cast<int>(threadIdx.x + j * blockDim.x), total - 1);
      const int t = idx / per_tok;
      const int rem = idx - t * per_tok;
      const int uu = rem / spu;
      const u64 off = ((u64)tm.x(t) * K + 32 * (c0 + uu)) * es + 16 * (rem - uu * spu);
      r.v[j] = *reinterpret_cast<const uint4*>(xb + off);
    }
  }
}

__device__ __forceinline__ void x_put(const XRegs& r, int x_f16, int ntok, int cw, int KC, float* s_x,
                                      float* s_sx, int base = 0) {
  const int spu = x_slots_per_unit(x_f16);
  const int per_tok = cw * spu;
  const int total = ntok * per_tok;
#pragma unroll
  for (int j = 0; j < kXRegs; ++j) {
    if (base + j * static_cast<int>(blockDim.x) >= total) break;  // uniform
    const int idx = base + threadIdx.x + j * blockDim.x;
    const int ic = min(idx, total - 1);
    const int t = ic / per_tok;
    const int rem = ic - t * per_tok;
    const int uu = rem / spu;
    const int q = rem - uu * spu;
    float* dst = &s_x[(t * KC + uu) * kXStride];
    float hs;
    if (x_f16) {
      // 8 activations; a half is two slots (lanes 2k, 2k+1)
      typedef _Float16 h8 __attribute__((ext_vector_type(8)));
      const h8 h = __builtin_bit_cast(h8, r.v[j]);
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = static_cast<float>(h[e]);
      if (idx < total) {
        *reinterpret_cast<float4*>(dst + 8 * q) = make_float4(f[0], f[1], f[2], f[3]);
        *reinterpret_cast<float4*>(dst + 8 * q + 4) = make_float4(f[4], f[5], f[6], f[7]);
      }
      hs = sum4(f[0], f[1], f[2], f[3]) + sum4(f[4], f[5], f[6], f[7]);
      hs += dpp_mov<0xB1>(hs);  // + slot of lane ^ 1
    } else {
      // 4 activations; a half is four slots (lanes 4k .. 4k+3)
      const float4 v = __builtin_bit_cast(float4, r.v[j]);
      if (idx < total) *reinterpret_cast<float4*>(dst + 4 * q) = v;
      hs = sum4(v.x, v.y, v.z, v.w);
      hs += dpp_mov<0xB1>(hs);  // lane ^ 1
      hs += dpp_mov<0x4E>(hs);  // lane ^ 2
    }
    // the first slot of each half writes its sum
    if (idx < total && (q & (spu / 2 - 1)) == 0) s_sx[(t * KC + uu) * 2 + q / (spu / 2)] = hs;
  }
}

// Stage a chunk too large for one register round: rounds of kXRegs slots per
// thread, each issuing all its loads before its stores.
__device__ __forceinline__ void stage_x(const void* x, int x_f16, int K, const TokMap& tm, int ntok, int c0, int cw,
                                        int KC, float* s_x, float* s_sx) {
  const int total = ntok * cw * x_slots_per_unit(x_f16);
  for (int base = 0; base < total; base += kXRegs * static_cast<int>(blockDim.x)) {
    XRegs xr;
    x_load(x, x_f16, K, tm, ntok, c0, cw, xr, base);
    x_put(xr, x_f16, ntok, cw, KC, s_x, s_sx, base);
  }
}

__device__ __forceinline__ void read_x32(const float* s_x, float (&v)[32]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float4 f = *reinterpret_cast<const float4*>(s_x + 4 * j);
    v[4 * j] = f.x; v[4 * j + 1] = f.y; v[4 * j + 2] = f.z; v[4 * j + 3] = f.w;
  }
}

// sum of q[i]*x[i] over one 16-weight half (first product, then 15 fmas)
__device__ __forceinline__ float half_dot(const float (&q)[32], const float (&x)[32], int h) {
  float s = q[16 * h] * x[16 * h];
#pragma unroll
  for (int i = 1; i < 16; ++i) s = __builtin_fmaf(q[16 * h + i], x[16 * h + i], s);
  return s;
}

// The same half sum with each code read as an fp16 subnormal, code * 2^-24, and
// multiplied by x with v_fma_mix_f32 (fp16 operand widened inside the fma): two
// codes per 32-bit word, built with one and (weights 4j, 4j+2) and one byte
// permute (weights 4j+1, 4j+3), instead of one conversion per code.  code * 2^-24
// widens exactly, so every product and partial sum is the one of half_dot scaled
// by 2^-24, exactly, while it stays a normal fp32 number (|x| above ~2^-100);
// the caller scales the coefficient by 2^24 instead.  Codes carry no bias.
__device__ __forceinline__ float code_lo(u32 v) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<u16>(v & 0xFFFFu)));
}
__device__ __forceinline__ float code_hi(u32 v) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<u16>(v >> 16)));
}
// An item's codes as fp16 pairs: ev[r][k] holds the codes of weights 4k and 4k+2
// of run r (low and high half), od[r][k] those of 4k+1 and 4k+3; run r's codes
// are scaled by 2^sh[r] (a high nibble left in place is 16*code).  The default
// takes the unit's code bytes apart; Q4_K and Q6_K build the pairs from the raw
// bytes directly, which saves a mask per word.
template <int F>
struct MixPairs {
  static constexpr int RUNS = Item<F>::RUNS;
  u32 ev[RUNS][8], od[RUNS][8];
  static constexpr int sh(int) { return 0; }
  __device__ __forceinline__ void make(const typename Item<F>::Raw&, const Unit (&o)[RUNS]) {
#pragma unroll
    for (int r = 0; r < RUNS; ++r)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        ev[r][k] = o[r].c[k] & 0x00FF00FFu;
        od[r][k] = __builtin_amdgcn_perm(o[r].c[k], o[r].c[k], 0x0C030C01u);
      }
  }
};

// bytes 1 and 3 of v moved to bytes 0 and 2, zeros above them
__device__ __forceinline__ u32 odd_bytes(u32 v) { return __builtin_amdgcn_perm(v, v, 0x0C030C01u); }

template <>
struct MixPairs<FMT_Q4_K> {
  u32 ev[2][8], od[2][8];
  static constexpr int sh(int) { return 0; }  // run 1 already carries a/16
  __device__ __forceinline__ void make(const Item<FMT_Q4_K>::Raw& w, const Unit (&)[2]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const u32 t = odd_bytes(w.q[k]);
      ev[0][k] = w.q[k] & 0x000F000Fu;
      od[0][k] = t & 0x000F000Fu;
      ev[1][k] = w.q[k] & 0x00F000F0u;
      od[1][k] = t & 0x00F000F0u;
    }
  }
};

// Q6_K: run 0 code = low nibble | qh bits (hs, hs+1) << 4; run 1 keeps the high
// nibble in place and puts qh bits (hs+4, hs+5) at bits 8, 9: 16 * code (< 1024).
template <>
struct MixPairs<FMT_Q6_K> {
  u32 ev[2][8], od[2][8];
  static constexpr int sh(int r) { return r == 1 ? 4 : 0; }
  __device__ __forceinline__ void make(const Item<FMT_Q6_K>::Raw& w, const Unit (&)[2]) {
    const u32 up = 4u - 2u * static_cast<u32>(w.a >> 1);  // 4 - hs
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const u32 ql = w.ql.word(k), qh = w.qh.word(k);
      const u32 t = qh << up, qlo = odd_bytes(ql), tod = odd_bytes(qh) << up;
      ev[0][k] = (ql & 0x000F000Fu) | (t & 0x00300030u);
      ev[1][k] = (ql & 0x00F000F0u) | (t & 0x03000300u);
      od[0][k] = (qlo & 0x000F000Fu) | (tod & 0x00300030u);
      od[1][k] = (qlo & 0x00F000F0u) | (tod & 0x03000300u);
    }
  }
};

// Q8_0: signed byte codes.  A pair is built as the fp16 normals 1024 + (q + 128), from
// which 1152 is subtracted in packed fp16 -- exact, all integers below 2048 -- so it holds
// q itself (sh = 24: no 2^-24 scaling), and every product and partial sum is item_partial's
// with the codes as signed floats, bit for bit.
template <>
struct MixPairs<FMT_Q8_0> {
  u32 ev[1][8], od[1][8];
  static constexpr int sh(int) { return 24; }
  __device__ __forceinline__ void make(const Item<FMT_Q8_0>::Raw& w, const Unit (&)[1]) {
    const half2v off = {1152, 1152};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const u32 c = w.q.word(k) ^ 0x80808080u;  // q + 128
      const half2v e = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, c, 0x04020400u)) - off;
      const half2v o = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, c, 0x04030401u)) - off;
      ev[0][k] = __builtin_bit_cast(u32, e);
      od[0][k] = __builtin_bit_cast(u32, o);
    }
  }
};

// All 2*RUNS half sums of an item, in lockstep: the chains are independent, and
// interleaving them keeps one chain's dependent fmas apart.
template <int F, int RUNS>
__device__ __forceinline__ void half_dots_mix(const MixPairs<F>& p, const float (&x)[RUNS][32],
                                              float (&s)[RUNS][2]) {
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int r = 0; r < RUNS; ++r)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32 w = e & 1 ? p.od[r][4 * h + k] : p.ev[r][4 * h + k];
          const float q = e < 2 ? code_lo(w) : code_hi(w);
          const float xv = x[r][16 * h + 4 * k + e];
          s[r][h] = k == 0 && e == 0 ? q * xv : __builtin_fmaf(q, xv, s[r][h]);
        }
}

// An item's partial sum a0*Sq0 + b0*Sx0 + a1*Sq1 + b1*Sx1 (Q8_0 has no b terms).
template <int F>
__device__ __forceinline__ float item_partial(const Unit& o, const float (&q)[32], const float (&x)[32],
                                              float sx0, float sx1) {
  const float sq0 = half_dot(q, x, 0), sq1 = half_dot(q, x, 1);
  if constexpr (F == FMT_Q8_0) {
    return __builtin_fmaf(o.a0, sq0, o.a1 * sq1);
  } else {
    return __builtin_fmaf(o.a0, sq0, __builtin_fmaf(o.b0, sx0, __builtin_fmaf(o.a1, sq1, o.b1 * sx1)));
  }
}

// item_partial through half_dots_mix, for all runs: the same values, bit for bit.
template <int F, int RUNS>
__device__ __forceinline__ void item_partials_mix(const typename Item<F>::Raw& w, const Unit (&o)[RUNS],
                                                  const float (&x)[RUNS][32], const float (&sx)[RUNS][2],
                                                  float (&v)[RUNS]) {
  static_assert(F != FMT_Q8_0, "Q8_0 codes carry a bias");
  MixPairs<F> p;
  p.make(w, o);
  float sq[RUNS][2];
  half_dots_mix<F, RUNS>(p, x, sq);
#pragma unroll
  for (int r = 0; r < RUNS; ++r) {
    const float sc = static_cast<float>(1u << (24 - MixPairs<F>::sh(r)));  // 2^24 / 2^sh
    v[r] = __builtin_fmaf(o[r].a0 * sc, sq[r][0],
                          __builtin_fmaf(o[r].b0, sx[r][0], __builtin_fmaf(o[r].a1 * sc, sq[r][1], o[r].b1 * sx[r][1])));
  }
}

// Output (row r, token t) of a workgroup = the sum of its units' partials
// part[(t * RW + r) * nU + u]: 16 lanes per output, lane j adding units j, j+16,
// ... in order, then a butterfly over the 16 lanes (DPP within a row of the
// wave).  Every path ends with this, in this order, so results do not depend on
// the launch shape and the dense and expert-indexed paths agree bit for bit.
__device__ __forceinline__ float sum16(float v) {
  v += dpp_mov<0xB1>(v);   // lane ^ 1
  v += dpp_mov<0x4E>(v);   // lane ^ 2
  v += dpp_mov<0x141>(v);  // row_half_mirror: the other quad of the 8
  v += dpp_mov<0x140>(v);  // row_mirror: the other 8 of the 16
  return v;
}

__device__ __forceinline__ void reduce_rows(const float* s_part, int rows, int ntok, int nU, int RW, int M, int r0,
                                            const TokMap& tm, float* y) {
  const int tid = threadIdx.x;
  const int grp = tid >> 4, j = tid & 15, ngrp = blockDim.x >> 4;
  for (int o = grp; o < rows * ntok; o += ngrp) {
    const int row = o / ntok, t = o - row * ntok;
    const float* pp = s_part + (t * RW + row) * nU;
    float v = 0.0f;
    for (int u = j; u < nU; u += 16) v += pp[u];
    v = sum16(v);
    if (j == 0) y[(u64)tm.y(t) * M + r0 + row] = v;
  }
}

// Tokens per work unit: a call with more tokens spreads them over more threads.
constexpr int kTokPerUnit = 4;

// Items per thread per batch.  A thread holds two batches: while it decodes one,
// the loads of the next are in flight.
// Q6_K items carry 34 raw bytes and two scale pairs (Q3_K and Q5_K units 70-80 bytes),
// so they hold fewer.
template <int F>
constexpr int ipt_max(int NB) {
  if (F == FMT_Q6_K || F == FMT_Q3_K || F == FMT_Q5_K) return NB <= 2 ? 2 : 1;
  return NB <= 2 ? 3 : 2;
}

// Rows [r0, r0 + rows) of the matrix at W (rows <= RW), all tokens t < ntok.
// Byte offsets within one matrix fit 32 bits (checked by the host).  KC is a
// multiple of 8 units, so chunk boundaries never split an item's runs.
template <int F, int NB, bool XR>
__device__ __forceinline__ void gemv_rows(const u8* W, u32 rb, int M, int nU, int K, int r0, int rows, int RW,
                                          int KC, const void* x, int x_f16, const TokMap& tm, int ntok, float* y,
                                          float* lds) {
  using It = Item<F>;
  constexpr int RUNS = It::RUNS;
  constexpr int kIpt = ipt_max<F>(NB);
  float* s_x = lds;
  float* s_sx = s_x + NB * KC * kXStride;
  float* s_part = s_sx + NB * KC * 2;
  const int T = blockDim.x;
  const int tid = threadIdx.x;

  // Work unit = (token group, item): an item against NT consecutive tokens of the
  // call.  Splitting the tokens gives a workgroup more threads than it has items
  // when the call has many tokens.  A batch is this thread's work units
  // b0 + tid + j*T (j < n) of the chunk's list, token group major.
  constexpr int NT = NB < kTokPerUnit ? NB : kTokPerUnit;
  const int TG = (ntok + NT - 1) / NT;
  struct Batch {
    typename It::Raw raw[kIpt];
    int irow[kIpt], iit[kIpt], t0[kIpt];
    int n;
  };

  for (int c0 = 0; c0 < nU; c0 += KC) {
    const int cw = min(KC, nU - c0);
    const int ipr = cw / RUNS;        // items per row in the chunk
    const int i0 = c0 / RUNS;         // first item of the chunk
    const int items = rows * ipr;
    const int works = items * TG;
    const int step = T * kIpt;

    // Loads are unconditional (work units past the list repeat its last item and
    // are not computed): with no branch around them the compiler counts the loads
    // in flight exactly and waits for each one only where its bytes are used.
    auto load = [&](int b0, Batch& bt) {
      const int first = b0 + tid;
      bt.n = first < works ? min(kIpt, (works - first + T - 1) / T) : 0;
#pragma unroll
      for (int j = 0; j < kIpt; ++j) {
        const int w = min(first + j * T, works - 1);
        const int tg = w / items;
        const int it = w - tg * items;
        const int row = it / ipr;
        bt.irow[j] = row;
        bt.iit[j] = i0 + (it - row * ipr);
        bt.t0[j] = tg * NT;
        It::load(W, (u32)(r0 + row) * rb, bt.iit[j], bt.raw[j]);
      }
    };
    auto compute = [&](const Batch& bt) {
#pragma unroll
      for (int j = 0; j < kIpt; ++j) {
        if (j < bt.n) {
          Unit o[RUNS];
          It::unpack(bt.raw[j], o);
#pragma unroll
          for (int r = 0; r < RUNS; ++r) {
            const int u = It::unit(bt.iit[j], r);
            float q[32];
            unit_codes<F>(o[r], q);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
              const int t = bt.t0[j] + tt;
              if (t < ntok) {
                float xv[32];
                const int xo = t * KC + (u - c0);
                read_x32(s_x + xo * kXStride, xv);
                s_part[(t * RW + bt.irow[j]) * nU + u] =
                    item_partial<F>(o[r], q, xv, s_sx[xo * 2], s_sx[xo * 2 + 1]);
              }
            }
          }
        }
      }
    };

    Batch A, B;
    if (XR && x_fits_regs(x_f16, ntok, cw)) {
      XRegs xr;
      x_load(x, x_f16, K, tm, ntok, c0, cw, xr);
      load(0, A);
      if (c0 > 0) __syncthreads();  // readers of the previous chunk are done
      x_put(xr, x_f16, ntok, cw, KC, s_x, s_sx);
    } else {
      load(0, A);
      if (c0 > 0) __syncthreads();
      stage_x(x, x_f16, K, tm, ntok, c0, cw, KC, s_x, s_sx);
    }
    __syncthreads();  // the chunk's activations and half sums are in LDS
    for (int b0 = 0; b0 < works; b0 += 2 * step) {
      if (b0 + step < works) load(b0 + step, B);
      compute(A);
      if (b0 + step >= works) break;
      if (b0 + 2 * step < works) load(b0 + 2 * step, A);
      compute(B);
    }
  }
  __syncthreads();

  reduce_rows(s_part, rows, ntok, nU, RW, M, r0, tm, y);
  __syncthreads();  // LDS is reused by the caller's next pass
}

extern __shared__ float s_dyn[];  // sized at launch: lds_floats(NB, KC, RW, nU), or RW * nU floats

template <int F, int NB>
__global__ __launch_bounds__(512) void k_gemv(GemvArgs a) {
  const int r0 = blockIdx.x * a.rows_per_wg;
  const int rows = min(a.rows_per_wg, a.M - r0);
  const TokMap tm{nullptr, 1, 1};
  gemv_rows<F, NB, true>(a.W, static_cast<u32>(a.row_bytes), a.M, a.nU, a.K, r0, rows, a.rows_per_wg,
                         a.chunk_units, a.x, a.x_f16, tm, a.N, a.y, s_dyn);
}

// ---------------------------------------------------------------------------------------------
// One token.  Threads are laid out unit-major: thread t takes item column
// i = t % ipr of rows g, g + G, g + 2G, ... (g = t / ipr, G row groups, at most R
// rows per thread), so it needs the activations of one item only, and reuses
// them for every row.  Consecutive threads still read consecutive items of a row.
// Partial sums and their reduction are those of the general path, so the results
// are the same bits.
//
// The workgroup stages the activations once: each thread fetches 16-value
// chunks (at most kX1Rounds), then issues the weight loads of its first items,
// and only then converts the chunks, forms their half sums and writes both to
// LDS.  The per-thread activation reads therefore come from LDS instead of
// every row group fetching the same values through the vector memory path,
// which is shared with the weight stream.  LDS image: unit u's 32 values at
// kXU*u .. kXU*u+31, the sums of its halves at kXU*u+32 and +33 (the pad also
// spreads consecutive threads' 16-byte reads over the banks); one spare unit
// after the last takes the stores of threads past the end.
//
// The thread's rows g + G k (k < R): weight loads run kAhead items ahead of the
// products -- loads of item k+kAhead are issued just before item k is computed,
// a scheduling barrier pinning the order -- so a wave computes the items that
// have arrived instead of stalling on the issue of loads the memory system cannot
// take yet.  One item ahead measured faster than two, three or four on the
// decode-layer shapes: more loads in flight per thread only lengthen the queue
// in front of every wave's first item.  Every item is computed and stored unconditionally (rows past the
// slice repeat its last row and store to a spare slot after the partials): a
// branch around the products or the store would let the compiler sink the
// products, and their loads, into it.
constexpr int kAhead = 1;
constexpr int kXU = 36;        // floats per unit in the LDS image
constexpr int kX1Rounds = 4;   // chunks per thread: 2 nU chunks, at least nU / 2 threads

template <int F, int R>
__device__ __forceinline__ void one_items(const u8* W, u32 rb, int r0, const float (&xv)[Item<F>::RUNS][32],
                                          const float (&sx)[Item<F>::RUNS][2], int g, int G, int gi, bool active,
                                          int rows, int nU, float* s_part, int spare, typename Item<F>::Raw (&wr)[R]) {
  using It = Item<F>;
  constexpr int RUNS = It::RUNS;
  auto load = [&](int k) { It::load(W, (u32)(r0 + min(g + G * k, rows - 1)) * rb, gi, wr[k]); };
#pragma unroll
  for (int k = 0; k < R; ++k) {
    if (k + kAhead < R) {
      load(k + kAhead);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int row = g + G * k;
    Unit o[RUNS];
    It::unpack(wr[k], o);
    float v[RUNS];
    if constexpr (F == FMT_Q8_0) {
      float q[32];
      unit_codes<F>(o[0], q);
      v[0] = item_partial<F>(o[0], q, xv[0], sx[0][0], sx[0][1]);
    } else {
      item_partials_mix<F, RUNS>(wr[k], o, xv, sx, v);
    }
#pragma unroll
    for (int r = 0; r < RUNS; ++r) {
      const int slot = active && row < rows ? row * nU + It::unit(gi, r) : spare;
      s_part[slot] = v[r];
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// 16 activations from global memory (4 fp32 or 2 fp16 slots of 16 bytes)
template <bool XH>
__device__ __forceinline__ void x1_fetch(const void* x, int c, uint4 (&v)[4]) {
  const uint4* p = XH ? reinterpret_cast<const uint4*>(reinterpret_cast<const _Float16*>(x) + 16 * c)
                      : reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(x) + 16 * c);
#pragma unroll
  for (int k = 0; k < (XH ? 2 : 4); ++k) v[k] = p[k];
}

// the chunk's values and half sum into the LDS image (dst: its 16 values)
template <bool XH>
__device__ __forceinline__ void x1_put(const uint4 (&v)[4], float* dst, float* dsum) {
  float f[16];
  if constexpr (XH) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const h8 h = __builtin_bit_cast(h8, v[k]);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[8 * k + e] = static_cast<float>(h[e]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[4 * k] = __uint_as_float(v[k].x); f[4 * k + 1] = __uint_as_float(v[k].y);
      f[4 * k + 2] = __uint_as_float(v[k].z); f[4 * k + 3] = __uint_as_float(v[k].w);
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k)
    *reinterpret_cast<float4*>(dst + 4 * k) = make_float4(f[4 * k], f[4 * k + 1], f[4 * k + 2], f[4 * k + 3]);
  *dsum = half_sum16(f);
}

// LDS floats of the one-token kernel: activation image (nU + 1 units), then
// RW * nU partial sums and one spare slot
inline size_t one_lds_floats(int nU, int RW) {
  return static_cast<size_t>(kXU) * (nU + 1) + static_cast<size_t>(RW) * nU + 1;
}

// This workgroup's matrix: a's own fields for a single call (they load with the
// rest of the arguments), else the grp entry whose workgroups hold blockIdx.x; wg0
// receives that matrix's first workgroup.
__device__ __forceinline__ void group_matrix(const GemvArgs& a, const GemvGroup& grp, const u8*& W, const void*& x,
                                             float*& y, int& M, int& wg0) {
  W = a.W;
  x = a.x;
  y = a.y;
  M = a.M;
  wg0 = 0;
  if (grp.n > 1) {
    int mi = 0;
#pragma unroll
    for (int i = 1; i < kGemvGroupMax; ++i) mi += i < grp.n && static_cast<int>(blockIdx.x) >= grp.first[i] ? 1 : 0;
#pragma unroll
    for (int i = 0; i < kGemvGroupMax; ++i)
      if (mi == i) {
        W = grp.W[i]; x = grp.x[i]; y = grp.y[i]; M = grp.M[i]; wg0 = grp.first[i];
      }
  }
}

// rows_per_wg = RW, chunk_units = G (row groups): one workgroup's rows of matrix W
// (its activations xg, outputs yg, Mg rows; its workgroups start at wg0)
template <int F, bool XH, int R>
__device__ __forceinline__ void gemv1_rows(const GemvArgs& a, const u8* W, const void* xg, float* yg, int Mg,
                                           int wg0, u32 rb) {
  using It = Item<F>;
  constexpr int RUNS = It::RUNS;
  const int RW = a.rows_per_wg;
  const int r0 = (static_cast<int>(blockIdx.x) - wg0) * RW;
  const int rows = min(RW, Mg - r0);
  const int nU = a.nU;
  const int ipr = nU / RUNS;
  const int G = a.chunk_units;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int g = tid / ipr;
  const bool active = g < G;
  const int gi = active ? tid - g * ipr : 0;
  float* s_x = s_dyn;
  float* s_part = s_dyn + kXU * (nU + 1);

  // activation chunks first (their loads retire first), then the weight bytes of
  // the first items; threads past the last chunk fetch nothing and store their
  // (unset) registers to the spare unit
  const int chunks = 2 * nU;
  const int nr = (chunks + nthr - 1) / nthr;
  uint4 xr[kX1Rounds][4];
#pragma unroll
  for (int j = 0; j < kX1Rounds; ++j)
    if (j < nr && tid + j * nthr < chunks) x1_fetch<XH>(xg, tid + j * nthr, xr[j]);
  typename It::Raw wr[R];
#pragma unroll
  for (int k = 0; k < R && k < kAhead; ++k) It::load(W, (u32)(r0 + min(g + G * k, rows - 1)) * rb, gi, wr[k]);
  // keep the weight loads above the staging: the scheduler would otherwise sink
  // them next to their first use, behind the wait for the activations
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < kX1Rounds; ++j)
    if (j < nr) {
      const int c = tid + j * nthr;
      const int base = c < chunks ? kXU * (c >> 1) + 16 * (c & 1) : kXU * nU;
      const int sum = c < chunks ? kXU * (c >> 1) + 32 + (c & 1) : kXU * nU + 32;
      x1_put<XH>(xr[j], s_x + base, s_x + sum);
    }
  __syncthreads();

  float xv[RUNS][32], sx[RUNS][2];
#pragma unroll
  for (int r = 0; r < RUNS; ++r) {
    const float* p = s_x + kXU * It::unit(gi, r);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float4 f = *reinterpret_cast<const float4*>(p + 4 * k);
      xv[r][4 * k] = f.x; xv[r][4 * k + 1] = f.y; xv[r][4 * k + 2] = f.z; xv[r][4 * k + 3] = f.w;
    }
    const float2 h = *reinterpret_cast<const float2*>(p + 32);
    sx[r][0] = h.x;
    sx[r][1] = h.y;
  }
  one_items<F, R>(W, rb, r0, xv, sx, g, G, gi, active, rows, nU, s_part, RW * nU, wr);
  __syncthreads();
  const TokMap tm{nullptr, 1, 1};
  reduce_rows(s_part, rows, 1, nU, RW, Mg, r0, tm, yg);
}

// The one-token kernel: the matrices of grp share the launch (one matrix for a single
// call), each workgroup on rows of one of them.
template <int F, bool XH, int R>
__global__ __launch_bounds__(512) void k_gemv1(GemvArgs a, GemvGroup grp) {
  const u8* W;
  const void* xg;
  float* yg;
  int Mg, wg0;
  group_matrix(a, grp, W, xg, yg, Mg, wg0);
  gemv1_rows<F, XH, R>(a, W, xg, yg, Mg, wg0, static_cast<u32>(a.row_bytes));
}

// The one-token kernel for a group that mixes two formats of one item width (the
// K-quant mixes that keep a few tensors in Q6_K beside Q4_K): bit i of grp.fmt_b
// marks matrix i as format FB, the others are FA.  A workgroup runs its matrix's
// format, so every output is the single call's.
template <int FA, int FB, bool XH, int R>
__global__ __launch_bounds__(512) void k_gemv1_pair(GemvArgs a, GemvGroup grp) {
  static_assert(Item<FA>::RUNS == Item<FB>::RUNS, "one launch shape for both formats");
  const u8* W;
  const void* xg;
  float* yg;
  int Mg, wg0;
  group_matrix(a, grp, W, xg, yg, Mg, wg0);
  int mi = 0;
#pragma unroll
  for (int i = 1; i < kGemvGroupMax; ++i) mi += i < grp.n && static_cast<int>(blockIdx.x) >= grp.first[i] ? 1 : 0;
  // row bytes of each format at this K: (32 nU / block weights) blocks
  constexpr u32 ua = FmtInfo<FA>::BW / 32, ub = FmtInfo<FB>::BW / 32;
  const u32 nU = static_cast<u32>(a.nU);
  if ((grp.fmt_b >> mi) & 1)
    gemv1_rows<FB, XH, R>(a, W, xg, yg, Mg, wg0, nU / ub * FmtInfo<FB>::BB);
  else
    gemv1_rows<FA, XH, R>(a, W, xg, yg, Mg, wg0, nU / ua * FmtInfo<FA>::BB);
}

// ---------------------------------------------------------------------------------------------
// A few tokens (2 .. 32).  The one-token layout (thread = item column gi of row
// group g, R rows g + G k) gains token groups: thread tg of TGN computes tokens
// tg, tg + TGN, ... of each pass.  A pass stages the activations of TP tokens
// (the most the LDS budget holds) as images like the one-token kernel's -- fp32
// values, or the fp16 values themselves when the call's activations are fp16 --
// then every thread decodes its rows' items once into code pairs and runs them
// against each of its tokens, the activations of one (token, run) read once
// from LDS for all R rows.  After the products the pass's outputs are reduced
// as everywhere else, so the results are the bits of the other paths.  The
// weight bytes stay in registers across passes.
constexpr int kXNRounds = 4;   // chunks per thread when staging a pass

// floats per staged unit: 32 values (fp32) or 32 halves in 16 floats (fp16),
// then the two half sums and a pad
template <bool XH> struct XImg { static constexpr int U = XH ? 20 : kXU; };

template <int F, int R>
__device__ __forceinline__ void multi_run(const MixPairs<F> (&pk)[R], const Unit (&o)[R][Item<F>::RUNS], int r,
                                          const float (&x)[32], float sx0, float sx1, float (&v)[R]) {
  float s[R][2];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int q = 0; q < R; ++q)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32 w = e & 1 ? pk[q].od[r][4 * h + k] : pk[q].ev[r][4 * h + k];
          const float c = e < 2 ? code_lo(w) : code_hi(w);
          const float xv = x[16 * h + 4 * k + e];
          s[q][h] = k == 0 && e == 0 ? c * xv : __builtin_fmaf(c, xv, s[q][h]);
        }
  const float sc = static_cast<float>(1u << (24 - MixPairs<F>::sh(r)));
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const Unit& u = o[q][r];
    if constexpr (F == FMT_Q8_0) {  // item_partial's expression (no b terms)
      v[q] = __builtin_fmaf(u.a0, s[q][0], u.a1 * s[q][1]);
    } else {
      v[q] = __builtin_fmaf(u.a0 * sc, s[q][0],
                            __builtin_fmaf(u.b0, sx0, __builtin_fmaf(u.a1 * sc, s[q][1], u.b1 * sx1)));
    }
  }
}

// Rows [r0, r0 + rows) of the matrix at W against the n tokens of tm (their
// activation rows tm.x(t), output rows tm.y(t)); G row groups x TGN token groups
// of ipr threads, R rows per thread, TP tokens per pass.
template <int F, bool XH, int R, int XRND>
__device__ __forceinline__ void multi_rows(const GemvArgs& a, const u8* W, int r0, int rows, int RW, int G, int TGN,
                                           int TP, const TokMap& tm, int n, float* lds) {
  using It = Item<F>;
  constexpr int RUNS = It::RUNS;
  constexpr int XU = XImg<XH>::U;
  const int nU = a.nU;
  const int ipr = nU / RUNS;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int gg = tid / ipr;            // row group + G * token group
  const bool active = gg < G * TGN;
  const int gi = active ? tid - gg * ipr : 0;
  const int g = active ? gg % G : 0;
  const int tg = active ? gg / G : TGN;  // inactive threads take no token
  const u32 rb = static_cast<u32>(a.row_bytes);
  const int img = XU * nU;               // floats per token image
  float* s_x = lds;                      // TP images, then one spare unit
  float* s_part = lds + TP * img + XU;
  const int spare_part = TP * RW * nU;

  typename It::Raw wr[R];
  // a pass; the first one issues the weight loads right after its activation
  // loads, so the staging waits for the activations only
  auto pass = [&](auto first, int t0) {
    const int tp = min(TP, n - t0);
    // stage the pass: chunk c = (token c / (2 nU), half unit c % (2 nU))
    const int chunks = tp * 2 * nU;
    uint4 xr[XRND][4];
#pragma unroll
    for (int j = 0; j < XRND; ++j) {
      const int c = tid + j * nthr;
      if (c < chunks) {
        const int t = c / (2 * nU), cc = c - t * 2 * nU;
        const size_t row = static_cast<size_t>(tm.x(t0 + t));
        x1_fetch<XH>(reinterpret_cast<const u8*>(a.x) + row * a.K * (XH ? 2 : 4), cc, xr[j]);
      }
    }
    if constexpr (decltype(first)::value) {
#pragma unroll
      for (int k = 0; k < R; ++k) It::load(W, (u32)(r0 + min(g + G * k, rows - 1)) * rb, gi, wr[k]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < XRND; ++j) {
      const int c = tid + j * nthr;
      if (j * nthr < chunks) {
        const int t = c / (2 * nU), cc = c - t * 2 * nU;
        float* ub = c < chunks ? s_x + t * img + XU * (cc >> 1) : s_x + TP * img;
        const int hf = c < chunks ? (cc & 1) : 0;
        if constexpr (XH) {
          // 16 halves as they are, and the half sum of their fp32 values
          *reinterpret_cast<uint4*>(ub + 8 * hf) = xr[j][0];
          *reinterpret_cast<uint4*>(ub + 8 * hf + 4) = xr[j][1];
          typedef _Float16 h8 __attribute__((ext_vector_type(8)));
          float f[16];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const h8 h = __builtin_bit_cast(h8, xr[j][k]);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[8 * k + e] = static_cast<float>(h[e]);
          }
          ub[16 + hf] = half_sum16(f);
        } else {
          x1_put<false>(xr[j], ub + 16 * hf, ub + 32 + hf);
        }
      }
    }
    __syncthreads();

    // decode the rows' items into code pairs once per pass
    MixPairs<F> pk[R];
    Unit o[R][RUNS];
#pragma unroll
    for (int k = 0; k < R; ++k) {
      It::unpack(wr[k], o[k]);
      pk[k].make(wr[k], o[k]);
    }
    for (int t = tg; t < tp; t += TGN) {
      // the pairs stay fp16 codes widened inside fma_mix: converted once per pass
      // they would hold 32 registers per run and row
#pragma unroll
      for (int k = 0; k < R; ++k)
#pragma unroll
        for (int r = 0; r < RUNS; ++r)
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            pk[k].ev[r][w] = opaque(pk[k].ev[r][w]);
            pk[k].od[r][w] = opaque(pk[k].od[r][w]);
          }
#pragma unroll
      for (int r = 0; r < RUNS; ++r) {
        const int u = It::unit(gi, r);
        const float* ub = s_x + t * img + XU * u;
        float xv[32];
        if constexpr (XH) {
          typedef _Float16 h8 __attribute__((ext_vector_type(8)));
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const h8 h = __builtin_bit_cast(h8, *reinterpret_cast<const uint4*>(ub + 4 * k));
#pragma unroll
            for (int e = 0; e < 8; ++e) xv[8 * k + e] = static_cast<float>(h[e]);
          }
        } else {
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float4 f4 = *reinterpret_cast<const float4*>(ub + 4 * k);
            xv[4 * k] = f4.x; xv[4 * k + 1] = f4.y; xv[4 * k + 2] = f4.z; xv[4 * k + 3] = f4.w;
          }
        }
        const float2 sx = *reinterpret_cast<const float2*>(ub + (XH ? 16 : 32));
        float v[R];
        multi_run<F, R>(pk, o, r, xv, sx.x, sx.y, v);
#pragma unroll
        for (int k = 0; k < R; ++k) {
          const int row = g + G * k;
          s_part[active && row < rows ? (t * RW + row) * nU + u : spare_part] = v[k];
        }
      }
    }
    __syncthreads();
    if (tm.pairs) {
      const TokMap pm{tm.pairs + t0, tm.S, tm.per_slot};
      reduce_rows(s_part, rows, tp, nU, RW, a.M, r0, pm, a.y);
    } else {
      reduce_rows(s_part, rows, tp, nU, RW, a.M, r0, tm, a.y + static_cast<size_t>(t0) * a.M);
    }
  };
  pass(std::true_type{}, 0);
  for (int t0 = TP; t0 < n; t0 += TP) pass(std::false_type{}, t0);
}

template <int F, bool XH, int R>
__global__ __launch_bounds__(512) void k_gemvn(GemvArgs a, GemvGroup grp) {
  GemvArgs b = a;  // this workgroup's matrix (see group_matrix)
  int wg0;
  group_matrix(a, grp, b.W, b.x, b.y, b.M, wg0);
  const int RW = b.rows_per_wg;
  const int r0 = (static_cast<int>(blockIdx.x) - wg0) * RW;
  const TokMap tm{nullptr, 1, 1};
  multi_rows<F, XH, R, kXNRounds>(b, b.W, r0, min(RW, b.M - r0), RW, b.chunk_units, b.tok_groups, b.tok_pass, tm,
                                  b.N, s_dyn);
}

// ---------------------------------------------------------------------------------------------
// A few fp16 tokens of 4-bit affine groups on the matrix cores.  With scale s and bias b
// for a group of 64 weights, each output takes, per group,
//   s * (sum of q_k x_k over the group) + b * (sum of x_k over the group),
// and both sums run on v_mfma_f32_16x16x32_f16 with exact operands: the codes as fp16
// subnormals q * 2^-24 (exact, q < 16), the activations as they are, and a B operand of
// ones for the activation sums.  The products are exact in fp32 and the matrix core
// accumulates them in fp32; s * 2^24 (exact) and b then scale the two sums in fp32 fmas.
// The weight is never rounded to fp16: this is the matrix-vector arithmetic, its
// products taken 32 at a time.  For a one-hot token the first sum is q exactly and the
// second 1, so the output is fma-exact: round(s * q + b), the fp32 weight.
//
// Tokens are the A rows (token block b: tokens 16b .. 16b + 15, lane l: token l % 16,
// k-slots 8 (l / 16) .. +7), weight rows the B columns (lane l: row l % 16, the same
// k-slots), and the k-slots of a step are 32 consecutive weights of one half of a group:
// lane group l / 16 reads code bytes 8 (l / 16) .. +7 of the group (the low nibbles are
// weights 8 (l / 16) .. +7 of the first half, the high nibbles those of the second) and
// the matching 16 bytes of each token's activations.  A wave holds RT tiles of 16 rows
// against the same activation registers (the activations are 2 bytes per weight and
// token block, four times the codes: RT = 2 halves what a weight costs in loads); a
// workgroup owns the 16 RT rows, its KS waves split K, wave w taking GPW groups from
// group w * GPW, with every load issued before the first product.  The waves' partial
// outputs are summed in LDS in wave order, so an output's value depends on its token's
// activations and K only (not on M, N, RT or the launch's other matrices): grouped and
// single calls, and calls with other token counts, agree bit for bit.
template <int NTB, int GPW, int RT>
__global__ __launch_bounds__(1024) void k_gemvm_a4(GemvArgs a, GemvGroup grp) {
  const u8* W;
  const void* xv;
  float* y;
  int M, wg0;
  group_matrix(a, grp, W, xv, y, M, wg0);
  const int r0 = (static_cast<int>(blockIdx.x) - wg0) * 16 * RT;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int KS = blockDim.x >> 6;
  const int K = a.K, N = a.N;
  const int G = K >> 6;
  const int kq = lane >> 4;
  const _Float16* x = static_cast<const _Float16*>(xv);
  const int g0 = w * GPW;

  u32 hdr[RT][GPW], q[RT][GPW][2];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = min(r0 + 16 * rt + (lane & 15), M - 1);  // rows past M repeat the last one (never stored)
    const u32 row_off = static_cast<u32>(row) * static_cast<u32>(a.row_bytes);
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
      const int g = min(g0 + j, G - 1);  // slots past K repeat the last group (never added)
      const u32* p = reinterpret_cast<const u32*>(W + row_off + 36u * static_cast<u32>(g));
      hdr[rt][j] = p[0];
      q[rt][j][0] = p[1 + 2 * kq];
      q[rt][j][1] = p[2 + 2 * kq];
    }
  }
  // activations of the real tokens only: the lanes of padding rows load nothing (their
  // zeros give zero outputs, never stored), so below 16 tokens the loads move N / 16 of
  // a full block's bytes
  uint4 xa[NTB][GPW][2];
#pragma unroll
  for (int b = 0; b < NTB; ++b) {
#pragma unroll
    for (int j = 0; j < GPW; ++j) xa[b][j][0] = xa[b][j][1] = uint4{0, 0, 0, 0};
    const int tok = 16 * b + (lane & 15);
    if (tok < N) {
#pragma unroll
      for (int j = 0; j < GPW; ++j) {
        const int g = min(g0 + j, G - 1);
        const uint4* px = reinterpret_cast<const uint4*>(x + static_cast<size_t>(tok) * K + 64 * g + 8 * kq);
        xa[b][j][0] = px[0];  // weights 8kq .. +7 of the first half
        xa[b][j][1] = px[4];  // and of the second (32 activations on)
      }
    }
  }

  const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
  float acc[RT][NTB][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int b = 0; b < NTB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[rt][b][i] = 0.0f;
#pragma unroll
  for (int j = 0; j < GPW; ++j) {
    // slots past the last group are computed and dropped by a select: a branch would let
    // the compiler sink their loads behind the products of the slots before them
    const bool live = g0 + j < G;
    // bytes (2v, 2v+1) of each code word as an fp16 pair, low and high nibbles apart
    half8 c[RT][2];
    float s24[RT], bias[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32 v[4];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const u32 n = h ? (q[rt][j][e] >> 4) : q[rt][j][e];
          v[2 * e] = __builtin_amdgcn_perm(0u, n, 0x0C010C00u) & 0x000F000Fu;
          v[2 * e + 1] = __builtin_amdgcn_perm(0u, n, 0x0C030C02u) & 0x000F000Fu;
        }
        c[rt][h] = __builtin_bit_cast(half8, uint4{v[0], v[1], v[2], v[3]});
      }
      s24[rt] = h2f(hdr[rt][j]) * 16777216.0f;  // scale * 2^24, exact
      bias[rt] = h2f(hdr[rt][j] >> 16);
    }
#pragma unroll
    for (int b = 0; b < NTB; ++b) {
      const half8 x0 = __builtin_bit_cast(half8, xa[b][j][0]);
      const half8 x1 = __builtin_bit_cast(half8, xa[b][j][1]);
      // the activation sums do not depend on the rows: one pair of products for all tiles
      floatx4 sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(x0, ones, floatx4{0, 0, 0, 0}, 0, 0, 0);
      sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(x1, ones, sx, 0, 0, 0);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        floatx4 sq = __builtin_amdgcn_mfma_f32_16x16x32_f16(x0, c[rt][0], floatx4{0, 0, 0, 0}, 0, 0, 0);
        sq = __builtin_amdgcn_mfma_f32_16x16x32_f16(x1, c[rt][1], sq, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float t = fmaf(bias[rt], sx[i], fmaf(s24[rt], sq[i], acc[rt][b][i]));
          acc[rt][b][i] = live ? t : acc[rt][b][i];
        }
      }
    }
  }

  // D[4 (l / 16) + i][l % 16] of token block b, tile rt: token 16b + 4 (l / 16) + i,
  // row r0 + 16 rt + l % 16
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int b = 0; b < NTB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_dyn[(((w * RT + rt) * NTB + b) * 4 + i) * 64 + lane] = acc[rt][b][i];
  __syncthreads();
  constexpr int kOut = RT * NTB * 256;
  for (int o = threadIdx.x; o < kOut; o += blockDim.x) {
    float sum = s_dyn[o];
    for (int ww = 1; ww < KS; ++ww) sum += s_dyn[ww * kOut + o];
    const int rt = o / (NTB * 256), b = (o >> 8) % NTB, i = (o >> 6) & 3, l = o & 63;
    const int tok = 16 * b + 4 * (l >> 4) + i;
    const int r = r0 + 16 * rt + (l & 15);
    if (tok < N && r < M) y[static_cast<size_t>(tok) * M + r] = sum;
  }
}

// ---------------------------------------------------------------------------------------------
// The same matrix-core arithmetic for the other formats, unit by unit (Q8_0's signed
// codes as exact fp16 normals, with no bias term): a unit's 32 weights share one
// (a, b) pair, or one per 16-weight half (Q6_K, Q2_K, Q3_K), and each output takes
// a * (sum of q_k x_k) + b * (sum of x_k) per unit or half, both sums on the matrix
// cores with exact operands (codes as fp16 subnormals, fp16 activations, fp32 sums):
// a 32-deep v_mfma_f32_16x16x32_f16 step per unit, or a 16-deep v_mfma_f32_16x16x16_f16
// step per half.  Lane group l / 16 holds the unit's weights 8 (l / 16) .. +7 (or 4 (l / 16)
// .. +3 of each half).  A wave runs UPW consecutive units of its 16 rows in steps of 4:
// lane group g loads and decodes unit g of the step with the format's unit decoder (each
// unit once, not once per lane group) and leaves its 32 codes and (a * 2^24, b) pairs in
// the wave's LDS slot, from which every lane group reads the words and coefficients of
// each unit it multiplies.  D steps of loads are in flight (a ring, its last turn
// peeled; units past K multiply zero coefficients by zero activations), with one
// accumulator per unit of a step; the KS waves of a workgroup cover K and their sums are
// added in LDS in wave order, so an output depends on its token's activations and K only.
template <int F> constexpr bool unit_halves() { return F == FMT_Q6_K || F == FMT_Q2_K || F == FMT_Q3_K; }
// at most 8 waves per workgroup (256 registers: the widest decoders' raw units, and two
// token blocks, spill at 128), for one token block as for two, so that the split of K --
// and with it every output's bits -- does not depend on the token count
constexpr int kUnitMaxWaves = 8;
constexpr int kExWords = 12;  // LDS words per (row, unit): 8 code words, a0 * 2^24, b0, a1 * 2^24, b1
typedef _Float16 half4 __attribute__((ext_vector_type(4)));

// codes of bytes 0, 1 and 2, 3 of w as fp16 subnormal pairs (code * 2^-24, exact)
__device__ __forceinline__ uint2 code_pairs(u32 w) {
  return uint2{__builtin_amdgcn_perm(0u, w, 0x0C010C00u), __builtin_amdgcn_perm(0u, w, 0x0C030C02u)};
}

template <int F, int NTB>
__global__ __launch_bounds__(64 * kUnitMaxWaves) void k_gemvm(GemvArgs a, GemvGroup grp) {
  using Dec = Decoder<F>;
  constexpr int D = 2;  // steps in flight
  constexpr bool H = unit_halves<F>();
  const u8* W;
  const void* xv;
  float* y;
  int M, wg0;
  group_matrix(a, grp, W, xv, y, M, wg0);
  const int r0 = (static_cast<int>(blockIdx.x) - wg0) * 16;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int KS = blockDim.x >> 6;
  const int K = a.K, N = a.N, nU = a.nU;
  const int kq = lane >> 4, rr = lane & 15;
  const int upw = a.chunk_units;  // units per wave, a multiple of 4 * D
  const int ub = w * upw;
  const int row = min(r0 + rr, M - 1);  // rows past M repeat the last one (never stored)
  const u32 row_off = static_cast<u32>(row) * static_cast<u32>(a.row_bytes);
  const u32 xbytes = static_cast<u32>(N) * static_cast<u32>(K) * 2u;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(xv), 0, static_cast<int>(xbytes), 0x00020000);
  u32* ex = reinterpret_cast<u32*>(s_dyn) + KS * NTB * 256 + w * (16 * 4 * kExWords);  // this wave's slot
  u32* mine = ex + (rr * 4 + kq) * kExWords;  // (row rr, unit kq of the step)

  typename Dec::Raw rw[D];
  uint4 xs[D][4][NTB];
  auto fetch = [&](int u0, int d) {  // step of units u0 .. u0 + 3
    Dec::load(W, row_off, min(u0 + kq, nU - 1), rw[d]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int u = u0 + j, uc = min(u, nU - 1);
#pragma unroll
      for (int b = 0; b < NTB; ++b) {
        const int tok = 16 * b + rr;
        const bool in = tok < N && u < nU;
        const u32 base = (static_cast<u32>(tok) * static_cast<u32>(K) + 32u * static_cast<u32>(uc)) * 2u;
        if constexpr (H) {
          const u32 o0 = in ? base + 8u * kq : xbytes, o1 = in ? base + 32u + 8u * kq : xbytes;
          const uint2 v0 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, o0, 0, 0));
          const uint2 v1 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, o1, 0, 0));
          xs[d][j][b] = uint4{v0.x, v0.y, v1.x, v1.y};
        } else {
          xs[d][j][b] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, in ? base + 16u * kq : xbytes, 0, 0));
        }
      }
    }
  };
  floatx4 acc[4][NTB];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int b = 0; b < NTB; ++b) acc[j][b] = floatx4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int u0, int d) {
    {  // this lane group's unit into the wave's slot
      Unit o;
      Dec::unpack(rw[d], o);
      const bool live = u0 + kq < nU;
      const float sc = F == FMT_Q8_0 ? 1.0f : 16777216.0f;  // Q8_0: codes enter as q, not q * 2^-24
      uint4* m4 = reinterpret_cast<uint4*>(mine);
      m4[0] = uint4{o.c[0], o.c[1], o.c[2], o.c[3]};
      m4[1] = uint4{o.c[4], o.c[5], o.c[6], o.c[7]};
      m4[2] = uint4{__builtin_bit_cast(u32, live ? o.a0 * sc : 0.0f), __builtin_bit_cast(u32, live ? o.b0 : 0.0f),
                    __builtin_bit_cast(u32, live ? o.a1 * sc : 0.0f), __builtin_bit_cast(u32, live ? o.b1 : 0.0f)};
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32* e = ex + (rr * 4 + j) * kExWords;
      const float4 cf = *reinterpret_cast<const float4*>(e + 8);  // (a0', b0, a1', b1) of row rr, unit j
      if constexpr (H) {
        const half4 c0 = __builtin_bit_cast(half4, code_pairs(e[kq]));
        const half4 c1 = __builtin_bit_cast(half4, code_pairs(e[4 + kq]));
        const half4 ones = {1, 1, 1, 1};
#pragma unroll
        for (int b = 0; b < NTB; ++b) {
          const half4 x0 = __builtin_bit_cast(half4, uint2{xs[d][j][b].x, xs[d][j][b].y});
          const half4 x1 = __builtin_bit_cast(half4, uint2{xs[d][j][b].z, xs[d][j][b].w});
          const floatx4 z = {0.f, 0.f, 0.f, 0.f};
          const floatx4 q0 = __builtin_amdgcn_mfma_f32_16x16x16f16(x0, c0, z, 0, 0, 0);
          const floatx4 s0 = __builtin_amdgcn_mfma_f32_16x16x16f16(x0, ones, z, 0, 0, 0);
          const floatx4 q1 = __builtin_amdgcn_mfma_f32_16x16x16f16(x1, c1, z, 0, 0, 0);
          const floatx4 s1 = __builtin_amdgcn_mfma_f32_16x16x16f16(x1, ones, z, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[j][b][i] = fmaf(cf.w, s1[i], fmaf(cf.z, q1[i], fmaf(cf.y, s0[i], fmaf(cf.x, q0[i], acc[j][b][i]))));
        }
      } else if constexpr (F == FMT_Q8_0) {
        const uint2 cw = *reinterpret_cast<const uint2*>(e + 2 * kq);
        const half2v off = {1152, 1152};
        half2v h[4] = {__builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, cw.x, 0x04010400u)),
                       __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, cw.x, 0x04030402u)),
                       __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, cw.y, 0x04010400u)),
                       __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, cw.y, 0x04030402u))};
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = h[i] - off;
        const half8 c = {h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
#pragma unroll
        for (int b = 0; b < NTB; ++b) {
          const floatx4 q = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, xs[d][j][b]), c,
                                                                   floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[j][b][i] = fmaf(cf.x, q[i], acc[j][b][i]);
        }
      } else {
        const uint2 cw = *reinterpret_cast<const uint2*>(e + 2 * kq);
        const uint2 p0 = code_pairs(cw.x), p1 = code_pairs(cw.y);
        const half8 c = __builtin_bit_cast(half8, uint4{p0.x, p0.y, p1.x, p1.y});
        const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
        for (int b = 0; b < NTB; ++b) {
          const half8 xh = __builtin_bit_cast(half8, xs[d][j][b]);
          const floatx4 z = {0.f, 0.f, 0.f, 0.f};
          const floatx4 q = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, c, z, 0, 0, 0);
          const floatx4 sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, ones, z, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[j][b][i] = fmaf(cf.y, sx[i], fmaf(cf.x, q[i], acc[j][b][i]));
        }
      }
    }
    // every lane group has read this step's slot before the next step writes it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
#pragma unroll
  for (int d = 0; d < D; ++d) fetch(ub + 4 * d, d);
  int u = ub;
  for (int turn = 4 * D; turn < upw; turn += 4 * D, u += 4 * D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      compute(u + 4 * d, d);
      __builtin_amdgcn_sched_barrier(0);
      fetch(u + 4 * d + 4 * D, d);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d) {
    compute(u + 4 * d, d);
    __builtin_amdgcn_sched_barrier(0);
  }

#pragma unroll
  for (int b = 0; b < NTB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = acc[0][b][i];
#pragma unroll
      for (int j = 1; j < 4; ++j) v += acc[j][b][i];
      s_dyn[((w * NTB + b) * 4 + i) * 64 + lane] = v;
    }
  __syncthreads();
  constexpr int kOut = NTB * 256;
  for (int oi = threadIdx.x; oi < kOut; oi += blockDim.x) {
    float sum = s_dyn[oi];
    for (int ww = 1; ww < KS; ++ww) sum += s_dyn[ww * kOut + oi];
    const int b = oi >> 8, i = (oi >> 6) & 3, l = oi & 63;
    const int tok = 16 * b + 4 * (l >> 4) + i;
    const int r = r0 + (l & 15);
    if (tok < N && r < M) y[static_cast<size_t>(tok) * M + r] = sum;
  }
}

// LDS floats of the multi-token kernel: TP token images and a spare unit, then
// TP * RW * nU partial sums and a spare slot
inline size_t multi_lds_floats(bool xh, int nU, int RW, int TP) {
  const size_t U = xh ? XImg<true>::U : XImg<false>::U;
  return static_cast<size_t>(TP) * U * nU + U + static_cast<size_t>(TP) * RW * nU + 1;
}

// Expert-indexed: blockIdx.y = rank k of the expert among the distinct valid ids
// of this call (ascending), blockIdx.x = row slice.  Each workgroup builds, in LDS,
// the presence bitmap of the ids, finds its expert and the (token, slot) pairs
// routed to it, and streams that expert's rows of its slice once per NB pairs.
constexpr int kIdBitmapWords = static_cast<int>(kMaxExperts / 32);
constexpr int kIdMaxPairs = static_cast<int>(kMaxGemvTokens * kMaxSlots);

// The workgroup's expert (rank blockIdx.y among the distinct valid ids of the
// call, ascending; -1 if there are fewer) and the (token, slot) pairs routed to
// it, in sh.pairs[0 .. sh.npairs).  Rank-0 workgroups also write the NaN rows of ids
// outside [0, E) for their row slice.
struct IdShared {
  u32 bits[kIdBitmapWords];
  int pairs[kIdMaxPairs];
  int expert, npairs, bad;
};

__device__ __forceinline__ int id_route(const GemvArgs& a, int r0, int rows, IdShared& sh) {
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int P = a.N * a.S;
  const int nwords = (a.E + 31) >> 5;

  for (int w = tid; w < nwords; w += nthr) sh.bits[w] = 0u;
  if (tid == 0) { sh.expert = -1; sh.npairs = 0; sh.bad = 0; }
  __syncthreads();
  for (int p = tid; p < P; p += nthr) {
    const int e = a.ids[p];
    if (e >= 0 && e < a.E)
      atomicOr(&sh.bits[e >> 5], 1u << (e & 31));
    else
      sh.bad = 1;
  }
  __syncthreads();

  // k-th set bit, found by the first wave: lane l counts words [l*wpl, (l+1)*wpl),
  // an inclusive prefix over the lanes, then the lane holding rank k walks its words.
  const int k = blockIdx.y;
  if (tid < 64) {
    const int wpl = (nwords + 63) >> 6;
    const int w0 = tid * wpl, w1 = min(nwords, w0 + wpl);
    int cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(sh.bits[w]);
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (tid >= off) incl += v;
    }
    const int excl = incl - cnt;
    if (k >= excl && k < incl) {
      int seen = excl;
      for (int w = w0; w < w1; ++w) {
        u32 bits = sh.bits[w];
        while (bits) {
          const int b = __ffs(bits) - 1;
          if (seen == k) sh.expert = (w << 5) + b;
          ++seen;
          bits &= bits - 1u;
        }
      }
    }
  }
  __syncthreads();
  const int e = sh.expert;

  // Ids outside [0, E) have no matrix: their output rows are NaN (written by the
  // rank-0 workgroups, which exist for every row slice).
  if (blockIdx.y == 0 && sh.bad) {
    const float qnan = __builtin_nanf("");
    for (int i = tid; i < P * rows; i += nthr) {
      const int p = i / rows, r = i - p * rows;
      const int id = a.ids[p];
      if (id < 0 || id >= a.E) a.y[(u64)p * a.M + r0 + r] = qnan;
    }
  }
  if (e < 0) return -1;  // uniform over the workgroup

  // (pair order within the list does not matter: each pair's outputs are
  // computed on their own)
  for (int p = tid; p < P; p += nthr)
    if (a.ids[p] == e) sh.pairs[atomicAdd(&sh.npairs, 1)] = p;
  __syncthreads();
  return e;
}

// Expert-indexed: blockIdx.y = rank of the expert, blockIdx.x = row slice.  Each
// workgroup builds, in LDS, the presence bitmap of the ids, finds its expert and
// the (token, slot) pairs routed to it, and streams that expert's rows of its
// slice once per NB pairs.
template <int F, int NB>
__global__ __launch_bounds__(512) void k_gemv_id(GemvArgs a) {
  __shared__ IdShared sh;
  const int r0 = blockIdx.x * a.rows_per_wg;
  const int rows = min(a.rows_per_wg, a.M - r0);
  const int e = id_route(a, r0, rows, sh);
  if (e < 0) return;
  const int np = sh.npairs;
  const u8* W = a.W + (u64)e * a.expert_bytes;
  for (int c = 0; c < np; c += NB) {
    const TokMap tm{sh.pairs + c, a.S, a.x_per_slot};
    // (the K-quant formats stage activations directly: the pass loop leaves no
    // registers for the activation slots)
    gemv_rows<F, NB, F != FMT_Q4_K && F != FMT_Q6_K>(W, static_cast<u32>(a.row_bytes), a.M, a.nU, a.K, r0, rows,
                                                     a.rows_per_wg, a.chunk_units, a.x, a.x_f16, tm,
                                                     min(NB, np - c), a.y, s_dyn);
  }
}

// Expert-indexed through the few-token layout (formats whose codes carry no
// bias): the pairs routed to the workgroup's expert are its tokens.  Rows per
// thread: 4 for one-run items, 2 for two-run items (more would spill); one
// staging round per pass.
template <int F> constexpr int id_rows() { return Item<F>::RUNS == 1 ? 4 : 2; }

template <int F, bool XH>
__global__ __launch_bounds__(512) void k_gemvn_id(GemvArgs a) {
  __shared__ IdShared sh;
  const int RW = a.rows_per_wg;
  const int r0 = blockIdx.x * RW;
  const int rows = min(RW, a.M - r0);
  const int e = id_route(a, r0, rows, sh);
  if (e < 0) return;
  const TokMap tm{sh.pairs, a.S, a.x_per_slot};
  multi_rows<F, XH, id_rows<F>(), 1>(a, a.W + (u64)e * a.expert_bytes, r0, rows, RW, a.chunk_units, a.tok_groups,
                                     a.tok_pass, tm, sh.npairs, s_dyn);
}

constexpr int kNarrowAhead = 4;  // items in flight per lane on the narrow-row kernels

// Expert-indexed, narrow rows (Q4_0 at K = 512), for up to 64 pairs (or more than
// k_gemv_id_narrow takes): the grid is (row slice, expert rank), each workgroup
// routing the ids for itself.  Lane l
// of a wave takes item l % 16 of one of the wave's four rows per step, so the 16
// lanes of a row sum their partials with the same butterfly as every other path
// (and in the same order as reduce_rows: 0 + the unit's partial, then sum16):
// results are the bits of the dense paths.  There are no partials in LDS, so a
// workgroup streams a long slice of its expert's rows with kNarrowAhead items in
// flight per lane, routing once; each lane holds its unit's activations of up to
// two pairs in registers (loaded from global memory with their half sums formed
// as everywhere else), and further pairs take another sweep of the rows.
template <bool XH>
__global__ __launch_bounds__(256) void k_gemv_id_slices(GemvArgs a) {
  using It = Item<FMT_Q4_0>;
  constexpr int D = kNarrowAhead;
  constexpr int TPM = 2;
  __shared__ IdShared sh;
  const int RW = a.rows_per_wg;
  const int r0 = blockIdx.x * RW;
  const int rows = min(RW, a.M - r0);
  const int e = id_route(a, r0, rows, sh);
  if (e < 0) return;
  const TokMap tm{sh.pairs, a.S, a.x_per_slot};
  const int np = sh.npairs;
  const int lane = threadIdx.x & 63;
  const int gi = lane & 15;
  const int per_step = 4 * (blockDim.x >> 6);             // rows per step of the workgroup
  const int rsub = 4 * (threadIdx.x >> 6) + (lane >> 4);  // this lane's row within a step
  const int steps = (rows + per_step - 1) / per_step;
  static_assert(8 % D == 0, "the ring divides a block of 8 steps");
  const int steps_pad = (steps + 7) / 8 * 8;  // whole blocks of 8 steps
  const u8* W = a.W + (u64)e * a.expert_bytes;
  const u32 rb = static_cast<u32>(a.row_bytes);
  auto load = [&](int st, typename It::Raw& w) {
    It::load(W, (u32)(r0 + min(st * per_step + rsub, rows - 1)) * rb, gi, w);
  };

  for (int t0 = 0; t0 < np; t0 += TPM) {
    const int tp = min(TPM, np - t0);
    // this lane's unit of each pair's activations, and its two half sums
    float xv[TPM][32], sx[TPM][2];
#pragma unroll
    for (int t = 0; t < TPM; ++t) {
      const size_t xrow = static_cast<size_t>(tm.x(t0 + min(t, tp - 1)));
      if constexpr (XH) {
        typedef _Float16 h8 __attribute__((ext_vector_type(8)));
        const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const _Float16*>(a.x) + xrow * a.K + 32 * gi);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const h8 h = __builtin_bit_cast(h8, p[k]);
#pragma unroll
          for (int q = 0; q < 8; ++q) xv[t][8 * k + q] = static_cast<float>(h[q]);
        }
      } else {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.x) + xrow * a.K + 32 * gi);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float4 f = p[k];
          xv[t][4 * k] = f.x; xv[t][4 * k + 1] = f.y; xv[t][4 * k + 2] = f.z; xv[t][4 * k + 3] = f.w;
        }
      }
      sx[t][0] = half_sum16(xv[t]);
      sx[t][1] = half_sum16(xv[t] + 16);
    }

    // one sweep of the rows for TP_ pairs: no branch in the steady loop, so the
    // load counter's waits stay those of the ring
    auto sweep = [&](auto tpc) {
      constexpr int TP_ = decltype(tpc)::value;
      typename It::Raw wr[D];
      // lane gi keeps the sum of step 8 b + gi % 8 of each block b of 8 steps
      // (the 16 lanes of a row all hold each step's sum) and stores it once per
      // block: two lanes per output instead of sixteen
      float outv[TP_];
      // step st (slot k % D of the ring, step k of the block), then (RELOAD) the
      // slot refilled with step st + D
      auto step = [&](auto reload, int k, int st) {
        Unit o[1][1];
        MixPairs<FMT_Q4_0> pk[1];
        It::unpack(wr[k % D], o[0]);
        pk[0].make(wr[k % D], o[0]);
        if constexpr (decltype(reload)::value) load(st + D, wr[k % D]);
#pragma unroll
        for (int t = 0; t < TP_; ++t) {
          float v[1];
          multi_run<FMT_Q4_0, 1>(pk, o, 0, xv[t], sx[t][0], sx[t][1], v);
          const float sum = sum16(0.0f + v[0]);
          outv[t] = (gi & 7) == k ? sum : outv[t];
        }
      };
      // the block's stores: step s0 + gi % 8's row (rows past the slice repeat
      // its last row, with the same bits)
      auto store = [&](int s0) {
        const int row = min((s0 + (gi & 7)) * per_step + rsub, rows - 1);
#pragma unroll
        for (int t = 0; t < TP_; ++t) a.y[(u64)tm.y(t0 + t) * a.M + r0 + row] = outv[t];
      };
#pragma unroll
      for (int k = 0; k < D; ++k) load(k, wr[k]);
      int s0 = 0;
      for (; s0 + 8 < steps_pad; s0 += 8) {
#pragma unroll
        for (int k = 0; k < 8; ++k) step(std::true_type{}, k, s0 + k);
        store(s0);
      }
#pragma unroll
      for (int k = 0; k < 8 - D; ++k) step(std::true_type{}, k, s0 + k);
#pragma unroll
      for (int k = 8 - D; k < 8; ++k) step(std::false_type{}, k, s0 + k);
      store(s0);
    };
    if (tp == 2)
      sweep(std::integral_constant<int, 2>{});
    else
      sweep(std::integral_constant<int, 1>{});
  }
}

// Expert-indexed, narrow rows: Q4_0 at K = 512, the shape of p2's case (its
// section "Additional information"), where a row is 16 one-block items.  Lane l
// of a wave takes item l % 16 of one of the wave's four rows per step, so the 16
// lanes of a row sum their partials with the same butterfly as every other path
// (and in the same order as reduce_rows: 0 + the unit's partial, then sum16):
// results are the bits of the dense paths.
//
// The grid is as many workgroups as the device holds at once.  Each routes the
// call's ids once, into an LDS table: the distinct valid experts in ascending
// order (their ranks), the pairs sorted by expert, and the pair chunks -- an
// expert's pairs two at a time.  The work is then one list of steps, chunk by
// chunk, SPC steps of four rows per chunk (the expert's rows, padded to a
// multiple of 8 steps); wave w streams steps [w T, (w + 1) T), T a multiple of 8,
// with kNarrowAhead items in flight per lane, the ring running on across chunk
// boundaries.  Each lane holds its unit's activations of the chunk's pairs in
// registers, reloaded where a chunk begins.  Against k_gemv_id_slices, each of
// whose workgroups routes, loads its activations and fills its ring before a short
// stream of its own, this routes once per workgroup and streams without a pause;
// it takes calls of more than 64 pairs, below which its routing, repeated by every
// workgroup and longer with more pairs, costs more than it saves.

// LDS ints of the narrow kernel's routing: each pair's expert (P rounded up to 4),
// presence bitmap and its word prefix counts (E / 32 words each), per rank the first
// sorted pair and the first chunk (P + 1 each) and the expert (P), per pair its place
// among its expert's pairs, the sorted pairs and the chunks (P each), then the
// counts of chunks and ranks and the flag of invalid ids.  The kernel takes at most
// kNarrowMaxPairs pairs (each thread counts the pairs before its own).
constexpr int kNarrowMaxPairs = 512;
inline size_t narrow_lds_ints(int E, int P) {
  const size_t w = (static_cast<size_t>(E) + 31) / 32;
  const size_t p4 = (static_cast<size_t>(P) + 3) / 4 * 4;
  return p4 + 2 * w + 2 * (static_cast<size_t>(P) + 1) + 4 * static_cast<size_t>(P) + 3;
}

template <bool XH>
__global__ __launch_bounds__(256, 2) void k_gemv_id_narrow(GemvArgs a) {
  using It = Item<FMT_Q4_0>;
  constexpr int D = kNarrowAhead;
  static_assert(8 % D == 0 && D <= 8, "the ring divides a block of 8 steps");
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int P = a.N * a.S;
  const int E = a.E;
  const int M = a.M;
  const int nwords = (E + 31) >> 5;
  const int P4 = (P + 3) & ~3;
  int* idl = reinterpret_cast<int*>(s_dyn);  // by pair: its expert, -1 for an id outside [0, E); -2 past P
  u32* bits = reinterpret_cast<u32*>(idl + P4);
  int* wpre = reinterpret_cast<int*>(bits + nwords);
  int* off = wpre + nwords;  // by rank: pair count, then (after the scan) first sorted pair
  int* coff = off + P + 1;   // by rank: first chunk
  int* ex = coff + P + 1;    // by rank: expert
  int* slot = ex + P;        // by pair: place among its expert's pairs
  int* sorted = slot + P;    // pairs by expert
  int* chunk = sorted + P;   // chunk: rank | (index among its expert's chunks) << 16
  int* cnts = chunk + P;     // chunks, invalid ids seen, ranks

  for (int w = tid; w < nwords; w += nthr) bits[w] = 0u;
  for (int r = tid; r <= P; r += nthr) off[r] = 0;
  for (int q = P + tid; q < P4; q += nthr) idl[q] = -2;
  if (tid < 3) cnts[tid] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += nthr) {
    const int e = a.ids[p];
    const bool valid = e >= 0 && e < E;
    idl[p] = valid ? e : -1;
    if (valid)
      atomicOr(&bits[e >> 5], 1u << (e & 31));
    else
      cnts[1] = 1;
  }
  __syncthreads();
  const int lane = tid & 63;
  if (tid < 64) {  // word prefix counts of the bitmap (ranks): lane l takes words [l wpl, (l + 1) wpl)
    const int wpl = (nwords + 63) >> 6;
    const int w0 = lane * wpl, w1 = min(nwords, w0 + wpl);
    int cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(bits[w]);
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    int run = incl - cnt;
    for (int w = w0; w < w1; ++w) {
      wpre[w] = run;
      run += __popc(bits[w]);
    }
    if (lane == 63) cnts[2] = incl;
  }
  __syncthreads();
  auto rank_of = [&](int e) { return wpre[e >> 5] + __popc(bits[e >> 5] & ((1u << (e & 31)) - 1u)); };
  // each pair's place among its expert's pairs, in pair order (the pairs before it with
  // its expert): the workgroups share out one list of chunks, so every workgroup must
  // build the same tables, which an atomic counter would not (it orders the pairs as
  // the lanes and waves happen to arrive).  The ids are read four at a time, the same
  // for every lane.
  for (int p = tid; p < P; p += nthr) {
    const int e = idl[p];
    int lower = 0;
#pragma unroll 8
    for (int q = 0; q < P4; q += 4) {
      const int4 k = *reinterpret_cast<const int4*>(idl + q);
      lower += (q < p && k.x == e ? 1 : 0) + (q + 1 < p && k.y == e ? 1 : 0) + (q + 2 < p && k.z == e ? 1 : 0) +
               (q + 3 < p && k.w == e ? 1 : 0);
    }
    if (e >= 0) {
      const int r = rank_of(e);
      slot[p] = lower;
      ex[r] = e;
      atomicAdd(&off[r], 1);
    }
  }
  __syncthreads();
  if (tid < 64) {
    // pair and chunk offsets by rank: lane l takes ranks [l rpl, (l + 1) rpl)
    const int nr = cnts[2];
    const int rpl = (nr + 63) >> 6;
    const int q0 = lane * rpl, q1 = min(nr, q0 + rpl);
    int np = 0, nc = 0;
    for (int r = q0; r < q1; ++r) {
      np += off[r];
      nc += (off[r] + 1) >> 1;
    }
    int ip = np, ic = nc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int vp = __shfl_up(ip, o), vc = __shfl_up(ic, o);
      if (lane >= o) {
        ip += vp;
        ic += vc;
      }
    }
    int rp = ip - np, rc = ic - nc;
    for (int r = q0; r < q1; ++r) {
      const int c = off[r];
      off[r] = rp;
      coff[r] = rc;
      rp += c;
      rc += (c + 1) >> 1;
    }
    if (lane == 63) {
      off[nr] = ip;
      coff[nr] = ic;
      cnts[0] = ic;
    }
    // (the lanes see one another's stores after a wave sync)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int p = lane; p < P; p += 64) {
      const int e = idl[p];
      if (e >= 0) sorted[off[rank_of(e)] + slot[p]] = p;
    }
    for (int r = lane; r < nr; r += 64) {
      const int n = (off[r + 1] - off[r] + 1) >> 1;
      for (int j = 0; j < n; ++j) chunk[coff[r] + j] = r | (j << 16);
    }
  }
  // ids outside [0, E) have no matrix: NaN rows, each workgroup a slice of the rows
  if (cnts[1]) {
    const int rpw = (M + static_cast<int>(gridDim.x) - 1) / static_cast<int>(gridDim.x);
    const int rlo = static_cast<int>(blockIdx.x) * rpw;
    const float qnan = __builtin_nanf("");
    for (int i = tid; i < P * rpw; i += nthr) {
      const int p = i / rpw, r = rlo + (i - p * rpw);
      if (r < M && idl[p] < 0) a.y[(u64)p * M + r] = qnan;
    }
  }
  __syncthreads();

  // this wave's steps: blocks of 8, each within one chunk
  const int spc = (((M + 3) >> 2) + 7) & ~7;
  const int total = cnts[0] * spc;  // the host keeps P * spc below 2^30
  const int nwv = static_cast<int>(gridDim.x) * (nthr >> 6);
  const int gw = static_cast<int>(blockIdx.x) * (nthr >> 6) + __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = ((total + nwv - 1) / nwv + 7) & ~7;
  const int s_begin = gw * T;
  const int s_end = min(total, s_begin + T);
  if (s_begin >= s_end) return;  // (no barrier follows)

  const int gi = lane & 15;
  const int rsub = lane >> 4;  // this lane's row within a step
  const u32 rb = static_cast<u32>(a.row_bytes);
  // chunk c's expert base, first pair and pair count
  auto chunk_base = [&](int c) {
    const int r = chunk[c] & 0xFFFF;
    return a.W + (u64)ex[r] * a.expert_bytes;
  };
  auto load = [&](const u8* Wb, int rs, typename It::Raw& w) {
    It::load(Wb, (u32)min(4 * rs + rsub, M - 1) * rb, gi, w);
  };
  float xv[2][32], sx[2][2];
  int yrow[2];
  int npair = 1;
  auto load_x = [&](int c) {  // the chunk's pairs' activations
    const int r = chunk[c] & 0xFFFF, j = chunk[c] >> 16;
    const int f = off[r] + 2 * j, n = min(2, off[r + 1] - f);
    npair = n;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t >= n) break;  // (uniform)
      const int p = sorted[f + t];
      yrow[t] = p;
      const size_t xrow = static_cast<size_t>(a.x_per_slot ? p : p / a.S);
      if constexpr (XH) {
        typedef _Float16 h8 __attribute__((ext_vector_type(8)));
        const uint4* px = reinterpret_cast<const uint4*>(reinterpret_cast<const _Float16*>(a.x) + xrow * a.K + 32 * gi);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const h8 h = __builtin_bit_cast(h8, px[k]);
#pragma unroll
          for (int q = 0; q < 8; ++q) xv[t][8 * k + q] = static_cast<float>(h[q]);
        }
      } else {
        const float4* px = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.x) + xrow * a.K + 32 * gi);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float4 v = px[k];
          xv[t][4 * k] = v.x; xv[t][4 * k + 1] = v.y; xv[t][4 * k + 2] = v.z; xv[t][4 * k + 3] = v.w;
        }
      }
      sx[t][0] = half_sum16(xv[t]);
      sx[t][1] = half_sum16(xv[t] + 16);
    }
  };

  typename It::Raw wr[D];
  float outv[2];
  // block at step s (chunk c, first row step rs), the next block at (Wn, nrs): step k
  // computes slot k % D and refills it with the step D later, in this block or
  // (RELOAD: not in a wave's last block) the next; then the block's stores -- lane
  // gi keeps step gi % 8's sums, two lanes per output.  TP: the chunk's pairs.
  auto block = [&](auto reload, auto tpc, const u8* Wb, int rs, const u8* Wn, int nrs) {
    constexpr int TP = decltype(tpc)::value;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      Unit o[1][1];
      MixPairs<FMT_Q4_0> pk[1];
      It::unpack(wr[k % D], o[0]);
      pk[0].make(wr[k % D], o[0]);
      if (k + D < 8) {
        load(Wb, rs + k + D, wr[k % D]);
      } else {
        if constexpr (decltype(reload)::value) load(Wn, nrs + k + D - 8, wr[k % D]);
      }
#pragma unroll
      for (int t = 0; t < TP; ++t) {
        float v[1];
        multi_run<FMT_Q4_0, 1>(pk, o, 0, xv[t], sx[t][0], sx[t][1], v);
        const float sum = sum16(0.0f + v[0]);
        outv[t] = (gi & 7) == k ? sum : outv[t];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    const int row = min(4 * (rs + (gi & 7)) + rsub, M - 1);  // rows past M repeat the last one
#pragma unroll
    for (int t = 0; t < TP; ++t) a.y[(u64)yrow[t] * M + row] = outv[t];
  };

  int c = s_begin / spc;
  int rs = s_begin - c * spc;
  const u8* Wb = chunk_base(c);
  load_x(c);  // (issued before the ring: the first step waits for both)
  int xc = c;
#pragma unroll
  for (int k = 0; k < D; ++k) load(Wb, rs + k, wr[k]);
  for (int s = s_begin; s < s_end; s += 8) {
    if (c != xc) {
      load_x(c);
      xc = c;
    }
    // the next block: the same chunk 8 steps on, or the next chunk's first
    const bool same = rs + 8 < spc;
    const int nc = same ? c : c + 1;
    const int nrs = same ? rs + 8 : 0;
    if (s + 8 < s_end) {
      const u8* Wn = same ? Wb : chunk_base(nc);
      if (npair == 2)
        block(std::true_type{}, std::integral_constant<int, 2>{}, Wb, rs, Wn, nrs);
      else
        block(std::true_type{}, std::integral_constant<int, 1>{}, Wb, rs, Wn, nrs);
      c = nc;
      rs = nrs;
      Wb = Wn;
    } else if (npair == 2) {
      block(std::false_type{}, std::integral_constant<int, 2>{}, Wb, rs, Wb, rs);
    } else {
      block(std::false_type{}, std::integral_constant<int, 1>{}, Wb, rs, Wb, rs);
    }
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

typedef void (*GemvKernel)(GemvArgs);
typedef void (*GemvGroupKernel)(GemvArgs, GemvGroup);  // one-token and few-token kernels

template <int F, int... BI>
constexpr void fill_dense(GemvKernel* t, std::integer_sequence<int, BI...>) {
  ((t[BI] = k_gemv<F, kBuckets[BI]>), ...);
}
// The expert-indexed path takes at most 4 pairs of an expert per pass.
constexpr int kIdBuckets = 4;  // buckets 1, 2, 3, 4
template <int F, int... BI>
constexpr void fill_id(GemvKernel* t, std::integer_sequence<int, BI...>) {
  ((t[BI] = k_gemv_id<F, kBuckets[BI]>), ...);
}

template <int F>
constexpr void fill_one(GemvGroupKernel (&t)[2][4]) {
  t[0][0] = k_gemv1<F, false, 1>; t[0][1] = k_gemv1<F, false, 2>; t[0][2] = k_gemv1<F, false, 4>;
  t[1][0] = k_gemv1<F, true, 1>;  t[1][1] = k_gemv1<F, true, 2>;  t[1][2] = k_gemv1<F, true, 4>;
  t[0][3] = k_gemv1<F, false, 8>; t[1][3] = k_gemv1<F, true, 8>;
}

template <int F>
constexpr void fill_multi(GemvGroupKernel (&t)[2], GemvKernel (&ti)[2]) {
  t[0] = k_gemvn<F, false, 1>;
  t[1] = k_gemvn<F, true, 1>;
  ti[0] = k_gemvn_id<F, false>;
  ti[1] = k_gemvn_id<F, true>;
}

struct Tables {
  GemvKernel dense[kNumFormats][kNumBuckets];
  GemvKernel id[kNumFormats][kIdBuckets];
  GemvGroupKernel one[kNumFormats][2][4];  // [format][fp16 activations][rows per thread 1, 2, 4, 8]
  int one_regs[kNumFormats][2][4];    // their VGPRs per lane (512 when unknown)
  GemvGroupKernel multi[kNumFormats][2];   // [format][fp16 activations], one row per thread
  GemvGroupKernel pair[2][3];             // k_gemv1_pair<Q4_K, Q6_K>: [fp16 activations][rows per thread]
  int pair_regs[2][3];
  GemvKernel multi_id[kNumFormats][2];
  GemvKernel narrow_id[2];  // [fp16 activations]: Q4_0 at K = 512, more than 64 pairs
  GemvKernel slices_id[2];  // [fp16 activations]: Q4_0 at K = 512, up to 64 pairs
  int narrow_occ[2];        // their resident workgroups per CU
  GemvGroupKernel mma[2][3][2];  // k_gemvm_a4: [token blocks - 1][groups per wave - 2][row tiles - 1]
  GemvGroupKernel gm[kNumFormats][2];  // k_gemvm: [format][token blocks - 1] (null: not on that path)
  template <int F>
  void fill_format() {
    if constexpr (F == FMT_A4G64) {
      gm[F][0] = gm[F][1] = nullptr;
    } else {
      gm[F][0] = k_gemvm<F, 1>;
      gm[F][1] = k_gemvm<F, 2>;
    }
    fill_multi<F>(multi[F], multi_id[F]);
    fill_one<F>(one[F]);
    fill_dense<F>(dense[F], std::make_integer_sequence<int, kNumBuckets>{});
    fill_id<F>(id[F], std::make_integer_sequence<int, kIdBuckets>{});
  }
  Tables() {
    mma[0][0][0] = k_gemvm_a4<1, 2, 1>;
    mma[0][1][0] = k_gemvm_a4<1, 3, 1>;
    mma[0][2][0] = k_gemvm_a4<1, 4, 1>;
    mma[1][0][0] = k_gemvm_a4<2, 2, 1>;
    mma[1][1][0] = k_gemvm_a4<2, 3, 1>;
    mma[1][2][0] = k_gemvm_a4<2, 4, 1>;
    mma[0][0][1] = k_gemvm_a4<1, 2, 2>;
    mma[0][1][1] = k_gemvm_a4<1, 3, 2>;
    mma[0][2][1] = k_gemvm_a4<1, 4, 2>;
    mma[1][0][1] = k_gemvm_a4<2, 2, 2>;
    mma[1][1][1] = k_gemvm_a4<2, 3, 2>;
    mma[1][2][1] = k_gemvm_a4<2, 4, 2>;
    narrow_id[0] = k_gemv_id_narrow<false>;
    narrow_id[1] = k_gemv_id_narrow<true>;
    slices_id[0] = k_gemv_id_slices<false>;
    slices_id[1] = k_gemv_id_slices<true>;
    fill_format<FMT_Q4_0>();
    fill_format<FMT_Q8_0>();
    fill_format<FMT_Q4_K>();
    fill_format<FMT_Q6_K>();
    fill_format<FMT_A4G64>();
    fill_format<FMT_Q4_1>();
    fill_format<FMT_Q5_0>();
    fill_format<FMT_Q5_1>();
    fill_format<FMT_Q2_K>();
    fill_format<FMT_Q3_K>();
    fill_format<FMT_Q5_K>();
    pair[0][0] = k_gemv1_pair<FMT_Q4_K, FMT_Q6_K, false, 1>;
    pair[0][1] = k_gemv1_pair<FMT_Q4_K, FMT_Q6_K, false, 2>;
    pair[0][2] = k_gemv1_pair<FMT_Q4_K, FMT_Q6_K, false, 4>;
    pair[1][0] = k_gemv1_pair<FMT_Q4_K, FMT_Q6_K, true, 1>;
    pair[1][1] = k_gemv1_pair<FMT_Q4_K, FMT_Q6_K, true, 2>;
    pair[1][2] = k_gemv1_pair<FMT_Q4_K, FMT_Q6_K, true, 4>;
    auto regs = [](GemvGroupKernel k) {
      hipFuncAttributes at{};
      const bool ok = hipFuncGetAttributes(&at, reinterpret_cast<const void*>(k)) == hipSuccess;
      return ok && at.numRegs > 0 ? at.numRegs : 512;
    };
    for (int h = 0; h < 2; ++h)
      for (int r = 0; r < 4; ++r) {
        for (int f = 0; f < kNumFormats; ++f) one_regs[f][h][r] = regs(one[f][h][r]);
        if (r < 3) pair_regs[h][r] = regs(pair[h][r]);
      }
    // a CU holds, per SIMD, 512 / VGPRs waves (at most 8) of each 256-thread
    // workgroup's four: that many workgroups
    for (int h = 0; h < 2; ++h) {
      hipFuncAttributes at{};
      const bool ok = hipFuncGetAttributes(&at, reinterpret_cast<const void*>(narrow_id[h])) == hipSuccess;
      const int v = ok && at.numRegs > 0 ? (at.numRegs + 7) / 8 * 8 : 512;
      narrow_occ[h] = std::max(1, std::min(8, 512 / v));
    }
  }
};

const Tables& tables() {
  static const Tables t;
  return t;
}

constexpr int kLdsBudget = 64 * 1024;  // bytes of dynamic LDS per workgroup

struct Shape {
  int RW;       // rows per workgroup
  int KC;       // activation units staged per chunk
  int threads;  // workgroup size
  int grid;     // row slices
  size_t lds;   // dynamic LDS bytes
};

// A workgroup of RW rows (clamped so that its partial sums use at most half the
// LDS budget), one thread per work unit (item x token group) up to 512 threads
// (more: further batches); the activation chunk takes the LDS that is left.
Shape make_shape(int M, int nU, int runs, int NB, int RW, int max_threads = 512) {
  const int TG = (NB + kTokPerUnit - 1) / kTokPerUnit;
  Shape s;
  const int max_rw_lds = (kLdsBudget / 2 / 4) / (NB * nU);
  if (RW > max_rw_lds) RW = max_rw_lds;
  if (RW > M) RW = M;
  if (RW < 1) RW = 1;
  s.RW = RW;
  const int works = RW * (nU / runs) * TG;
  const int threads = (works + 63) / 64 * 64;
  s.threads = threads > max_threads ? max_threads : (threads < 64 ? 64 : threads);
  int KC = (kLdsBudget / 4 - NB * RW * nU) / (NB * (kXStride + 2));
  KC = KC / 8 * 8;  // chunks hold whole super-blocks, so an item's runs share a chunk
  s.KC = KC >= nU ? nU : (KC < 8 ? 8 : KC);
  s.grid = (M + RW - 1) / RW;
  s.lds = static_cast<size_t>(lds_floats(NB, s.KC, RW, nU)) * sizeof(float);
  return s;
}

}  // namespace

// Runs (32-weight units) per work item of each format.
constexpr int kRuns[kNumFormats] = {1, 1, 2, 2, 2, 1, 1, 1, 1, 1, 1};

namespace {

// Launch shape of the one-token kernel for M rows (of one matrix, or of the matrices
// of a grouped launch) of format fmt and K = 32 nU: G row groups (G * ipr <= 512
// threads) x R rows per thread, RW = G * R rows per workgroup, so every thread has
// R rows to compute.  Two workgroups per CU when R in {1, 2} makes G * ipr fill at
// least 3/4 of their waves and the kernel's registers let both sit on the CU at once
// (the second workgroup's loads and products overlap the first one's reduction);
// otherwise about one workgroup per CU, R in {1, 2, 4, 8} the smallest that covers
// M / 256 rows (at 8 rows per thread the decode layer's ffn_gate + ffn_up launch takes
// 244 workgroups instead of 406 at 4, two of which a CU could not hold: the decode
// step 32.1 -> 31.0 us).  False when the activation image and partials do not fit
// the LDS budget (the general path takes such shapes).
struct OneShape {
  int ri, Ge, RW, threads;
  size_t lds;
};

bool one_shape(int fmt, int nU, int64_t M, int x_f16, int cus, OneShape& o, const int (*fam_regs)[3] = nullptr) {
  const int ipr = nU / kRuns[fmt];
  if (ipr > 512 || ipr < 1) return false;
  const int Gmax = 512 / ipr;
  const int want = static_cast<int>((M + cus - 1) / cus);
  const int xh = x_f16 ? 1 : 0;
  auto two_fit = [&](int r, int ri) {
    const int G2 = (want + 2 * r - 1) / (2 * r);
    const int thr = (G2 * ipr + 63) / 64 * 64;
    const int regs = ((fam_regs ? fam_regs[xh][ri] : tables().one_regs[fmt][xh][ri]) + 7) / 8 * 8;
    const int waves_per_simd = (thr / 64 + 3) / 4;  // one workgroup's waves on each SIMD
    return G2 <= Gmax && 4 * G2 * ipr >= 3 * thr && 2 * waves_per_simd * regs <= 512;
  };
  int R, Ge;
  if (two_fit(1, 0) || two_fit(2, 1)) {
    R = two_fit(1, 0) ? 1 : 2;
    o.ri = R - 1;
    Ge = (want + 2 * R - 1) / (2 * R);
  } else {
    // (no 8-row form of the mixed-format kernel)
    R = want <= Gmax ? 1 : (want <= 2 * Gmax ? 2 : (want <= 4 * Gmax || fam_regs ? 4 : 8));
    o.ri = R == 1 ? 0 : (R == 2 ? 1 : (R == 4 ? 2 : 3));
    Ge = (want + R - 1) / R;
  }
  if (Ge > Gmax) Ge = Gmax;
  o.Ge = Ge;
  o.RW = Ge * R;
  o.threads = (Ge * ipr + 63) / 64 * 64;
  o.lds = one_lds_floats(nU, o.RW) * sizeof(float);
  return o.lds <= static_cast<size_t>(kLdsBudget);
}

hipError_t launch_one(int fmt, int nU, int64_t row_bytes, const OneShape& o, const GemvGroup& grp, int x_f16,
                      hipStream_t st, bool pair = false) {
  GemvArgs a{};
  a.W = grp.W[0];  // a single matrix is read from these fields
  a.x = grp.x[0];
  a.y = grp.y[0];
  a.M = grp.M[0];
  a.row_bytes = row_bytes;
  a.nU = nU;
  a.K = 32 * nU;
  a.rows_per_wg = o.RW;
  a.chunk_units = o.Ge;
  a.x_f16 = x_f16;
  a.N = 1;
  GemvGroupKernel k = pair ? tables().pair[x_f16 ? 1 : 0][o.ri] : tables().one[fmt][x_f16 ? 1 : 0][o.ri];
  hipLaunchKernelGGL(k, dim3(grp.first[grp.n]), dim3(o.threads), o.lds, st, a, grp);
  return hipGetLastError();
}

// A few tokens (2 .. 32): the one-token layout with one row per thread (two would
// spill registers with fp32 activations), about one workgroup per CU (two above 8
// tokens, where the products outweigh staging the activations once more: the
// 4-bit-group layer at 16 tokens 53.6 -> 50.5 us, while 2 and 4 tokens lose 4-5%),
// TGN token groups filling up to 512 threads, TP tokens per pass as the LDS budget
// and kXNRounds staging rounds allow.  M: the rows of the launch (of one matrix or
// of a group).  False for shapes that do not fit.
struct MultiShape {
  int Ge, RW, TGN, TP, threads;
  size_t lds;
};

bool multi_shape(int fmt, int nU, int64_t M, int N, int x_f16, int cus, MultiShape& o) {
  const int ipr2 = nU / kRuns[fmt];
  if (ipr2 < 1 || ipr2 > 512) return false;
  const int Gmax = 512 / ipr2;
  const int per_cu = N > 8 ? 2 : 1;
  const int want = static_cast<int>((M + cus * per_cu - 1) / (cus * per_cu));
  int Ge = want;
  if (Ge > Gmax) Ge = Gmax;
  const int RW = Ge;
  const bool xh = x_f16 != 0;
  int TP = N;
  while (TP > 0 && multi_lds_floats(xh, nU, RW, TP) * sizeof(float) > static_cast<size_t>(kLdsBudget)) --TP;
  int TGN = TP < 512 / (Ge * ipr2) ? TP : 512 / (Ge * ipr2);
  if (TGN < 1) TGN = 1;
  const int threads = (Ge * TGN * ipr2 + 63) / 64 * 64;
  const int tp_rounds = kXNRounds * threads / (2 * nU);
  if (TP > tp_rounds) TP = tp_rounds;
  if (TP >= 1) TP = (N + (N + TP - 1) / TP - 1) / ((N + TP - 1) / TP);  // passes of equal size
  if (TGN > TP) TGN = TP;
  if (TP < 1) return false;
  o.Ge = Ge;
  o.RW = RW;
  o.TGN = TGN;
  o.TP = TP;
  o.threads = threads;
  o.lds = multi_lds_floats(xh, nU, RW, TP) * sizeof(float);
  return true;
}

hipError_t launch_multi(int fmt, int nU, int64_t row_bytes, int N, const MultiShape& o, const GemvGroup& grp,
                        int x_f16, hipStream_t st) {
  GemvArgs a{};
  a.W = grp.W[0];  // a single matrix is read from these fields
  a.x = grp.x[0];
  a.y = grp.y[0];
  a.M = grp.M[0];
  a.row_bytes = row_bytes;
  a.nU = nU;
  a.K = 32 * nU;
  a.rows_per_wg = o.RW;
  a.chunk_units = o.Ge;
  a.x_f16 = x_f16;
  a.N = N;
  a.tok_groups = o.TGN;
  a.tok_pass = o.TP;
  hipLaunchKernelGGL(tables().multi[fmt][x_f16 ? 1 : 0], dim3(grp.first[grp.n]), dim3(o.threads), o.lds, st, a,
                     grp);
  return hipGetLastError();
}

// Few fp16 tokens of 4-bit affine groups on the matrix cores (k_gemvm_a4): KS =
// ceil(G / GPW) waves over the G = K / 64 groups, GPW the smallest of 2, 3, 4 that
// keeps KS <= 16 -- a function of K alone, so the waves' partial sums of an output are
// added in the same order whichever launch the matrix is in -- and RT row tiles of 16 per
// wave (RT changes which wave computes a row, not how).
constexpr int kMmaMinTokens = 5;  // below it the vector kernel is as fast (4 tokens) or faster
struct MmaShape {
  int gpw, ks, ntb, rt;
  int upw;  // k_gemvm (the formats other than A4G64): units per wave; 0 for k_gemvm_a4
  size_t lds;
};

// k_gemvm's shape: KS = ceil(units / UPW) waves (at most 8), UPW a multiple of 8 (two
// steps of 4 units) -- a function of K alone.
// k_gemvm takes fp16 calls from kMmaMinTokens tokens, as k_gemvm_a4 does.  On a 4096 x
// 4096 matrix it was the faster of the two from 2..5 tokens by format (fp16 tokens,
// weights rotated over 32 copies; us at 2 / 4 / 8 / 16 tokens, vector kernel -> matrix
// cores: Q4_0 9.7/10.2/16.7/27.3 -> 9.2/9.3/9.2/10.0, Q6_K 9.6/11.9/19.3/31.2 ->
// 12.1/12.2/13.1/15.5), but on the decode layer's larger matrices the vector kernel
// streams near its one-token rate at 2..4 tokens while this kernel stays near 1.2 TB/s
// (layer at 2 / 3 / 4 tokens: 51.6 / 65.9 / 72.9 us from 5 tokens on, 64.3 / 73.6 /
// 76.2 with Q4_K from 2); at 6 tokens the layer takes 75 us with it, 97 without.

bool mma_unit_shape(int fmt, int64_t K, int N, int x_f16, MmaShape& o) {
  if (!x_f16 || N < kMmaMinTokens || N > 32 || K % 32 != 0 || K < 32 || !tables().gm[fmt][0]) return false;
  // the activations are read through a buffer of N * K fp16 values with 32-bit offsets
  if (static_cast<int64_t>(N) * K * 2 >= (int64_t(1) << 31)) return false;
  const int64_t nU = K / 32;
  const int64_t per = (nU + kUnitMaxWaves - 1) / kUnitMaxWaves;
  const int64_t upw = (per + 7) / 8 * 8;  // whole steps of 4 units, 2 in flight
  if (upw > INT_MAX) return false;
  o.upw = static_cast<int>(upw);
  o.ks = static_cast<int>((nU + upw - 1) / upw);
  o.gpw = 0;
  o.ntb = N > 16 ? 2 : 1;
  o.rt = 1;
  o.lds = (static_cast<size_t>(o.ks) * o.ntb * 256 + static_cast<size_t>(o.ks) * 16 * 4 * kExWords) * sizeof(float);
  return true;
}

bool mma_shape(int fmt, int64_t K, int N, int x_f16, int64_t M, int cus, MmaShape& o) {
  if (fmt != FMT_A4G64) return mma_unit_shape(fmt, K, N, x_f16, o);
  o.upw = 0;
  if (!x_f16 || N < kMmaMinTokens || N > 32 || K % 64 != 0 || K < 64) return false;
  const int64_t G = K / 64;
  int gpw = 2;
  while (gpw <= 4 && (G + gpw - 1) / gpw > 16) ++gpw;
  if (gpw > 4) return false;
  o.gpw = gpw;
  o.ks = static_cast<int>((G + gpw - 1) / gpw);
  o.ntb = N > 16 ? 2 : 1;
  // two row tiles per wave (half the activation bytes per weight) when one-tile
  // workgroups would be more than one per CU: the 6144-row ffn_gate + ffn_up launch at
  // 16 tokens 6.97 -> 5.79 us; with fewer rows the halved workgroup count loses more
  // (q+k+v, 4096 rows: 5.05 -> 5.70 us)
  o.rt = (M + 15) / 16 > cus ? 2 : 1;
  o.lds = static_cast<size_t>(o.ks) * o.rt * o.ntb * 256 * sizeof(float);
  return true;
}

hipError_t launch_mma(int fmt, int64_t row_bytes, int64_t K, int N, const MmaShape& o, const GemvGroup& grp,
                      hipStream_t st) {
  GemvArgs a{};
  a.W = grp.W[0];  // a single matrix is read from these fields
  a.x = grp.x[0];
  a.y = grp.y[0];
  a.M = grp.M[0];
  a.row_bytes = row_bytes;
  a.nU = static_cast<int>(K / 32);
  a.K = static_cast<int>(K);
  a.rows_per_wg = 16 * o.rt;
  a.x_f16 = 1;
  a.N = N;
  a.chunk_units = o.upw;
  GemvGroupKernel k = o.upw > 0 ? tables().gm[fmt][o.ntb - 1] : tables().mma[o.ntb - 1][o.gpw - 2][o.rt - 1];
  hipLaunchKernelGGL(k, dim3(grp.first[grp.n]), dim3(64 * o.ks), o.lds, st, a,
                     grp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_group(const MatDesc* const* ms, const void* const* xs, float* const* ys, int n, int N,
                             int x_f16, hipStream_t st) {
  if (n < 1 || n > kGemvGroupMax || N < 1) return hipErrorNotSupported;
  const MatDesc& m0 = *ms[0];
  int64_t rows = 0;
  int fmt_b = 0;
  bool mixed = false;
  for (int i = 0; i < n; ++i) {
    if (ms[i]->K != m0.K || ms[i]->blocks == nullptr) return hipErrorNotSupported;
    if (ms[i]->fmt != m0.fmt) mixed = true;
    if (ms[i]->fmt == FMT_Q6_K) fmt_b |= 1 << i;
    rows += ms[i]->M;
  }
  if (mixed) {  // only Q4_K with Q6_K, at one token (k_gemv1_pair)
    if (N != 1) return hipErrorNotSupported;
    for (int i = 0; i < n; ++i)
      if (ms[i]->fmt != FMT_Q4_K && ms[i]->fmt != FMT_Q6_K) return hipErrorNotSupported;
  }
  const int nU = static_cast<int>(m0.K / 32);
  OneShape o;
  MultiShape mo;
  MmaShape mm;
  const bool mma = !mixed && mma_shape(m0.fmt, m0.K, N, x_f16, rows, m0.cus, mm);
  int RW;
  if (mma) {
    RW = 16 * mm.rt;
  } else if (N == 1) {
    if (!one_shape(mixed ? FMT_Q4_K : m0.fmt, nU, rows, x_f16, m0.cus, o, mixed ? tables().pair_regs : nullptr))
      return hipErrorNotSupported;
    RW = o.RW;
  } else {
    if (!multi_shape(m0.fmt, nU, rows, N, x_f16, m0.cus, mo)) return hipErrorNotSupported;
    RW = mo.RW;
  }
  // in a mixed launch the Q6_K matrices (the dearer decode) take the first workgroups,
  // so they are not the launch's tail (about 1% of the decode step)
  int order[kGemvGroupMax], k = 0;
  for (int pass = 0; pass < 2; ++pass)
    for (int i = 0; i < n; ++i)
      if (((fmt_b >> i) & 1) == (pass == 0 ? 1 : 0)) order[k++] = i;
  GemvGroup grp{};
  grp.n = n;
  grp.fmt_b = 0;
  int64_t wg = 0;
  for (int e = 0; e < n; ++e) {
    const int i = mixed ? order[e] : e;
    grp.W[e] = ms[i]->blocks;
    grp.x[e] = xs[i];
    grp.y[e] = ys[i];
    grp.M[e] = static_cast<int>(ms[i]->M);
    grp.first[e] = static_cast<int>(wg);
    if (mixed && ((fmt_b >> i) & 1)) grp.fmt_b |= 1 << e;
    wg += (ms[i]->M + RW - 1) / RW;
  }
  if (wg > INT_MAX) return hipErrorNotSupported;
  grp.first[n] = static_cast<int>(wg);
  if (mixed) {
    // (the formats' row bytes differ: the pair kernel derives each from its format)
    return launch_one(FMT_Q4_K, nU, 0, o, grp, x_f16, st, true);
  }
  const int64_t rb = static_cast<int64_t>(m0.row_bytes);
  if (mma) return launch_mma(m0.fmt, rb, m0.K, N, mm, grp, st);
  return N == 1 ? launch_one(m0.fmt, nU, rb, o, grp, x_f16, st) : launch_multi(m0.fmt, nU, rb, N, mo, grp, x_f16, st);
}

hipError_t launch_gemv(const MatDesc& m, const void* x, int x_f16, int N, float* y, hipStream_t st) {
  const int cus = m.cus;
  const int bi = bucket_index(N);
  if (bi < 0) return hipErrorInvalidValue;
  const int nU = static_cast<int>(m.K / 32);
  const int M = static_cast<int>(m.M);
  OneShape o;
  if (N == 1 && one_shape(m.fmt, nU, M, x_f16, cus, o)) {
    GemvGroup grp{};
    grp.n = 1;
    grp.W[0] = m.blocks;
    grp.x[0] = x;
    grp.y[0] = y;
    grp.M[0] = M;
    grp.first[0] = 0;
    grp.first[1] = (M + o.RW - 1) / o.RW;
    return launch_one(m.fmt, nU, static_cast<int64_t>(m.row_bytes), o, grp, x_f16, st);
  }
  MmaShape mm;
  if (mma_shape(m.fmt, m.K, N, x_f16, M, cus, mm)) {
    GemvGroup grp{};
    grp.n = 1;
    grp.W[0] = m.blocks;
    grp.x[0] = x;
    grp.y[0] = y;
    grp.M[0] = M;
    grp.first[0] = 0;
    grp.first[1] = (M + 16 * mm.rt - 1) / (16 * mm.rt);
    return launch_mma(m.fmt, static_cast<int64_t>(m.row_bytes), m.K, N, mm, grp, st);
  }
  if (N >= 2) {
    MultiShape ms;
    if (multi_shape(m.fmt, nU, M, N, x_f16, cus, ms)) {
      GemvGroup grp{};
      grp.n = 1;
      grp.W[0] = m.blocks;
      grp.x[0] = x;
      grp.y[0] = y;
      grp.M[0] = M;
      grp.first[0] = 0;
      grp.first[1] = (M + ms.RW - 1) / ms.RW;
      return launch_multi(m.fmt, nU, static_cast<int64_t>(m.row_bytes), N, ms, grp, x_f16, st);
    }
  }
  // about one workgroup per CU
  const Shape s = make_shape(M, nU, kRuns[m.fmt], kBuckets[bi], (M + cus - 1) / cus);
  GemvArgs a{};
  a.W = m.blocks;
  a.row_bytes = m.row_bytes;
  a.expert_bytes = m.row_bytes * static_cast<u64>(m.M);
  a.M = static_cast<int>(m.M);
  a.nU = nU;
  a.K = static_cast<int>(m.K);
  a.rows_per_wg = s.RW;
  a.chunk_units = s.KC;
  a.x = x;
  a.x_f16 = x_f16;
  a.y = y;
  a.N = N;
  hipLaunchKernelGGL(tables().dense[m.fmt][bi], dim3(s.grid), dim3(s.threads), s.lds, st, a);
  return hipGetLastError();
}

hipError_t launch_gemv_id(const MatDesc& m, const void* x, int x_f16, int N, int S, int x_per_slot,
                          const int32_t* ids, float* y, hipStream_t st) {
  const int cus = m.cus;
  // pairs per expert: at most N when a token's ids are distinct, and about
  // N * S / E in a routed batch; a workgroup takes them NB <= 4 at a time
  const int bi = bucket_index(N < 4 ? N : 4);
  if (bi < 0) return hipErrorInvalidValue;
  const int nU = static_cast<int>(m.K / 32);
  const int64_t P = static_cast<int64_t>(N) * S;
  const int ranks = static_cast<int>(P < m.n_experts ? P : m.n_experts);
  // the grid is ranks x row slices: about two workgroups per CU over all the
  // active experts
  const int M = static_cast<int>(m.M);
  const int64_t spc = ((m.M + 3) / 4 + 7) / 8 * 8;  // the narrow kernel's steps per pair chunk
  if (m.fmt == FMT_Q4_0 && nU == 16) {
    GemvArgs a{};
    a.W = m.blocks;
    a.row_bytes = m.row_bytes;
    a.expert_bytes = m.row_bytes * static_cast<u64>(m.M);
    a.M = M;
    a.nU = nU;
    a.K = static_cast<int>(m.K);
    a.x = x;
    a.x_f16 = x_f16;
    a.y = y;
    a.N = N;
    a.ids = ids;
    a.S = S;
    a.x_per_slot = x_per_slot;
    a.E = static_cast<int>(m.n_experts);
    const int h = x_f16 ? 1 : 0;
    if (P <= 64 || P > kNarrowMaxPairs || P * spc >= (int64_t(1) << 30)) {
      // about four 256-thread workgroups per CU over the ranks, each streaming a
      // slice of its expert's rows (a multiple of the 16 rows of a step), at least
      // 128 rows so that the routing stays a small part of it.  Measured on 128
      // experts of 4096 rows at 2, 8 and 24 tokens (slices of 128-1024 rows, rings
      // of 4-16 items).
      const int slices = (4 * cus + ranks - 1) / ranks;
      int RW = (M + slices - 1) / slices;
      RW = (RW + 15) / 16 * 16;
      if (RW < 128) RW = 128;
      a.rows_per_wg = RW;
      hipLaunchKernelGGL(tables().slices_id[h], dim3((M + RW - 1) / RW, ranks), dim3(256), 0, st, a);
      return hipGetLastError();
    }
    // a persistent grid (every workgroup resident at once), the work split evenly
    // over its waves
    const size_t lds = narrow_lds_ints(a.E, static_cast<int>(P)) * sizeof(int);
    hipLaunchKernelGGL(tables().narrow_id[h], dim3(tables().narrow_occ[h] * cus), dim3(256), lds, st, a);
    return hipGetLastError();
  }
  {
    // the few-token layout per expert: about two workgroups per CU over the
    // active experts, each G row groups x id_rows rows per thread, the pairs
    // staged TP at a time in one round
    const int ipr = nU / kRuns[m.fmt];
    const int Rk = kRuns[m.fmt] == 1 ? 4 : 2;
    const int Gmax = 512 / ipr;
    if (Gmax >= 1) {
      const int slices_want = (2 * cus + ranks - 1) / ranks;
      const int rows_want = (M + slices_want - 1) / slices_want;
      int Ge = (rows_want + Rk - 1) / Rk;
      if (Ge > Gmax) Ge = Gmax;
      const int RW = Ge * Rk;
      const bool xh = x_f16 != 0;
      const int P = N * S;
      int TP = P;
      // (the routing tables take static LDS besides the dynamic budget)
      const size_t budget = static_cast<size_t>(kLdsBudget) - sizeof(IdShared);
      while (TP > 0 && multi_lds_floats(xh, nU, RW, TP) * sizeof(float) > budget) --TP;
      int TGN = TP < 512 / (Ge * ipr) ? TP : 512 / (Ge * ipr);
      if (TGN < 1) TGN = 1;
      const int threads = (Ge * TGN * ipr + 63) / 64 * 64;
      if (TP > threads / (2 * nU)) TP = threads / (2 * nU);
      if (TGN > TP) TGN = TP;
      if (TP >= 1) {
        GemvArgs a{};
        a.W = m.blocks;
        a.row_bytes = m.row_bytes;
        a.expert_bytes = m.row_bytes * static_cast<u64>(m.M);
        a.M = M;
        a.nU = nU;
        a.K = static_cast<int>(m.K);
        a.rows_per_wg = RW;
        a.chunk_units = Ge;
        a.x = x;
        a.x_f16 = x_f16;
        a.y = y;
        a.N = N;
        a.ids = ids;
        a.S = S;
        a.x_per_slot = x_per_slot;
        a.E = static_cast<int>(m.n_experts);
        a.tok_groups = TGN;
        a.tok_pass = TP;
        const size_t lds = multi_lds_floats(xh, nU, RW, TP) * sizeof(float);
        hipLaunchKernelGGL(tables().multi_id[m.fmt][xh ? 1 : 0], dim3((M + RW - 1) / RW, ranks), dim3(threads), lds,
                           st, a);
        return hipGetLastError();
      }
    }
  }
  const int slices = (2 * cus + ranks - 1) / ranks;
  // (256 threads: each workgroup streams a short slice, and two share a CU)
  const Shape s = make_shape(M, nU, kRuns[m.fmt], kBuckets[bi], (M + slices - 1) / slices, 256);
  GemvArgs a{};
  a.W = m.blocks;
  a.row_bytes = m.row_bytes;
  a.expert_bytes = m.row_bytes * static_cast<u64>(m.M);
  a.M = M;
  a.nU = nU;
  a.K = static_cast<int>(m.K);
  a.rows_per_wg = s.RW;
  a.chunk_units = s.KC;
  a.x = x;
  a.x_f16 = x_f16;
  a.y = y;
  a.N = N;
  a.ids = ids;
  a.S = S;
  a.x_per_slot = x_per_slot;
  a.E = static_cast<int>(m.n_experts);
  hipLaunchKernelGGL(tables().id[m.fmt][bi], dim3(s.grid, ranks), dim3(s.threads), s.lds, st, a);
  return hipGetLastError();
}

}  // namespace qmm
