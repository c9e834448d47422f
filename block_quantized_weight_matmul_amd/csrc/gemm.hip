// gemm.hip -- token-tiled matrix-matrix path on the gfx950 matrix cores.
//
// Candle pull request "Metal: 64-token tile for the quantized matrix-matrix
// kernel": a workgroup owns a tile of weight rows; on every step along K it
// reads those rows' blocks, dequantizes them once and multiplies them by every
// token of its token tile (section "Why the tile sets the weight reuse"); the
// token tile is 32 or 64, the 64-token tile used only when it pads no more
// tokens (section "Where the 64-token tile is used"), and both give
// bit-identical outputs (section "Same results, bit for bit").
//
// On gfx950.  A workgroup of 4 waves owns 64*RB weight rows and a super-tile of
// TT tokens (64, 128 or 256), made of whole 32- or 64-token tiles: the token
// tile T is the padding granularity of the last super-tile, the waste the rule
// above trades against reuse, and TT is the reuse the matrix cores need (a
// weight decoded costs a few VALU operations, which the 16-cycle
// v_mfma_f32_16x16x32_f16 only hides when each weight meets >= 128 tokens).
// Each wave owns 16*RB rows and decodes them straight into the A operand of
// the MFMA (lane l: row l % 16, weights 8*(l/16) .. +7 of a 32-deep step): the
// exact fp32 weight, rounded to fp16 nearest-even -- the value the pages stage
// in threadgroup memory -- kept in registers rather than LDS, since no other
// wave reads it.  Activations are staged as fp16 in LDS, double buffered over
// 64-deep K stages, and read as B operands by all four waves; the weight bytes
// and activations of stage s+1 are fetched while stage s is multiplied.
//
// Bit identity of the tiles: output (row r, token t) is accumulated by the wave
// owning r, at lane (r % 16, t % 16) of one 16x16 block, from the same fp16
// operands over the same 32-deep steps in the same order, whatever T, TT and
// RB are; T only changes how many padding blocks of the last super-tile are
// computed (and never stored).
#include <algorithm>
#include <atomic>
#include <climits>
#include <mutex>
#include <type_traits>

#include "decode.hpp"
#include "internal.hpp"
#include "qmm.h"

namespace qmm {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
  const u8* W;
  u32 row_bytes;
  int M, nU, K;
  const void* x;
  int N;
  float* y;
  int y_vec;        // y rows can take 16-byte stores (M % 4 == 0, y 16-byte aligned)
  int T;            // token tile (32 or 64)
  int n_row_tiles;  // blockIdx.x = super_tile * n_row_tiles + row_tile
  int split_stages; // K stages per split (blockIdx.y = split); all of K when unsplit
  u64 split_floats; // floats between the splits' partial outputs (0 when unsplit)
  // expert-indexed (k_gemm_id): ids [N, S], E experts of expert_bytes each;
  // id_groups row-tile groups per expert rank, ranks padded to a multiple of 8
  const int32_t* ids;
  int S, x_per_slot, E;
  u64 expert_bytes;
  int id_groups, id_ranks;
};

constexpr int kKS = 64;  // K per stage: two 32-deep MFMA steps (two units)
constexpr int64_t kSkMaxTokens = 16;  // split calls of up to this many tokens take k_gemm_sk

// LDS slot (in halves) of k-chunk c (8 values) of token row r of a stage buffer:
// 128-byte rows, so rows 2i and 2i+1 share one 256-byte line of the 64 four-byte
// banks, in its lower and upper half.  The chunk index is XOR-swizzled by
// (r / 2) % 8: the 16 rows a B-operand read touches (one chunk each) then cover
// all 64 banks once.  Swizzling by r % 8 would put rows r and r + 8 on the same
// banks, a two-way conflict on every B read.
__device__ __forceinline__ int x_slot(int r, int c) { return r * kKS + 8 * (c ^ ((r >> 1) & 7)); }

// ---------------------------------------------------------------------------------------------
// A operands.  The K order inside a 64-deep stage is permuted so that each lane
// decodes 16 weights of one unit with one set of coefficients: lane group
// g = l / 16 takes unit g / 2 of the stage, weights 16(g % 2) .. +15, which feed
// step j = 0, 1 as k-chunk 2g + j (8 weights).  The activations are read with
// the same chunk order, so each step is still a sum over 32 distinct K positions
// and the stage over all 64; every output uses the same order whatever the tile.
//
// Codes become fp16 without a conversion per weight: a byte b placed under the
// exponent byte 0x64 is the fp16 value 1024 + b (ulp 1 in [1024, 2048)), two per
// v_perm_b32; 1024 + z is then subtracted exactly in packed fp16.  The weight is
// formed either in packed fp16 -- when d * (q - z) is exact in fp32 and d is an
// fp16 value, one fp16 rounding of it is the fp16 rounding of the fp32 weight --
// or with v_fma_mix (fp16 code, fp32 coefficients, fp32 fma rounded to fp16),
// which rounds the same exact fp32 weight the dequantizer produces.

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half2v bits_h2(u32 v) { return __builtin_bit_cast(half2v, v); }

// fp16 pairs (1024 + byte0, 1024 + byte1) and (1024 + byte2, 1024 + byte3) of c
__device__ __forceinline__ half2v code_pair_lo(u32 c) { return bits_h2(__builtin_amdgcn_perm(c, 0x64646464u, 0x00050004u)); }
__device__ __forceinline__ half2v code_pair_hi(u32 c) { return bits_h2(__builtin_amdgcn_perm(c, 0x64646464u, 0x00070006u)); }
// fp16 pairs (byte0, byte1) * 2^-24 and (byte2, byte3) * 2^-24 of c: the bytes
// as fp16 subnormals, exact, which the fp32 widening inside v_fma_mix keeps
__device__ __forceinline__ half2v code_pair_lo_sub(u32 c) { return bits_h2(__builtin_amdgcn_perm(c, 0u, 0x0C050C04u)); }
__device__ __forceinline__ half2v code_pair_hi_sub(u32 c) { return bits_h2(__builtin_amdgcn_perm(c, 0u, 0x0C070C06u)); }

// 8 weights from two code words (4 codes each, in bytes), packed fp16 path:
// w = (code - zero) * d, with 1024 + zero subtracted exactly first.
__device__ __forceinline__ half8 weights_pk(u32 c0, u32 c1, half2v off, half2v d) {
  const half2v p0 = (code_pair_lo(c0) - off) * d;
  const half2v p1 = (code_pair_hi(c0) - off) * d;
  const half2v p2 = (code_pair_lo(c1) - off) * d;
  const half2v p3 = (code_pair_hi(c1) - off) * d;
  return half8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// 8 weights from code bytes, fp32-coefficient path, codes as fp16 subnormals:
// w = fp16(fma(code * 2^-24, a24, b)) with a24 = a * 2^24 (exact), so the fma
// forms the same exact code * a + b, rounded once to fp32 then to fp16, as
// fma(code, a, b) -- with no subtraction of an offset per pair.  The fp32 weight
// is held opaque before its conversion: the compiler would otherwise fuse the
// fma and the conversion into one v_fma_mix with an fp16 result, which rounds
// the exact code * a + b once, to fp16, and differs from the fp16 rounding of
// the fp32 weight where that weight is an fp16 tie (measured: a Q4_K weight of
// exact value 2 + 2^-10 + 2^-24 staged as 2 + 2^-9 instead of 2).  The pairs are
// converted by v_cvt_pk_f16_f32 (nearest even).
typedef float float2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ half8 weights_sub(u32 c0, u32 c1, float a24, float b) {
  const half2v p[4] = {code_pair_lo_sub(c0), code_pair_hi_sub(c0), code_pair_lo_sub(c1), code_pair_hi_sub(c1)};
  half8 h;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float f0 = __builtin_fmaf(static_cast<float>(p[i][0]), a24, b);
    float f1 = __builtin_fmaf(static_cast<float>(p[i][1]), a24, b);
    asm("" : "+v"(f0), "+v"(f1));
    const half2v r = __builtin_convertvector(float2v{f0, f1}, half2v);
    h[2 * i] = r[0];
    h[2 * i + 1] = r[1];
  }
  return h;
}

// 8 weights, fp32-coefficient path: w = fp16(fma(code - off, a, b)); off is
// subtracted exactly in fp16 (or 0 when b already absorbs it).  Used where the
// weight is exact in fp32 (Q6_K: (q - 32) * a), so the one rounding of a fused
// fma-to-fp16 is the fp16 rounding of the fp32 weight.
template <bool SUB>
__device__ __forceinline__ half8 weights_mix(u32 c0, u32 c1, half2v off, float a, float b) {
  half2v p[4] = {code_pair_lo(c0), code_pair_hi(c0), code_pair_lo(c1), code_pair_hi(c1)};
  half8 h;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2v q = SUB ? p[i] - off : p[i];
    h[2 * i] = static_cast<_Float16>(__builtin_fmaf(static_cast<float>(q[0]), a, b));
    h[2 * i + 1] = static_cast<_Float16>(__builtin_fmaf(static_cast<float>(q[1]), a, b));
  }
  return h;
}

// Weight bytes are addressed as a 32-bit offset from the matrix base (a matrix
// is below 4 GiB and its base 16-byte aligned), so the loads take the base from
// scalar registers and one 32-bit offset per lane.
__device__ __forceinline__ u32 ld32(const u8* base, u32 off) {
  return *reinterpret_cast<const u32*>(base + static_cast<u64>(off));
}
__device__ __forceinline__ u32 ld16(const u8* base, u32 off) {
  return *reinterpret_cast<const u16*>(base + static_cast<u64>(off));
}
__device__ __forceinline__ uint4 ld128(const u8* base, u32 off) {
  return *reinterpret_cast<const uint4*>(base + static_cast<u64>(off));
}
// 16 bytes at a dword-aligned offset, as one dwordx4 load.
typedef u32 u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
__device__ __forceinline__ void ld128_a4(const u8* base, u32 off, u32 (&w)[4]) {
  const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(base + static_cast<u64>(off));
  w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
}
// 16 bytes at base + off (off any alignment): the dwordx4 at the enclosing dword
// plus the dword holding the last byte (a repeat of the fourth when off is
// dword aligned), kept raw and realigned with v_alignbit when read, so the wait
// for the data comes where the words are used.  Two loads, no branch, nothing
// read past the dword of the range's last byte.
struct Bytes16 {
  u32 raw[5];
  u32 sh;
  __device__ __forceinline__ void load(const u8* base, u32 off) {
    u32 v[4];
    ld128_a4(base, off & ~3u, v);
    raw[0] = v[0]; raw[1] = v[1]; raw[2] = v[2]; raw[3] = v[3];
    raw[4] = ld32(base, (off + 15u) & ~3u);
    sh = (off & 3u) * 8u;
  }
  __device__ __forceinline__ u32 word(int j) const { return __builtin_amdgcn_alignbit(raw[j + 1], raw[j], sh); }
};

// zero_second(g): the lanes of the stage's second unit get zero coefficients
// (all-zero weights), for a last stage whose second unit lies past K.
template <int F> struct AStage;

// Q4_0 (unit = block): weights 16h .. 16h+15 are nibble h of code bytes 0 .. 15.
template <> struct AStage<FMT_Q4_0> {
  Bytes16 q;
  u32 d;
  __device__ __forceinline__ void zero_second(int g) { if (g >= 2) d = 0; }
  __device__ __forceinline__ void load(const u8* W, u32 row_off, int u0, int nU, int g) {
    const u32 bo = row_off + 18u * static_cast<u32>(min(u0 + (g >> 1), nU - 1));
    q.load(W, bo + 2);
    d = ld16(W, bo);
  }
  __device__ __forceinline__ void operands(int g, half8 (&A)[2]) const {
    const u32 sh = 4u * static_cast<u32>(g & 1);
    const half2v dd = bits_h2(d * 0x10001u);
    const half2v off = half2v{1032, 1032};
#pragma unroll
    for (int j = 0; j < 2; ++j)
      A[j] = weights_pk((q.word(2 * j) >> sh) & 0x0F0F0F0Fu, (q.word(2 * j + 1) >> sh) & 0x0F0F0F0Fu, off, dd);
  }
};

// Q8_0: weights 16h .. 16h+15 are code bytes 16h .. +15 (int8; ^0x80 gives q + 128).
template <> struct AStage<FMT_Q8_0> {
  Bytes16 q;
  u32 d;
  __device__ __forceinline__ void zero_second(int g) { if (g >= 2) d = 0; }
  __device__ __forceinline__ void load(const u8* W, u32 row_off, int u0, int nU, int g) {
    const u32 bo = row_off + 34u * static_cast<u32>(min(u0 + (g >> 1), nU - 1));
    q.load(W, bo + 2 + 16 * (g & 1));
    d = ld16(W, bo);
  }
  __device__ __forceinline__ void operands(int, half8 (&A)[2]) const {
    const half2v dd = bits_h2(d * 0x10001u);
    const half2v off = half2v{1152, 1152};
#pragma unroll
    for (int j = 0; j < 2; ++j) A[j] = weights_pk(q.word(2 * j) ^ 0x80808080u, q.word(2 * j + 1) ^ 0x80808080u, off, dd);
  }
};

// Q4_K: the stage is sub-blocks 2p (low nibbles) and 2p+1 (high nibbles) of code
// bytes 32p .. 32p+31; lane group g takes sub-block 2p + g/2, bytes 32p + 16(g%2)
// .. +15.  A high nibble stays in place (16 * code) and meets a / 16: the product
// is the same exact fp32 value.
template <> struct AStage<FMT_Q4_K> {
  u32 h[4];
  u32 q[4];
  int p;
  __device__ __forceinline__ void zero_second(int g) { if (g >= 2) h[0] = 0; }
  __device__ __forceinline__ void load(const u8* W, u32 row_off, int u0, int, int g) {
    const u32 so = row_off + 144u * static_cast<u32>(u0 >> 3);
    p = (u0 >> 1) & 3;
    const uint4 hv = ld128(W, so);
    const uint4 qv = ld128(W, so + 16 + 32 * p + 16 * (g & 1));
    h[0] = hv.x; h[1] = hv.y; h[2] = hv.z; h[3] = hv.w;
    q[0] = qv.x; q[1] = qv.y; q[2] = qv.z; q[3] = qv.w;
  }
  __device__ __forceinline__ void operands(int g, half8 (&A)[2]) const {
    const u32 hi = static_cast<u32>(g >> 1);
    // sc_j, m_j (j = 2p + hi): 6-bit fields at bits 6j and 48 + 6j of h[1..3]
    const u32 bs = 6u * (2u * static_cast<u32>(p) + hi);
    const u32 s0 = __builtin_amdgcn_alignbit(h[2], h[1], bs & 31u);
    const u32 s1 = __builtin_amdgcn_alignbit(h[3], h[2], bs & 31u);
    const u32 sc = (bs < 32 ? s0 : s1) & 63u;
    const u32 bm = 48u + bs;
    const u32 m0 = __builtin_amdgcn_alignbit(h[3], h[2], bm & 31u);
    const u32 m1 = h[3] >> (bm & 31u);
    const u32 m = (bm < 64 ? m0 : m1) & 63u;
    // a * 2^24, exact: the codes enter as fp16 subnormals (code * 2^-24)
    const float a24 = h2f(h[0]) * static_cast<float>(sc) * (hi ? 1048576.0f : 16777216.0f);
    const float b = -(h2f(h[0] >> 16) * static_cast<float>(m));  // exact
    const u32 mask = hi ? 0xF0F0F0F0u : 0x0F0F0F0Fu;
#pragma unroll
    for (int j = 0; j < 2; ++j) A[j] = weights_sub(q[2 * j] & mask, q[2 * j + 1] & mask, a24, b);
  }
};

// Q6_K: the stage is units a0, a0+1 (a0 even); lane group g takes unit a = a0 + g/2,
// weights 16(g%2) .. +15: nibble a/4 of ql[32(a%4) + i] and bits 2(a/2) .. +1 of
// qh[32(a%2) + i], i = 16(g%2) .. +15, all in sub-block 2a + g%2 (one scale).
// fma(1024 + q, a, -1056 a) is the exact (q - 32) a rounded once: -1056 a is exact.
template <> struct AStage<FMT_Q6_K> {
  Bytes16 ql;
  Bytes16 qh;
  u32 d;
  u32 sc;
  int a;
  __device__ __forceinline__ void zero_second(int g) { if (g >= 2) d = 0; }
  __device__ __forceinline__ void load(const u8* W, u32 row_off, int u0, int, int g) {
    const u32 so = row_off + 210u * static_cast<u32>(u0 >> 3);
    a = (u0 & 7) + (g >> 1);
    ql.load(W, so + 18 + 32 * (a & 3) + 16 * (g & 1));
    qh.load(W, so + 146 + 32 * (a & 1) + 16 * (g & 1));
    d = ld16(W, so);
    sc = W[static_cast<u64>(so + 2 + 2 * a + (g & 1))];
  }
  __device__ __forceinline__ void operands(int, half8 (&A)[2]) const {
    const u32 lsh = 4u * static_cast<u32>(a >> 2);
    const u32 hsh = 2u * static_cast<u32>(a >> 1);
    const float ac = h2f(d) * static_cast<float>(static_cast<int8_t>(sc & 0xFFu));  // exact
    const float bc = -1056.0f * ac;                                                 // exact
    u32 c[4];
#pragma unroll
    for (int w = 0; w < 4; ++w)
      c[w] = ((ql.word(w) >> lsh) & 0x0F0F0F0Fu) | (((qh.word(w) >> hsh) & 0x03030303u) << 4);
#pragma unroll
    for (int j = 0; j < 2; ++j) A[j] = weights_mix<false>(c[2 * j], c[2 * j + 1], half2v{0, 0}, ac, bc);
  }
};

// A4G64: the stage is one group; lane group g takes nibble g/2 of code bytes
// 16(g%2) .. +15 (high nibble in place with scale / 16).
template <> struct AStage<FMT_A4G64> {
  u32 hdr;
  u32 q[4];
  __device__ __forceinline__ void zero_second(int g) { if (g >= 2) hdr = 0; }
  __device__ __forceinline__ void load(const u8* W, u32 row_off, int u0, int, int g) {
    const u32 go = row_off + 36u * static_cast<u32>(u0 >> 1);
    hdr = ld32(W, go);
    ld128_a4(W, go + 4 + 16 * (g & 1), q);
  }
  __device__ __forceinline__ void operands(int g, half8 (&A)[2]) const {
    const bool hi = (g >> 1) != 0;
    const float a24 = h2f(hdr) * (hi ? 1048576.0f : 16777216.0f);  // scale * 2^24 (/16 high), exact
    const float b = h2f(hdr >> 16);
    const u32 mask = hi ? 0xF0F0F0F0u : 0x0F0F0F0Fu;
#pragma unroll
    for (int j = 0; j < 2; ++j) A[j] = weights_sub(q[2 * j] & mask, q[2 * j + 1] & mask, a24, b);
  }
};

// Q4_1 (unit = block, 20 bytes, 4-byte aligned): weights 16h .. 16h+15 are nibble h of
// code bytes 0 .. 15; w = d * q + m (one rounding: the fp32-then-fp16 path).
template <> struct AStage<FMT_Q4_1> {
  u32 hdr;
  u32 q[4];
  __device__ __forceinline__ void zero_second(int g) { if (g >= 2) hdr = 0; }
  __device__ __forceinline__ void load(const u8* W, u32 row_off, int u0, int nU, int g) {
    const u32 bo = row_off + 20u * static_cast<u32>(min(u0 + (g >> 1), nU - 1));
    hdr = ld32(W, bo);
    ld128_a4(W, bo + 4, q);
  }
  __device__ __forceinline__ void operands(int g, half8 (&A)[2]) const {
    const bool hi = (g & 1) != 0;
    const float a24 = h2f(hdr) * (hi ? 1048576.0f : 16777216.0f);  // d * 2^24 (/16 high), exact
    const float b = h2f(hdr >> 16);
    const u32 mask = hi ? 0xF0F0F0F0u : 0x0F0F0F0Fu;
#pragma unroll
    for (int j = 0; j < 2; ++j) A[j] = weights_sub(q[2 * j] & mask, q[2 * j + 1] & mask, a24, b);
  }
};

// The four-byte spread of the top bits of codes 4k .. 4k+3 (bits t .. t+3 of qh), at bit
// `at` of each byte.
__device__ __forceinline__ u32 top_bits4(u32 qh, u32 t, u32 at) { return spread4((qh >> t) & 15u) << at; }

// Q5_0 (22-byte blocks, 2-byte aligned): weights 16h + i are nibble h of code byte i with
// bit 16h + i of qh on top; w = d * (q - 16), exact in fp32, formed in packed fp16.
template <> struct AStage<FMT_Q5_0> {
  Bytes16 q;
  u32 qh0, qh1, qsh;
  u32 d;
  __device__ __forceinline__ void zero_second(int g) { if (g >= 2) d = 0; }
  __device__ __forceinline__ void load(const u8* W, u32 row_off, int u0, int nU, int g) {
    const u32 bo = row_off + 22u * static_cast<u32>(min(u0 + (g >> 1), nU - 1));
    q.load(W, bo + 6);
    qh0 = ld32(W, (bo + 2) & ~3u);   // the dwords holding qh's first and last byte
    qh1 = ld32(W, (bo + 5) & ~3u);
    qsh = ((bo + 2) & 3u) * 8u;
    d = ld16(W, bo);
  }
  __device__ __forceinline__ void operands(int g, half8 (&A)[2]) const {
    const u32 h = static_cast<u32>(g & 1);
    const u32 qh = __builtin_amdgcn_alignbit(qh1, qh0, qsh);
    const half2v dd = bits_h2(d * 0x10001u);
    const half2v off = half2v{1040, 1040};
    u32 c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = ((q.word(k) >> (4u * h)) & 0x0F0F0F0Fu) | top_bits4(qh, 16u * h + 4u * k, 4u);
#pragma unroll
    for (int j = 0; j < 2; ++j) A[j] = weights_pk(c[2 * j], c[2 * j + 1], off, dd);
  }
};

// Q5_1 (24-byte blocks, 8-byte aligned): codes as Q5_0; w = d * q + m.
template <> struct AStage<FMT_Q5_1> {
  u32 hdr, qh;
  u32 q[4];
  __device__ __forceinline__ void zero_second(int g) { if (g >= 2) hdr = 0; }
  __device__ __forceinline__ void load(const u8* W, u32 row_off, int u0, int nU, int g) {
    const u32 bo = row_off + 24u * static_cast<u32>(min(u0 + (g >> 1), nU - 1));
    hdr = ld32(W, bo);
    qh = ld32(W, bo + 4);
    ld128_a4(W, bo + 8, q);
  }
  __device__ __forceinline__ void operands(int g, half8 (&A)[2]) const {
    const u32 h = static_cast<u32>(g & 1);
    const float a24 = h2f(hdr) * 16777216.0f;  // d * 2^24, exact
    const float b = h2f(hdr >> 16);
    u32 c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = ((q[k] >> (4u * h)) & 0x0F0F0F0Fu) | top_bits4(qh, 16u * h + 4u * k, 4u);
#pragma unroll
    for (int j = 0; j < 2; ++j) A[j] = weights_sub(c[2 * j], c[2 * j + 1], a24, b);
  }
};

// Q2_K (84-byte super-blocks, 4-byte aligned): the stage is units a0, a0+1 (a0 even) of a
// super-block; lane group g takes unit a = a0 + g/2, 16-weight sub-block j = 2a + g%2:
// bits 2(a/2) .. +1 of qs[32(a%2) + 16(g%2) + i]; sc_j, m_j the nibbles of sm[j].
template <> struct AStage<FMT_Q2_K> {
  u32 hdr, sm, smsh;
  u32 q[4];
  int a;
  __device__ __forceinline__ void zero_second(int g) { if (g >= 2) hdr = 0; }
  __device__ __forceinline__ void load(const u8* W, u32 row_off, int u0, int, int g) {
    const u32 so = row_off + 84u * static_cast<u32>(u0 >> 3);
    a = (u0 & 7) + (g >> 1);
    const u32 jb = so + 4u + 2u * static_cast<u32>(a) + static_cast<u32>(g & 1);  // byte sm[j]
    hdr = ld32(W, so);
    sm = ld32(W, jb & ~3u);
    smsh = (jb & 3u) * 8u;
    ld128_a4(W, so + 20u + 32u * static_cast<u32>(a & 1) + 16u * static_cast<u32>(g & 1), q);
  }
  __device__ __forceinline__ void operands(int, half8 (&A)[2]) const {
    const u32 sh = 2u * static_cast<u32>(a >> 1);
    const u32 f = sm >> smsh;
    const float a24 = h2f(hdr) * static_cast<float>(f & 15u) * 16777216.0f;  // exact
    const float b = -(h2f(hdr >> 16) * static_cast<float>((f >> 4) & 15u));   // exact
#pragma unroll
    for (int j = 0; j < 2; ++j)
      A[j] = weights_sub((q[2 * j] >> sh) & 0x03030303u, (q[2 * j + 1] >> sh) & 0x03030303u, a24, b);
  }
};

// Q3_K (110-byte super-blocks, 2-byte aligned): lane group g takes unit a = a0 + g/2,
// sub-block j = 2a + g%2: low bits 2(a/2) .. +1 of ql[32(a%2) + 16(g%2) + i], top bit a
// of qh[16(g%2) + i], scale field j of the 6-bit string.  (q - 4) * d * (s - 32) is exact
// in fp32, so the fused fma-to-fp16 rounds it once, as the fp32-then-fp16 path would.
template <> struct AStage<FMT_Q3_K> {
  Bytes16 ql, qh;
  u32 d, s0, s1, ssh;
  int a;
  __device__ __forceinline__ void zero_second(int g) { if (g >= 2) d = 0; }
  __device__ __forceinline__ void load(const u8* W, u32 row_off, int u0, int, int g) {
    const u32 so = row_off + 110u * static_cast<u32>(u0 >> 3);
    a = (u0 & 7) + (g >> 1);
    const u32 h = static_cast<u32>(g & 1);
    const u32 j = 2u * static_cast<u32>(a) + h;
    ql.load(W, so + 14u + 32u * static_cast<u32>(a & 1) + 16u * h);
    qh.load(W, so + 78u + 16u * h);
    d = ld16(W, so);
    // the two bytes holding field j (bits 6j .. 6j+5 of the string at so + 2)
    const u32 fb = so + 2u + ((6u * j) >> 3);
    s0 = ld32(W, fb & ~3u);
    s1 = ld32(W, (fb + 1u) & ~3u);
    ssh = (fb & 3u) * 8u + ((6u * j) & 7u);
  }
  __device__ __forceinline__ void operands(int, half8 (&A)[2]) const {
    const u32 sh = 2u * static_cast<u32>(a >> 1);
    const u32 hb = static_cast<u32>(a);
    const u32 f = (__builtin_amdgcn_alignbit(s1, s0, ssh & 24u) >> (ssh & 7u)) & 63u;
    const float ac = h2f(d) * static_cast<float>(static_cast<int>(f) - 32);  // exact
    u32 c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      c[k] = ((ql.word(k) >> sh) & 0x03030303u) | (((qh.word(k) >> hb) & 0x01010101u) << 2);
#pragma unroll
    for (int j = 0; j < 2; ++j) A[j] = weights_mix<true>(c[2 * j], c[2 * j + 1], half2v{1028, 1028}, ac, 0.0f);
  }
};

// Q5_K (176-byte super-blocks, 16-byte aligned): lane group g takes sub-block a = a0 + g/2,
// weights 16(g%2) .. +15: nibble a%2 of qs[32(a/2) + 16(g%2) + i] with bit a of
// qh[16(g%2) + i] on top; sc_a, m_a as Q4_K.
template <> struct AStage<FMT_Q5_K> {
  u32 h[4];
  u32 q[4];
  u32 qh[4];
  int a;
  __device__ __forceinline__ void zero_second(int g) { if (g >= 2) h[0] = 0; }
  __device__ __forceinline__ void load(const u8* W, u32 row_off, int u0, int, int g) {
    const u32 so = row_off + 176u * static_cast<u32>(u0 >> 3);
    a = (u0 & 7) + (g >> 1);
    const u32 hh = 16u * static_cast<u32>(g & 1);
    const uint4 hv = ld128(W, so);
    const uint4 qhv = ld128(W, so + 16u + hh);
    const uint4 qv = ld128(W, so + 48u + 32u * static_cast<u32>(a >> 1) + hh);
    h[0] = hv.x; h[1] = hv.y; h[2] = hv.z; h[3] = hv.w;
    qh[0] = qhv.x; qh[1] = qhv.y; qh[2] = qhv.z; qh[3] = qhv.w;
    q[0] = qv.x; q[1] = qv.y; q[2] = qv.z; q[3] = qv.w;
  }
  __device__ __forceinline__ void operands(int, half8 (&A)[2]) const {
    const u32 j = static_cast<u32>(a);
    const u32 sc = six_bit_field(h[1], h[2], h[3], j);
    const u32 m = six_bit_field(h[1], h[2], h[3], 8u + j);
    const float a24 = h2f(h[0]) * static_cast<float>(sc) * 16777216.0f;  // exact
    const float b = -(h2f(h[0] >> 16) * static_cast<float>(m));           // exact
    const u32 sh = 4u * (j & 1u);
    u32 c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = ((q[k] >> sh) & 0x0F0F0F0Fu) | (((qh[k] >> j) & 0x01010101u) << 4);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) A[jj] = weights_sub(c[2 * jj], c[2 * jj + 1], a24, b);
  }
};

// ---------------------------------------------------------------------------------------------
// Activations of one stage: K [k0, k0 + 64) of tokens [tok0, tok0 + TT), as TT*8
// chunks of 8 values spread over the 256 threads; held in registers from load
// to store so the global loads stay in flight across the stage's products.
// fp32 input is rounded to fp16 (nearest even) at store time.  Stored in the
// natural chunk order; the K permutation of the A operands is applied when the
// B operands are read.
template <int TT, bool XF16> struct XStage;

// Loads are unconditional: token rows past N read token N-1 instead (they only
// feed outputs of tokens that are never stored).  Each lane's chunks sit at fixed
// 32-bit byte offsets from the super-tile's first row (TT * K * element size is
// below 4 GiB), the stage's K offset goes into the scalar base.  K past the end
// (K / 32 odd, last stage) is read clamped and cleared at store time.
template <int TT, int ES>
struct XLanes {
  static constexpr int kChunks = TT * kKS / 8 / 256;
  u32 off[kChunks];
  __device__ __forceinline__ void init(int K, int N, int tok0, int tid) {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int idx = tid + c * 256;
      const int row = min(tok0 + (idx >> 3), N - 1) - tok0;
      off[c] = (static_cast<u32>(row) * static_cast<u32>(K) + 8u * (idx & 7)) * ES;
    }
  }
  // gathered rows: token row i of the super-tile is activation row rows[i] (rows
  // past nvalid repeat the last valid one); offsets from the activations' start
  __device__ __forceinline__ void init_rows(int K, const int* rows, int nvalid, int tid) {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int idx = tid + c * 256;
      const int row = rows[min(idx >> 3, nvalid - 1)];
      off[c] = (static_cast<u32>(row) * static_cast<u32>(K) + 8u * (idx & 7)) * ES;
    }
  }
  // byte offset of chunk c for stage base k0, with the K clamp of a tail stage
  __device__ __forceinline__ u32 at(int c, int K, int k0, int tid, bool tail) const {
    if (!tail) return off[c];
    const int kk = k0 + 8 * ((tid + c * 256) & 7);
    return off[c] - static_cast<u32>(max(kk - (K - 8), 0)) * ES;
  }
};

template <int TT> struct XStage<TT, true> {
  static constexpr int kChunks = TT * kKS / 8 / 256;
  half8 v[kChunks];
  __device__ __forceinline__ void load(const u8* xb, const XLanes<TT, 2>& xl, int K, int k0, int tid, bool tail) {
    const u8* base = xb + static_cast<u64>(k0) * 2;
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
      v[c] = *reinterpret_cast<const half8*>(base + static_cast<u64>(xl.at(c, K, k0, tid, tail)));
  }
  __device__ __forceinline__ void store(_Float16* sx, int tid) const {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int idx = tid + c * 256;
      *reinterpret_cast<half8*>(&sx[x_slot(idx >> 3, idx & 7)]) = v[c];
    }
  }
};

template <int TT> struct XStage<TT, false> {
  static constexpr int kChunks = TT * kKS / 8 / 256;
  float4 v[kChunks][2];
  __device__ __forceinline__ void load(const u8* xb, const XLanes<TT, 4>& xl, int K, int k0, int tid, bool tail) {
    const u8* base = xb + static_cast<u64>(k0) * 4;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const float4* p = reinterpret_cast<const float4*>(base + static_cast<u64>(xl.at(c, K, k0, tid, tail)));
      v[c][0] = p[0];
      v[c][1] = p[1];
    }
  }
  __device__ __forceinline__ void store(_Float16* sx, int tid) const {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int idx = tid + c * 256;
      const float4 f0 = v[c][0], f1 = v[c][1];
      *reinterpret_cast<half8*>(&sx[x_slot(idx >> 3, idx & 7)]) =
          half8{static_cast<_Float16>(f0.x), static_cast<_Float16>(f0.y), static_cast<_Float16>(f0.z),
                static_cast<_Float16>(f0.w), static_cast<_Float16>(f1.x), static_cast<_Float16>(f1.y),
                static_cast<_Float16>(f1.z), static_cast<_Float16>(f1.w)};
    }
  }
};

// Clears the K positions [k_end, 64) of a stage buffer (a stage reaching past K).
template <int TT>
__device__ __forceinline__ void clear_k_tail(_Float16* sx, int tid, int k_end) {
  constexpr int kChunks = TT * kKS / 8 / 256;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int idx = tid + c * 256;
    if (8 * (idx & 7) >= k_end) *reinterpret_cast<half8*>(&sx[x_slot(idx >> 3, idx & 7)]) = half8{0, 0, 0, 0, 0, 0, 0, 0};
  }
}

// The stage's products: B operands of token block t from LDS (lane: token
// 16t + l % 16, k-chunks 2g and 2g+1 at offsets o0 and o1 of the block's first
// row), each used by the wave's RB row blocks, for the NA token blocks the
// super-tile computes (all NTB, or fewer in a last super-tile filled to whole
// T-token tiles).
template <int RB, int NTB, int NA>
__device__ __forceinline__ void stage_products(const _Float16* sx, int o0, int o1, const half8 (&A)[RB][2],
                                               floatx4 (&acc)[RB][NTB]) {
  static_assert(NA <= NTB, "active blocks");
#pragma unroll
  for (int t = 0; t < NA; ++t) {
    {
      const half8 B0 = *reinterpret_cast<const half8*>(sx + 16 * t * kKS + o0);
      const half8 B1 = *reinterpret_cast<const half8*>(sx + 16 * t * kKS + o1);
#pragma unroll
      for (int b = 0; b < RB; ++b)
        acc[b][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[b][0], B0, acc[b][t], 0, 0, 0);
#pragma unroll
      for (int b = 0; b < RB; ++b)
        acc[b][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[b][1], B1, acc[b][t], 0, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Workgroup barrier for the stage hand-over: the wave's own LDS writes are
// complete (lgkmcnt 0) before it arrives, so every wave sees the stage's
// activations after it; global loads in flight (the prefetch of the next two
// stages) are not waited for, unlike a full __syncthreads() fence.  The memory
// clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// sched_barrier mask: every instruction class but global memory may be moved
// across (ALU, VALU, SALU, MFMA, LDS, transcendental)
constexpr int kNoVmemCross = 0x0001 | 0x0002 | 0x0004 | 0x0008 | 0x0080 | 0x0100 | 0x0200 | 0x0400;

// Approximate VALU instructions of one row block's A-operand decode per stage.
template <int F> constexpr int kDecodeValu =
    F == FMT_Q6_K || F == FMT_Q3_K || F == FMT_Q5_K ? 90
    : (F == FMT_Q4_K || F == FMT_Q5_0 || F == FMT_Q5_1 || F == FMT_Q2_K ? 64 : 48);

// Instruction order asked of the scheduler for a steady full stage: the first
// two token blocks' B operands read from LDS up front, then each MFMA followed
// by its share of the next stage's decode and by the LDS read of a later
// block's B operand, so the matrix core, the VALU and LDS latency overlap within
// one wave instead of running as three serial phases.
template <int F, int RB, int NTB>
__device__ __forceinline__ void interleave_stage() {
  constexpr int kMfma = 2 * RB * NTB;
  constexpr int kValu = (kDecodeValu<F> * RB + kMfma - 1) / kMfma;
  constexpr int kAheadReads = 4 < 2 * NTB ? 4 : 2 * NTB;
  __builtin_amdgcn_sched_group_barrier(0x100, kAheadReads, 0);
#pragma unroll
  for (int i = 0; i < kMfma; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
    if (i % RB == RB - 1 && i / RB < 2 * NTB - kAheadReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// One workgroup's K loop for token blocks [0, NA).  The
// products of stage s run while the wave decodes the A operands of stage s+1,
// so the matrix cores and the VALU work side by side within one wave.  Weight
// bytes are fetched three stages ahead of their products (two ahead of their
// decode) and activations two ahead: stage s refills the weight set it just
// decoded with stage s+3, fetches the activations of stage s+2 into registers,
// and writes those of stage s+1 (fetched during stage s-1) into the other LDS
// buffer.  Stages are taken two at a time so the register sets swap roles
// without copies.
template <int F, int RB, int TT, bool XF16, int NA>
__device__ __forceinline__ void k_loop(const GemmArgs& a, _Float16 (&sX)[2][TT * kKS], floatx4 (&acc)[RB][TT / 16],
                                       const u32 (&row_off)[RB], const XLanes<TT, XF16 ? 2 : 4>& xl, const u8* xb,
                                       int o0, int o1, int tid, int g, int sb, int nstages) {
  // stages sb .. sb + nstages - 1 of K; s below counts from 0 within them
  AStage<F> w0[RB], w1[RB];
  XStage<TT, XF16> x0, x1;
  half8 A0[RB][2], A1[RB][2];

  // a stage past K (K / 32 odd, last stage) has its activations read clamped and
  // cleared, and its second unit's weights zeroed; LAST: s may be such a stage
  auto tail = [&](int s) { return kKS * (sb + s) + kKS > a.K; };
  auto fetch_w = [&](int s, AStage<F>(&w)[RB]) {
#pragma unroll
    for (int b = 0; b < RB; ++b) w[b].load(a.W, row_off[b], 2 * (sb + s), a.nU, g);
  };
  auto fetch_x = [&](int s, XStage<TT, XF16>& xs, bool last) {
    xs.load(xb, xl, a.K, kKS * (sb + s), tid, last && tail(s));
  };
  auto put = [&](int s, const XStage<TT, XF16>& xs, bool last) {
    xs.store(sX[s & 1], tid);
    if (last && tail(s)) clear_k_tail<TT>(sX[s & 1], tid, a.K - kKS * (sb + s));
  };
  auto decode = [&](int s, AStage<F>(&w)[RB], half8(&A)[RB][2], bool last) {
    if (last && 2 * (sb + s) + 1 == a.nU) {
#pragma unroll
      for (int b = 0; b < RB; ++b) w[b].zero_second(g);
    }
#pragma unroll
    for (int b = 0; b < RB; ++b) w[b].operands(g, A[b]);
  };
  // stage s: Ac = its A operands, wn = weight set of stage s+1 (decoded into An,
  // then refilled with s+3), xs = activation set refilled with s+2, xo = stage
  // s+1.  In the steady state (STEADY) stages s+1 .. s+3 exist and none is the
  // last, so the step is one branch-free block the scheduler can interleave.
  auto step = [&](auto steady, int s, AStage<F>(&wn)[RB], half8(&Ac)[RB][2], half8(&An)[RB][2],
                  XStage<TT, XF16>& xs, const XStage<TT, XF16>& xo) {
    constexpr bool STEADY = decltype(steady)::value;
    const bool next = STEADY || s + 1 < nstages;
    const bool fetch2 = STEADY || s + 2 < nstages;
    const bool fetch3 = STEADY || s + 3 < nstages;
    if (next) decode(s + 1, wn, An, !STEADY);
    // activations before weights: the load counter retires in order, so the wait
    // for these activations (next step, before they are written to LDS) must not
    // also wait for the weight bytes of stage s+3, which have two more steps
    if (fetch2) fetch_x(s + 2, xs, !STEADY);
    __builtin_amdgcn_sched_barrier(kNoVmemCross);
    if (fetch3) fetch_w(s + 3, wn);
    stage_products<RB, TT / 16, NA>(sX[s & 1], o0, o1, Ac, acc);
    if (next) put(s + 1, xo, !STEADY);
    if constexpr (STEADY) interleave_stage<F, RB, NA>();
    if (next) stage_barrier();
    // keep the next step's decode below this point: hoisted above the barrier it
    // waits for the weight loads this step just issued (the load counter retires
    // in order), which serialises the stage behind a full memory latency
    __builtin_amdgcn_sched_barrier(0);
  };
  using steady_t = std::integral_constant<bool, true>;
  using edge_t = std::integral_constant<bool, false>;

  fetch_w(0, w0);
  if (nstages > 1) fetch_w(1, w1);
  fetch_x(0, x0, true);
  if (nstages > 1) fetch_x(1, x1, true);
  put(0, x0, true);
  decode(0, w0, A0, true);
  if (nstages > 2) fetch_w(2, w0);
  stage_barrier();

  int s = 0;
  for (; s + 4 < nstages; s += 2) {
    step(steady_t{}, s, w1, A0, A1, x0, x1);
    step(steady_t{}, s + 1, w0, A1, A0, x1, x0);
  }
  // at most four stages left, starting with an even one
  while (s < nstages) {
    step(edge_t{}, s, w1, A0, A1, x0, x1);
    if (++s >= nstages) break;
    step(edge_t{}, s, w0, A1, A0, x1, x0);
    ++s;
  }
}

// The K loop for ntb active token blocks (an even count, 2 .. NTB), each count its own
// instance, so a partly filled last super-tile runs the same scheduled steady state
// over fewer blocks and never costs more than a full one.
template <int F, int RB, int TT, bool XF16, int NA = TT / 16>
__device__ __forceinline__ void k_loop_ntb(int ntb, const GemmArgs& a, _Float16 (&sX)[2][TT * kKS],
                                           floatx4 (&acc)[RB][TT / 16], const u32 (&row_off)[RB],
                                           const XLanes<TT, XF16 ? 2 : 4>& xl, const u8* xb, int o0, int o1, int tid,
                                           int g, int sb, int nstages) {
  if constexpr (NA <= 2) {
    k_loop<F, RB, TT, XF16, 2>(a, sX, acc, row_off, xl, xb, o0, o1, tid, g, sb, nstages);
  } else {
    if (ntb >= NA)
      k_loop<F, RB, TT, XF16, NA>(a, sX, acc, row_off, xl, xb, o0, o1, tid, g, sb, nstages);
    else
      k_loop_ntb<F, RB, TT, XF16, NA - 2>(ntb, a, sX, acc, row_off, xl, xb, o0, o1, tid, g, sb, nstages);
  }
}

// (the 256-token super-tile takes one workgroup per CU: its accumulators need
// the register file's accumulation half)
template <int F, int RB, int TT, bool XF16>
__global__ __launch_bounds__(256, TT >= 256 ? 1 : 2) void k_gemm(GemmArgs a) {
  constexpr int NTB = TT / 16;  // 16-token blocks of the super-tile
  __shared__ __attribute__((aligned(16))) _Float16 sX[2][TT * kKS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int row_tile = blockIdx.x % a.n_row_tiles;
  const int tok0 = (blockIdx.x / a.n_row_tiles) * TT;
  const int rw0 = row_tile * (64 * RB) + (tid >> 6) * (16 * RB);  // this wave's first row

  // 16-token blocks computed: whole T-token tiles up to N (at most the super-tile)
  const int rem = a.N - tok0;
  const int ntb = rem >= TT ? NTB : ((rem + a.T - 1) / a.T) * (a.T / 16);

  u32 row_off[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int r = rw0 + 16 * b + (lane & 15);
    row_off[b] = static_cast<u32>(r < a.M ? r : a.M - 1) * a.row_bytes;
  }
  // B-operand offsets of this lane within a token block: token row l % 16,
  // k-chunks 2g (step 0) and 2g + 1 (step 1)
  const int o0 = x_slot(lane & 15, 2 * g);
  const int o1 = x_slot(lane & 15, 2 * g + 1);

  floatx4 acc[RB][NTB];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int t = 0; t < NTB; ++t) acc[b][t] = floatx4{0.f, 0.f, 0.f, 0.f};

  // split blockIdx.y takes K stages [sb, sb + ns) and writes its partial products
  // to its own [N, M] slab of the workspace (y itself when unsplit)
  const int all = (a.nU + 1) >> 1;
  const int sb = blockIdx.y * a.split_stages;
  const int ns = min(a.split_stages, all - sb);
  float* const yo = a.y + blockIdx.y * a.split_floats;
  constexpr int ES = XF16 ? 2 : 4;
  XLanes<TT, ES> xl;
  xl.init(a.K, a.N, tok0, tid);
  const u8* xb = reinterpret_cast<const u8*>(a.x) + static_cast<u64>(tok0) * static_cast<u64>(a.K) * ES;
  k_loop_ntb<F, RB, TT, XF16>(ntb, a, sX, acc, row_off, xl, xb, o0, o1, tid, g, sb, ns);

  // D[4*(l/16) + v][l % 16] of block (b, t): row rw0 + 16b + 4g + v, token tok0 + 16t + l % 16
#pragma unroll
  for (int t = 0; t < NTB; ++t) {
    const int tok = tok0 + 16 * t + (lane & 15);
    if (t < ntb && tok < a.N) {
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const int r = rw0 + 16 * b + 4 * g;
        float* yp = yo + (u64)tok * a.M + r;
        if (a.y_vec && r + 3 < a.M) {
          *reinterpret_cast<float4*>(yp) = make_float4(acc[b][t][0], acc[b][t][1], acc[b][t][2], acc[b][t][3]);
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (r + v < a.M) yp[v] = acc[b][t][v];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Expert-indexed matrix-matrix path (any number of tokens).  Grid = (64*RB-row
// tiles) x (rank of the expert among the call's distinct valid ids).  A
// workgroup finds its expert as the expert-indexed matrix-vector path does (id
// bitmap in LDS, single-wave prefix scan), counts the (token, slot) pairs routed
// to it in ascending pair order (each thread counts a contiguous segment of the
// ids, then one exclusive scan), and runs the matrix-core loop over that
// expert's rows for each super-tile of its pairs: the pairs' activation rows are
// gathered into the staged tile, and output row p (the pair index) receives
// the results.  The pairs are padded to the token tile per expert (the tile
// rule applied to the expert's own pair count under QMM_TILE_AUTO).  Every
// output is accumulated as in the dense path, so each output row is, bit for
// bit, qmm_gemm of its expert on its activation row.
constexpr int kMmIdBitmapWords = static_cast<int>(kMaxExperts / 32);

struct MmIdShared {
  u32 bits[kMmIdBitmapWords];
  int base[256];       // exclusive prefix of the threads' segment counts
  int pair[128];       // pair index of each token of the current super-tile
  int xrow[128];       // its activation row
  int expert, count, bad;
};

__device__ __forceinline__ int tile_for_count(int n) {
  const int p64 = (n + 63) / 64 * 64 - n, p32 = (n + 31) / 32 * 32 - n;
  return p64 <= p32 ? 64 : 32;
}

template <int F, int RB, int TT, bool XF16>
__global__ __launch_bounds__(256, 2) void k_gemm_id(GemmArgs a) {
  constexpr int NTB = TT / 16;
  __shared__ __attribute__((aligned(16))) _Float16 sX[2][TT * kKS];
  __shared__ MmIdShared sh;

  // workgroup i runs on XCD i mod 8: the row-tile groups of one expert rank get
  // ids that are equal mod 8, so they share that XCD's L2 for the expert's
  // activation rows (read once per row tile)
  const int wid = blockIdx.x;
  const int xcd = wid & 7, q = wid >> 3;
  const int grp = q % a.id_groups;
  const int rank = (q / a.id_groups) * 8 + xcd;
  if (rank >= a.id_ranks) return;  // padding of the rank count (uniform)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int P = a.N * a.S;
  const int nwords = (a.E + 31) >> 5;

  // presence bitmap of the valid ids
  for (int w = tid; w < nwords; w += 256) sh.bits[w] = 0u;
  if (tid == 0) { sh.expert = -1; sh.bad = 0; }
  __syncthreads();
  for (int p = tid; p < P; p += 256) {
    const int e = a.ids[p];
    if (e >= 0 && e < a.E)
      atomicOr(&sh.bits[e >> 5], 1u << (e & 31));
    else
      sh.bad = 1;
  }
  __syncthreads();
  // the rank-th set bit (first wave)
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
    const int k = rank;
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
  // the workgroup takes row tiles grp, grp + id_groups, ... of its expert,
  // routing once for all of them
  const int n_tiles = (a.M + 64 * RB - 1) / (64 * RB);
  // ids outside [0, E): NaN rows, written by the rank-0 workgroups (which cover
  // every row tile)
  if (rank == 0 && sh.bad) {
    const float qnan = __builtin_nanf("");
    for (int rt = grp; rt < n_tiles; rt += a.id_groups) {
      const int r_lo = rt * 64 * RB;
      const int nr = min(a.M, r_lo + 64 * RB) - r_lo;
      for (int i = tid; i < P * nr; i += 256) {
        const int p = i / nr, r = r_lo + (i - p * nr);
        const int id = a.ids[p];
        if (id < 0 || id >= a.E) a.y[(u64)p * a.M + r] = qnan;
      }
    }
  }
  if (e < 0) return;  // uniform over the workgroup

  // pairs routed to e, in ascending order: thread segments (a multiple of 4 ids,
  // read 16 bytes at a time when the ids are 16-byte aligned), then an
  // exclusive scan
  const int L = ((P + 255) / 256 + 3) & ~3;
  const int s0 = min(P, tid * L), s1 = min(P, s0 + L);
  const bool vec = (reinterpret_cast<uintptr_t>(a.ids) & 15) == 0;
  // 16-byte output stores: rows r .. r+3 of a pair's output row (M % 4 == 0, y
  // 16-byte aligned)
  const bool y_vec = (a.M % 4 == 0) && (reinterpret_cast<uintptr_t>(a.y) & 15) == 0;
  auto visit = [&](auto fn) {
    int p = s0;
    if (vec) {
      // 16 ids per round, their four loads issued before any is examined
      for (; p + 16 <= s1; p += 16) {
        int4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = *reinterpret_cast<const int4*>(a.ids + p + 4 * j);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          fn(p + 4 * j, v[j].x); fn(p + 4 * j + 1, v[j].y); fn(p + 4 * j + 2, v[j].z); fn(p + 4 * j + 3, v[j].w);
        }
      }
      for (; p + 4 <= s1; p += 4) {
        const int4 v = *reinterpret_cast<const int4*>(a.ids + p);
        fn(p, v.x); fn(p + 1, v.y); fn(p + 2, v.z); fn(p + 3, v.w);
      }
    }
    for (; p < s1; ++p) fn(p, a.ids[p]);
  };
  // the pairs of super-tile tok0 (positions tok0 .. tok0 + TT - 1 of the
  // ascending list) into sh.pair / sh.xrow
  auto gather = [&](int tok0) {
    int pos = sh.base[tid];
    visit([&](int p, int id) {
      if (id == e) {
        if (pos >= tok0 && pos < tok0 + TT) {
          sh.pair[pos - tok0] = p;
          sh.xrow[pos - tok0] = a.x_per_slot ? p : p / a.S;
        }
        ++pos;
      }
    });
    __syncthreads();
  };
  int mine = 0;
  visit([&](int, int id) { mine += id == e; });
  {
    int incl = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    if (lane == 63) sh.base[tid >> 6] = incl;  // wave totals
    __syncthreads();
    int before = 0;
    for (int w = 0; w < (tid >> 6); ++w) before += sh.base[w];
    const int total = sh.base[0] + sh.base[1] + sh.base[2] + sh.base[3];
    __syncthreads();
    sh.base[tid] = before + incl - mine;
    if (tid == 0) sh.count = total;
    __syncthreads();
  }
  const int count = sh.count;
  const int T = a.T ? a.T : tile_for_count(count);

  GemmArgs ae = a;
  ae.W = a.W + static_cast<u64>(e) * a.expert_bytes;
  const int o0 = x_slot(lane & 15, 2 * g);
  const int o1 = x_slot(lane & 15, 2 * g + 1);
  const int all = (a.nU + 1) >> 1;
  constexpr int ES = XF16 ? 2 : 4;

  // one super-tile of pairs: gathered once for all the row tiles
  const bool one_tile = count <= TT;
  if (one_tile) gather(0);
  for (int rt = grp; rt < n_tiles; rt += a.id_groups) {
  const int r_lo = rt * 64 * RB;
  const int rw0 = r_lo + (tid >> 6) * (16 * RB);  // this wave's first row
  u32 row_off[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int r = rw0 + 16 * b + (lane & 15);
    row_off[b] = static_cast<u32>(r < a.M ? r : a.M - 1) * a.row_bytes;
  }
  for (int tok0 = 0; tok0 < count; tok0 += TT) {
    // this super-tile's pairs and activation rows
    if (!one_tile) gather(tok0);
    const int rem = count - tok0;
    const int ntb = rem >= TT ? NTB : ((rem + T - 1) / T) * (T / 16);
    XLanes<TT, ES> xl;
    xl.init_rows(a.K, sh.xrow, min(rem, TT), tid);
    floatx4 acc[RB][NTB];
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int t = 0; t < NTB; ++t) acc[b][t] = floatx4{0.f, 0.f, 0.f, 0.f};
    const u8* xb = reinterpret_cast<const u8*>(a.x);
    k_loop_ntb<F, RB, TT, XF16>(ntb, ae, sX, acc, row_off, xl, xb, o0, o1, tid, g, 0, all);
#pragma unroll
    for (int t = 0; t < NTB; ++t) {
      const int i = 16 * t + (lane & 15);
      if (t < ntb && i < rem) {
        const int p = sh.pair[i];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const int r = rw0 + 16 * b + 4 * g;
          float* yp = a.y + (u64)p * a.M + r;
          if (y_vec && r + 3 < a.M) {
            *reinterpret_cast<float4*>(yp) = make_float4(acc[b][t][0], acc[b][t][1], acc[b][t][2], acc[b][t][3]);
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (r + v < a.M) yp[v] = acc[b][t][v];
          }
        }
      }
    }
    __syncthreads();  // sX (and pair, xrow) are refilled for the next super-tile
  }
  }
}

// ---------------------------------------------------------------------------------------------
// Few tokens (1 .. 16) with the K split inside a workgroup (the split entry points,
// qmm_gemm_ws and qmm_gemm_noalloc).  The same fp16 operands as k_gemm -- the A
// operands of AStage (the exact fp32 weight rounded to fp16), the activations as fp16
// (fp32 input rounded to nearest even) in the same chunk order -- but no LDS staging:
// a wave owns 16 rows (A rows) against one 16-token block (B columns; lanes of tokens
// past N load nothing and multiply zeros) and a run of SPW consecutive K stages,
// its loads kept D stages ahead of its products in registers.  At a few tokens a weight
// meets at most 16 tokens, so fetching each weight's bytes and decoding it into an fp16
// operand -- which k_gemm spreads over 64 or more tokens -- set the time, not the
// products.  KS waves cover K; their partial outputs are summed in LDS in wave order, so
// an output depends on the call's shape and activation type (which fix SPW and KS) and
// not on N or the token tile: both tiles give the same bits.
// Activations of a stage through buffer loads: a lane of a token past N, or of a chunk
// past K, gets an offset past the buffer's end, which the hardware answers with zeros
// without touching memory -- no branch, so the loads of every stage are counted alike
// and each product waits for its own stage only.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t sk_rsrc(const void* p, u32 bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), 0x00020000);
}
template <bool XF16, int NTB> struct SkX;
template <int NTB> struct SkX<true, NTB> {
  uint4 v[NTB][2];
  __device__ __forceinline__ void load(int b, int j, __amdgpu_buffer_rsrc_t rs, u32 off) {
    v[b][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  }
  __device__ __forceinline__ half8 op(int b, int j) const { return __builtin_bit_cast(half8, v[b][j]); }
};
template <int NTB> struct SkX<false, NTB> {
  uint4 v[NTB][2][2];
  __device__ __forceinline__ void load(int b, int j, __amdgpu_buffer_rsrc_t rs, u32 off) {
    v[b][j][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    v[b][j][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u, 0, 0));
  }
  __device__ __forceinline__ half8 op(int b, int j) const {
    const float4 f0 = __builtin_bit_cast(float4, v[b][j][0]), f1 = __builtin_bit_cast(float4, v[b][j][1]);
    return half8{static_cast<_Float16>(f0.x), static_cast<_Float16>(f0.y), static_cast<_Float16>(f0.z),
                 static_cast<_Float16>(f0.w), static_cast<_Float16>(f1.x), static_cast<_Float16>(f1.y),
                 static_cast<_Float16>(f1.z), static_cast<_Float16>(f1.w)};
  }
};

// Stages in flight per wave, and waves per workgroup: 16 waves (four per SIMD, 128
// registers per lane) where the loads of four (fp16 activations) or three (fp32) stages
// fit beside the rest; 8 waves (256 registers) for the formats with the widest decode
// state and for fp32 activations of two token blocks, which spill at 128.
constexpr bool sk_wide(int F, bool xf16, int ntb) {
  return F == FMT_Q6_K || F == FMT_Q3_K || F == FMT_Q5_0 || F == FMT_Q5_K || (!xf16 && ntb == 2);
}
constexpr int sk_depth(bool xf16, int ntb) { return xf16 ? (ntb == 1 ? 4 : 3) : (ntb == 1 ? 3 : 2); }
constexpr int sk_max_waves(int F, bool xf16, int ntb) { return sk_wide(F, xf16, ntb) ? 8 : 16; }

// split_stages = SPW (stages per wave), a multiple of the depth; blockDim = 64 * KS
template <int F, bool XF16, int NTB>
__global__ __launch_bounds__(64 * sk_max_waves(F, XF16, NTB)) void k_gemm_sk(GemmArgs a) {
  constexpr int D = sk_depth(XF16, NTB);
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int KS = blockDim.x >> 6;
  const int r0 = static_cast<int>(blockIdx.x) * 16;
  const int nst = (a.nU + 1) >> 1;
  const int sb = w * a.split_stages;
  const int r = min(r0 + (lane & 15), a.M - 1);  // rows past M repeat the last one (never stored)
  const u32 row_off = static_cast<u32>(r) * a.row_bytes;

  AStage<F> ws[D];
  SkX<XF16, NTB> xs[D];
  constexpr u32 ES = XF16 ? 2 : 4;
  const u32 xbytes = static_cast<u32>(a.N) * static_cast<u32>(a.K) * ES;
  const __amdgpu_buffer_rsrc_t rs = sk_rsrc(a.x, xbytes);
  // stage s into slot d: the weights of the wave's 16 rows (clamped to the last stage,
  // so every address is inside the matrix) and each token block's two k-chunks 2g, 2g + 1
  // (zeros for tokens past N and for K past the end)
  auto fetch = [&](int s, int d) {
    const int sc = min(s, nst - 1);
    ws[d].load(a.W, row_off, 2 * sc, a.nU, g);
#pragma unroll
    for (int b = 0; b < NTB; ++b) {
      const int tok = 16 * b + (lane & 15);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int k = kKS * sc + 8 * (2 * g + j);
        const bool in = tok < a.N && k < a.K && s < nst;
        const u32 off = in ? (static_cast<u32>(tok) * static_cast<u32>(a.K) + k) * ES : xbytes;
        xs[d].load(b, j, rs, off);
      }
    }
  };
  // one accumulator per slot: a stage's products depend on the slot's previous stage
  // only (D stages back), never on a result of the stage before it
  floatx4 acc[D][NTB];
#pragma unroll
  for (int d = 0; d < D; ++d)
#pragma unroll
    for (int b = 0; b < NTB; ++b) acc[d][b] = floatx4{0.f, 0.f, 0.f, 0.f};
  // a stage past K (the last wave's run may end past it) multiplies zero weights by
  // zero activations; a last stage whose second unit lies past K has that unit's
  // weights zeroed (zero_second zeroes the coefficients of lane groups >= 2)
  auto compute = [&](int s, int d) {
    const int zg = s >= nst ? 2 : (2 * s + 1 == a.nU ? g : 0);
    ws[d].zero_second(zg);
    half8 A[2];
    ws[d].operands(g, A);
#pragma unroll
    for (int b = 0; b < NTB; ++b) {
      acc[d][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[0], xs[d].op(b, 0), acc[d][b], 0, 0, 0);
      acc[d][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[1], xs[d].op(b, 1), acc[d][b], 0, 0, 0);
    }
  };
  // SPW / D turns of the ring, the last one peeled (it fetches nothing): no branch
  // around a load, so before each product the wait is for that stage's loads only.
  // The last wave's stages past K re-read the last stage (clamped) and are dropped.
#pragma unroll
  for (int d = 0; d < D; ++d) fetch(sb + d, d);
  // (scheduling barriers keep each stage's decode behind its own wait: the scheduler
  // would otherwise hoist the next stages' decode, and with it their waits, forward;
  // the matrix cores still run a stage's products while the next one decodes)
  int s = sb;
  for (int turn = D; turn < a.split_stages; turn += D, s += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      compute(s + d, d);
      __builtin_amdgcn_sched_barrier(0);
      fetch(s + d + D, d);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d) {
    compute(s + d, d);
    __builtin_amdgcn_sched_barrier(0);
  }

  // D[4g + i][l % 16] of token block b: row r0 + 4g + i, token 16b + l % 16; the
  // slots' sums added in slot order
  extern __shared__ float s_sk[];
#pragma unroll
  for (int b = 0; b < NTB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = acc[0][b][i];
#pragma unroll
      for (int d = 1; d < D; ++d) v += acc[d][b][i];
      s_sk[((w * NTB + b) * 4 + i) * 64 + lane] = v;
    }
  __syncthreads();
  constexpr int kOut = NTB * 256;
  for (int o = threadIdx.x; o < kOut; o += blockDim.x) {
    // o = (block b, token t, row rr): consecutive threads store consecutive rows
    const int b = o >> 8, t = (o >> 4) & 15, rr = o & 15;
    const int src = (b * 4 + (rr & 3)) * 64 + 16 * (rr >> 2) + t;
    float sum = s_sk[src];
    for (int ww = 1; ww < KS; ++ww) sum += s_sk[ww * kOut + src];
    const int tok = 16 * b + t, row = r0 + rr;
    if (tok < a.N && row < a.M) a.y[static_cast<u64>(tok) * a.M + row] = sum;
  }
}

// y = sum of the S partial slabs of a split call, in split order (so the result
// does not depend on which workgroup finished first).
__global__ __launch_bounds__(256) void k_split_sum(const float* ws, int S, u64 stride, u64 count, int vec,
                                                   float* y) {
  const u64 i0 = static_cast<u64>(blockIdx.x) * blockDim.x + threadIdx.x;
  const u64 step = static_cast<u64>(gridDim.x) * blockDim.x;
  if (vec) {
    for (u64 i = i0; 4 * i < count; i += step) {
      float4 v = reinterpret_cast<const float4*>(ws)[i];
      for (int s = 1; s < S; ++s) {
        const float4 w = reinterpret_cast<const float4*>(ws + s * stride)[i];
        v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
      }
      reinterpret_cast<float4*>(y)[i] = v;
    }
  } else {
    for (u64 i = i0; i < count; i += step) {
      float v = ws[i];
      for (int s = 1; s < S; ++s) v += ws[s * stride + i];
      y[i] = v;
    }
  }
}

namespace {
typedef void (*GemmKernel)(GemmArgs);

// Workgroup shapes (RB, TT): 128 rows x 128 tokens, 64 x 128, 64 x 64 and 64 x 32.
// The first two amortise each decoded weight over 128 tokens; 64 x 64 gives small
// problems more workgroups; 64 x 32 serves K-split calls padded to 32 tokens.  Q6_K's raw bytes and fp32 activations (held twice
// as wide while in flight) leave no room for the 128 x 128 shape within 256
// registers per lane.  Q6_K, whose decode costs the most per weight, also has
// 64 x 256 and 128 x 256 with fp16 activations, one workgroup per CU.
constexpr bool shape_ok(int F, bool xf16, int RB, int TT) {
  if (TT == 256) return F == FMT_Q6_K && xf16 && (RB == 1 || RB == 2);
  // (Q3_K, Q5_0 and Q5_K x 128 rows spill: their decode state is wider)
  if (RB == 2) return TT == 128 && F != FMT_Q6_K && F != FMT_Q3_K && F != FMT_Q5_0 && F != FMT_Q5_K && xf16;
  return TT == 32 || TT == 64 || TT == 128;
}

template <int F, bool XF16, int RB, int TT>
GemmKernel kernel_if_ok() {
  if constexpr (shape_ok(F, XF16, RB, TT)) return k_gemm<F, RB, TT, XF16>;
  return nullptr;
}

template <int F>
GemmKernel pick(int RB, int TT, bool xf16) {
  if (xf16 && TT == 256) return RB == 2 ? kernel_if_ok<F, true, 2, 256>() : kernel_if_ok<F, true, 1, 256>();
  if (xf16)
    return RB == 2 ? kernel_if_ok<F, true, 2, 128>()
         : TT == 128 ? kernel_if_ok<F, true, 1, 128>()
         : TT == 64 ? kernel_if_ok<F, true, 1, 64>() : kernel_if_ok<F, true, 1, 32>();
  return RB == 2 ? kernel_if_ok<F, false, 2, 128>()
       : TT == 128 ? kernel_if_ok<F, false, 1, 128>()
       : TT == 64 ? kernel_if_ok<F, false, 1, 64>() : kernel_if_ok<F, false, 1, 32>();
}

// 128-row workgroups at the 64-token super-tile (twice the weight bytes in
// flight per workgroup; Q6_K's decode would not fit the registers), 64 rows at
// the 128-token one
template <int F, int TT>
constexpr int id_rows_blocks() { return TT == 64 && F != FMT_Q6_K && F != FMT_Q3_K && F != FMT_Q5_0 ? 2 : 1; }

// the formats whose expert-indexed kernel takes the 64-token super-tile only (their
// decode state spills the registers at 128 tokens)
constexpr bool id_narrow_tile(int F) { return F == FMT_Q6_K || F == FMT_Q3_K; }

template <int F, int TT>
GemmKernel pick_id(bool xf16) {
  constexpr int RB = id_rows_blocks<F, TT>();
  if (xf16) return k_gemm_id<F, RB, TT, true>;
  return k_gemm_id<F, RB, TT, false>;
}

// Workgroups of 256 threads (one wave per SIMD each) of kernel k that one CU
// holds at once: 512 registers per SIMD lane over the kernel's register count,
// and 160 KB of LDS over its LDS size; 2 when the attributes are unavailable,
// at most 3.  Memoised per (format, super-tile, activation type).
int id_resident_per_cu(int fmt, int TT, bool xf16, GemmKernel k) {
  static std::atomic<int> memo[kNumFormats][2][2];
  std::atomic<int>& slot = memo[fmt][TT == 128 ? 1 : 0][xf16 ? 1 : 0];
  int n = slot.load(std::memory_order_relaxed);
  if (n > 0) return n;
  hipFuncAttributes at{};
  n = 2;
  if (hipFuncGetAttributes(&at, reinterpret_cast<const void*>(k)) == hipSuccess && at.numRegs > 0) {
    const int by_regs = 512 / ((at.numRegs + 7) / 8 * 8);
    const int by_lds = at.sharedSizeBytes > 0 ? static_cast<int>(163840 / at.sharedSizeBytes) : by_regs;
    n = std::min(by_regs, by_lds);
    n = std::max(2, std::min(3, n));
  } else {
    (void)hipGetLastError();
  }
  slot.store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace

// K splits for N tokens: few tokens leave too few (row, token) tiles to fill the
// chip, so the K stages are divided among that many more workgroups, at least
// two stages each (above 64 tokens, the plan above).  A function of the shape and N only (not of the tile), so both
// tiles split alike and stay bit-identical.
namespace {

// Calls of more than 64 tokens: the split count (1 .. 3, at least 8 stages per
// split) and workgroup shape (64 rows x 128 or 64 tokens; for Q6_K with fp16
// activations also 64 or 128 rows x 256 tokens) that minimise a cost fitted to
// the decode-layer shapes at 130 .. 2048 tokens.  A workgroup runs about as fast
// alone on a CU as beside a second one, so a launch takes ceil(workgroups / CUs)
// rounds of (stages per split) x (time of one stage of that shape); a split adds
// a fixed 4 us plus the partial outputs written and summed at ~4 TB/s.  Stage
// times (us): 0.55 (64 x 128) and 0.38 (64 x 64) for the formats decoded in one
// multiply-add per weight; 0.73, 0.58, 1.15 (64 x 256) and 2.15 (128 x 256) for
// Q6_K.  The plan does not depend on the token tile (more than 64 tokens pad to
// more than 64 under both tiles), so both tiles split alike.
struct WidePlan {
  int splits, stages, RB, TT;
};

WidePlan wide_plan(const MatDesc& m, int64_t N, bool xf16) {
  const int64_t cus = m.cus;
  const int nst = static_cast<int>((m.K / 32 + 1) / 2);
  const bool q6 = m.fmt == FMT_Q6_K;
  WidePlan best{1, nst, 1, 64};
  double best_cost = 1e300;
  static const int kWide[4][2] = {{1, 128}, {1, 64}, {1, 256}, {2, 256}};
  for (const auto& c : kWide) {
    const int rb = c[0], tt = c[1];
    if (!shape_ok(m.fmt, xf16, rb, tt)) continue;
    const double stage_us = q6 ? (tt == 256 ? (rb == 2 ? 2.15 : 1.15) : (tt == 128 ? 0.73 : 0.58))
                               : (tt == 128 ? 0.55 : 0.38);
    const int64_t wgs = ((m.M + 64 * rb - 1) / (64 * rb)) * ((N + tt - 1) / tt);
    for (int S = 1; S <= 3; ++S) {
      const int per = (nst + S - 1) / S;
      if (S > 1 && per < 8) break;
      const int splits = (nst + per - 1) / per;
      const int64_t rounds = (wgs * splits + cus - 1) / cus;
      double cost = static_cast<double>(rounds) * per * stage_us;
      if (splits > 1) cost += 4.0 + static_cast<double>(N) * static_cast<double>(m.M) * 4.0 * (splits + 1) / 4e6;
      if (cost < best_cost) {
        best_cost = cost;
        best = WidePlan{splits, per, rb, tt};
      }
    }
  }
  return best;
}

}  // namespace

namespace {
GemmSplit split_for(const MatDesc& m, int64_t N, bool xf16) {
  const int64_t cus = m.cus;
  GemmSplit sp{1, static_cast<int>((m.K / 32 + 1) / 2)};
  if (N >= 1 && N <= kSkMaxTokens) return sp;  // k_gemm_sk: the split is inside the workgroup
  if (N > 64) {
    const WidePlan p = wide_plan(m, N, xf16);
    return GemmSplit{p.splits, p.stages};
  }
  // up to 64 tokens: split when the (64-row, 64-token) tiles number fewer than
  // one per CU (one per two CUs for Q6_K), into about that many workgroups (a
  // sweep of 1..16 splits on the decode-layer shapes at 7, 33 and 64 tokens
  // came within 2% of its best per projection with this count)
  const int64_t base = ((m.M + 63) / 64) * ((N + 63) / 64);
  const int64_t want = m.fmt == FMT_Q6_K ? cus / 2 : cus;
  if (N <= 0 || base >= want) return sp;
  const int64_t nst = sp.stages;
  int64_t S = (want + base - 1) / base;
  if (S > nst / 2) S = nst / 2;
  if (S < 2) return sp;
  const int64_t per = (nst + S - 1) / S;
  sp.stages = static_cast<int>(per);
  sp.splits = static_cast<int>((nst + per - 1) / per);
  return sp;
}
}  // namespace

// The split of a call with either activation type that needs the larger
// workspace (the workspace query does not know the type).
GemmSplit gemm_split(const MatDesc& m, int64_t N) {
  const GemmSplit a = split_for(m, N, false), b = split_for(m, N, true);
  return b.splits > a.splits ? b : a;
}

size_t gemm_workspace_bytes(const MatDesc& m, int64_t N) {
  const GemmSplit sp = gemm_split(m, N);
  return sp.splits > 1 ? static_cast<size_t>(sp.splits) * N * m.M * sizeof(float) : 0;
}

hipError_t launch_gemm_id(const MatDesc& m, const void* x, int x_f16, int64_t N, int64_t S, int x_per_slot,
                          const int32_t* ids, float* y, int tile, hipStream_t st) {
  const int64_t cus = m.cus;
  GemmArgs a{};
  a.W = m.blocks;
  a.row_bytes = static_cast<u32>(m.row_bytes);
  a.M = static_cast<int>(m.M);
  a.nU = static_cast<int>(m.K / 32);
  a.K = static_cast<int>(m.K);
  a.x = x;
  a.N = static_cast<int>(N);
  a.y = y;
  a.T = tile;  // 0: the tile rule on each expert's pair count
  a.ids = ids;
  a.S = static_cast<int>(S);
  a.x_per_slot = x_per_slot;
  a.E = static_cast<int>(m.n_experts);
  a.expert_bytes = m.row_bytes * static_cast<u64>(m.M);
  const int64_t P = N * S;
  const int64_t ranks = P < m.n_experts ? P : m.n_experts;
  // 64 rows x 64 tokens; 128 tokens when an expert averages 48 pairs or more,
  // so that the busier experts still take one super-tile (their weights decoded
  // once, their pairs gathered once): 128 experts at 1024 tokens, 64 pairs each
  // on average, run in 210 us at 128 against 322 at 64
  const bool xf16 = x_f16 != 0;
  const int TT = P >= 48 * m.n_experts && !id_narrow_tile(m.fmt) ? 128 : 64;  // (Q6_K, Q3_K x 128 spill)
  GemmKernel k = nullptr;
  switch (m.fmt) {
    case FMT_Q4_0: k = TT == 128 ? pick_id<FMT_Q4_0, 128>(xf16) : pick_id<FMT_Q4_0, 64>(xf16); break;
    case FMT_Q8_0: k = TT == 128 ? pick_id<FMT_Q8_0, 128>(xf16) : pick_id<FMT_Q8_0, 64>(xf16); break;
    case FMT_Q4_K: k = TT == 128 ? pick_id<FMT_Q4_K, 128>(xf16) : pick_id<FMT_Q4_K, 64>(xf16); break;
    case FMT_Q6_K: k = pick_id<FMT_Q6_K, 64>(xf16); break;
    case FMT_A4G64: k = TT == 128 ? pick_id<FMT_A4G64, 128>(xf16) : pick_id<FMT_A4G64, 64>(xf16); break;
    case FMT_Q4_1: k = TT == 128 ? pick_id<FMT_Q4_1, 128>(xf16) : pick_id<FMT_Q4_1, 64>(xf16); break;
    case FMT_Q5_0: k = TT == 128 ? pick_id<FMT_Q5_0, 128>(xf16) : pick_id<FMT_Q5_0, 64>(xf16); break;
    case FMT_Q5_1: k = TT == 128 ? pick_id<FMT_Q5_1, 128>(xf16) : pick_id<FMT_Q5_1, 64>(xf16); break;
    case FMT_Q2_K: k = TT == 128 ? pick_id<FMT_Q2_K, 128>(xf16) : pick_id<FMT_Q2_K, 64>(xf16); break;
    case FMT_Q3_K: k = pick_id<FMT_Q3_K, 64>(xf16); break;
    case FMT_Q5_K: k = TT == 128 ? pick_id<FMT_Q5_K, 128>(xf16) : pick_id<FMT_Q5_K, 64>(xf16); break;
    default: return hipErrorInvalidValue;
  }
  if (!k) return hipErrorInvalidValue;
  const int RB = TT == 64 && m.fmt != FMT_Q6_K && m.fmt != FMT_Q3_K && m.fmt != FMT_Q5_0 ? 2 : 1;  // as id_rows_blocks
  // as many workgroups over the ranks as the CUs hold at once (from the
  // kernel's registers and LDS: two for each of these kernels), each taking
  // every groups-th row tile of its expert (the routing is done once per
  // workgroup); a second round of workgroups measured slower than fewer,
  // longer ones
  const int64_t row_tiles = (m.M + 64 * RB - 1) / (64 * RB);
  if (ranks > 65535 || row_tiles > INT_MAX) return hipErrorInvalidValue;
  const int64_t per_cu = id_resident_per_cu(m.fmt, TT, xf16, k);
  int64_t groups = (per_cu * cus + ranks - 1) / ranks;
  if (groups > row_tiles) groups = row_tiles;
  const int64_t ranks8 = (ranks + 7) / 8 * 8;
  a.id_groups = static_cast<int>(groups);
  a.id_ranks = static_cast<int>(ranks);
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(groups * ranks8)), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Scratch of the allocation-free matrix-matrix entry point (qmm_gemm_noalloc): the K-split
// partial products of qmm_gemm_ws live in this file-scope device array instead of a
// caller's workspace.  Every GPU the library runs on holds its own copy until the process
// ends.  Host code never names the array in a launch or a copy: its device address is
// looked up once per device (hipGetSymbolAddress, with that device current) and kept.
constexpr size_t kScratchBytes = QMM_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};
}  // namespace

size_t gemm_scratch_bytes() { return kScratchBytes; }

hipError_t gemm_scratch_init(int dev) {
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev]) return hipSuccess;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!p) return hipErrorInvalidSymbol;
  g_scratch_ptr[dev] = p;
  return hipSuccess;
}

float* gemm_scratch(int dev) {
  if (dev < 0 || dev >= kScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return static_cast<float*>(g_scratch_ptr[dev]);
}

namespace {
template <int F>
void sk_kernels(GemmKernel (&t)[2]) {
  t[0] = k_gemm_sk<F, false, 1>;
  t[1] = k_gemm_sk<F, true, 1>;
}
struct SkTable {
  GemmKernel k[kNumFormats][2];  // [format][fp16 activations]
  SkTable() {
    sk_kernels<FMT_Q4_0>(k[FMT_Q4_0]);
    sk_kernels<FMT_Q8_0>(k[FMT_Q8_0]);
    sk_kernels<FMT_Q4_K>(k[FMT_Q4_K]);
    sk_kernels<FMT_Q6_K>(k[FMT_Q6_K]);
    sk_kernels<FMT_A4G64>(k[FMT_A4G64]);
    sk_kernels<FMT_Q4_1>(k[FMT_Q4_1]);
    sk_kernels<FMT_Q5_0>(k[FMT_Q5_0]);
    sk_kernels<FMT_Q5_1>(k[FMT_Q5_1]);
    sk_kernels<FMT_Q2_K>(k[FMT_Q2_K]);
    sk_kernels<FMT_Q3_K>(k[FMT_Q3_K]);
    sk_kernels<FMT_Q5_K>(k[FMT_Q5_K]);
  }
};

// k_gemm_sk's shape: KS waves per workgroup, each with SPW stages (a multiple of the
// depth) -- a function of the format, M, K, the activation type and the token blocks,
// never of the tile.
hipError_t launch_gemm_sk(const MatDesc& m, const void* x, bool xf16, int64_t N, float* y, hipStream_t st) {
  static const SkTable tab;
  const int ntb = 1;
  const int D = sk_depth(xf16, ntb);
  const int64_t nst = (m.K / 32 + 1) / 2;
  const int cap = sk_max_waves(m.fmt, xf16, ntb);
  // waves per workgroup: about 16 per CU over the launch's row tiles (so every
  // workgroup is resident at once and each wave streams its run through the ring),
  // within the kernel's cap
  const int64_t tiles = (m.M + 15) / 16;
  int64_t want = (16 * static_cast<int64_t>(m.cus) + tiles - 1) / tiles;
  want = want < 1 ? 1 : (want > cap ? cap : want);
  const int64_t per = (nst + want - 1) / want;
  const int64_t spw = (per + D - 1) / D * D;
  const int64_t KS = (nst + spw - 1) / spw;
  GemmArgs a{};
  a.W = m.blocks;
  a.row_bytes = static_cast<u32>(m.row_bytes);
  a.M = static_cast<int>(m.M);
  a.nU = static_cast<int>(m.K / 32);
  a.K = static_cast<int>(m.K);
  a.x = x;
  a.N = static_cast<int>(N);
  a.y = y;
  a.split_stages = static_cast<int>(spw);
  const int64_t blocks = (m.M + 15) / 16;
  if (blocks > INT_MAX || spw > INT_MAX) return hipErrorInvalidValue;
  const size_t lds = static_cast<size_t>(KS) * ntb * 256 * sizeof(float);
  hipLaunchKernelGGL(tab.k[m.fmt][xf16 ? 1 : 0], dim3(static_cast<unsigned>(blocks)),
                     dim3(static_cast<unsigned>(64 * KS)), lds, st, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm(const MatDesc& m, const void* x, int x_f16, int64_t N, float* y, int tile, float* ws,
                       bool split_ok, hipStream_t st) {
  const int64_t cus = m.cus;
  if (split_ok && N >= 1 && N <= kSkMaxTokens) return launch_gemm_sk(m, x, x_f16 != 0, N, y, st);
  const GemmSplit sp = split_ok ? split_for(m, N, x_f16 != 0) : GemmSplit{1, static_cast<int>((m.K / 32 + 1) / 2)};
  GemmArgs a{};
  a.W = m.blocks;
  a.row_bytes = static_cast<u32>(m.row_bytes);
  a.M = static_cast<int>(m.M);
  a.nU = static_cast<int>(m.K / 32);
  a.K = static_cast<int>(m.K);
  a.x = x;
  a.N = static_cast<int>(N);
  a.y = y;
  a.y_vec = (m.M % 4 == 0) && ((reinterpret_cast<uintptr_t>(y) & 15) == 0);
  a.T = tile;
  a.split_stages = sp.stages;
  a.split_floats = sp.splits > 1 ? static_cast<u64>(N) * static_cast<u64>(m.M) : 0;
  if (sp.splits > 1) a.y = ws;
  // Rows x tokens per workgroup: the first shape, in order of decreasing reuse,
  // that gives two workgroups per CU (one per two CUs for Q6_K, whose wider
  // decode favours reuse over parallelism: ffn_down at 512 tokens takes 122 us
  // at 64 x 128 on 160 workgroups against 189 at 64 x 64 on 320), else 64 x 64.
  // Measured on the decode-layer shapes.
  const int64_t padded = (N + tile - 1) / tile * tile;
  auto wgs = [&](int rb, int tt) { return ((m.M + 64 * rb - 1) / (64 * rb)) * ((padded + tt - 1) / tt); };
  static const int kShapes[3][2] = {{2, 128}, {1, 128}, {1, 64}};
  const int64_t want = m.fmt == FMT_Q6_K ? cus / 2 : 2 * cus;
  const bool xf16 = x_f16 != 0;
  // split calls take 64 rows x the planned super-tile above 64 tokens, else x 64,
  // or x 32 when the call pads to 32: activations of absent tokens are not
  // staged then
  int RB = 1, TT = sp.splits > 1 && padded <= 32 ? 32 : 64;
  if (N > 64 && ws) {
    // the planned shape, split or not, when it is one of the 256-token ones
    const WidePlan p = wide_plan(m, N, xf16);
    if (sp.splits > 1 || p.TT == 256) {
      RB = p.RB;
      TT = p.TT;
    }
  }
  for (const auto& c : kShapes) {
    if (sp.splits > 1 || TT == 256) break;
    if (!shape_ok(m.fmt, xf16, c[0], c[1])) continue;
    if (c[1] > 64 && padded <= c[1] / 2) continue;  // a super-tile at most half used
    if (wgs(c[0], c[1]) >= want) {
      RB = c[0];
      TT = c[1];
      break;
    }
  }
  GemmKernel k = nullptr;
  switch (m.fmt) {
    case FMT_Q4_0: k = pick<FMT_Q4_0>(RB, TT, xf16); break;
    case FMT_Q8_0: k = pick<FMT_Q8_0>(RB, TT, xf16); break;
    case FMT_Q4_K: k = pick<FMT_Q4_K>(RB, TT, xf16); break;
    case FMT_Q6_K: k = pick<FMT_Q6_K>(RB, TT, xf16); break;
    case FMT_A4G64: k = pick<FMT_A4G64>(RB, TT, xf16); break;
    case FMT_Q4_1: k = pick<FMT_Q4_1>(RB, TT, xf16); break;
    case FMT_Q5_0: k = pick<FMT_Q5_0>(RB, TT, xf16); break;
    case FMT_Q5_1: k = pick<FMT_Q5_1>(RB, TT, xf16); break;
    case FMT_Q2_K: k = pick<FMT_Q2_K>(RB, TT, xf16); break;
    case FMT_Q3_K: k = pick<FMT_Q3_K>(RB, TT, xf16); break;
    case FMT_Q5_K: k = pick<FMT_Q5_K>(RB, TT, xf16); break;
    default: return hipErrorInvalidValue;
  }
  if (!k) return hipErrorInvalidValue;
  a.n_row_tiles = static_cast<int>((m.M + 64 * RB - 1) / (64 * RB));
  const int64_t blocks = static_cast<int64_t>(a.n_row_tiles) * ((N + TT - 1) / TT);
  if (blocks > INT_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(blocks), sp.splits), dim3(256), 0, st, a);
  if (sp.splits > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const u64 count = static_cast<u64>(N) * static_cast<u64>(m.M);
    const int vec = (count % 4 == 0) && ((reinterpret_cast<uintptr_t>(y) & 15) == 0) ? 1 : 0;
    const u64 items = vec ? count / 4 : count;
    const unsigned grid = static_cast<unsigned>(std::min<u64>((items + 255) / 256, 2048));
    hipLaunchKernelGGL(k_split_sum, dim3(grid), dim3(256), 0, st, ws, sp.splits, a.split_floats, count, vec, y);
  }
  return hipGetLastError();
}

}  // namespace qmm
