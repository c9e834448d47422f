// decode.hpp -- per-format block decoders for gfx950 (device code).
//
// Every kernel of the library works on "units": 32 consecutive weights of one
// row (K positions 32u .. 32u+31).  A unit is one Q4_0 or Q8_0 block, half an
// A4G64 group, one 32-weight sub-block of a Q4_K super-block, or two 16-weight
// sub-blocks of a Q6_K super-block.  Decoding a unit is three steps:
//
//   1. load   -- fetch the unit's bytes (scale fields and code bytes) from the
//                block stream into registers.  Blocks of 18, 34 and 210 bytes
//                are only 2-byte aligned, so those loaders read the enclosing
//                aligned dwords and realign them with v_alignbit; they never
//                read a dword past the one holding the unit's last byte.
//   2. codes  -- the unit's 32 codes as four 32-bit words of 8 codes in bytes
//                (byte b of word j is the code of weight 4j+b of the unit...
//                see each format), each code already a non-negative integer.
//   3. value  -- w = fma(code, a, b) in fp32.  For every format the two
//                coefficients a and b are exact in fp32 and the product
//                code*a is exact, so the single rounding of the fma gives the
//                fp32 round-to-nearest-even of the formula's exact value.
//
// Formulas (the block formats the candle pull request "Metal: 64-token tile
// for the quantized matrix-matrix kernel" lists in section "What changes",
// plus the 4-bit affine groups of the tiny-llm pull request "perf: Optimize
// quantized matmul for small decode batches"):
//   Q4_0   w = d*(q-8)         -> fma(q, d, -8d)
//   Q8_0   w = d*q, q signed   -> fma(q, d, 0) (code stored as q+128, bias removed exactly)
//   Q4_K   w = d*sc*q - dmin*m -> fma(q, d*sc, -(dmin*m))
//   Q6_K   w = d*sc*(q-32)     -> fma(q, d*sc, -32*d*sc)
//   A4G64  w = scale*q + bias  -> fma(q, scale, bias)
// and the other types that section lists, whose formulas are read from their
// names (a scale times a zero-centred code for an "_0" type, a scale and a
// minimum for an "_1" type, per-sub-block scales and minimums in a K-quant):
//   Q4_1, Q5_1  w = d*q + m    -> fma(q, d, m)
//   Q5_0   w = d*(q-16)        -> fma(q, d, -16d)
//   Q2_K   w = d*sc*q - dmin*m -> fma(q, d*sc, -(dmin*m))   (16-weight sub-blocks)
//   Q3_K   w = d*(s-32)*(q-4)  -> fma(q, d*(s-32), -4*d*(s-32))
//   Q5_K   w = d*sc*q - dmin*m -> fma(q, d*sc, -(dmin*m))   (a fifth code bit)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

using u8 = uint8_t;
using u16 = uint16_t;
using u32 = uint32_t;
using u64 = uint64_t;

enum : int {
  FMT_Q4_0 = 0, FMT_Q8_0 = 1, FMT_Q4_K = 2, FMT_Q6_K = 3, FMT_A4G64 = 4,
  FMT_Q4_1 = 5, FMT_Q5_0 = 6, FMT_Q5_1 = 7, FMT_Q2_K = 8, FMT_Q3_K = 9, FMT_Q5_K = 10,
  kNumFormats = 11
};

template <int F> struct FmtInfo;
template <> struct FmtInfo<FMT_Q4_0> { static constexpr int BW = 32, BB = 18; };
template <> struct FmtInfo<FMT_Q8_0> { static constexpr int BW = 32, BB = 34; };
template <> struct FmtInfo<FMT_Q4_K> { static constexpr int BW = 256, BB = 144; };
template <> struct FmtInfo<FMT_Q6_K> { static constexpr int BW = 256, BB = 210; };
template <> struct FmtInfo<FMT_A4G64> { static constexpr int BW = 64, BB = 36; };
template <> struct FmtInfo<FMT_Q4_1> { static constexpr int BW = 32, BB = 20; };
template <> struct FmtInfo<FMT_Q5_0> { static constexpr int BW = 32, BB = 22; };
template <> struct FmtInfo<FMT_Q5_1> { static constexpr int BW = 32, BB = 24; };
template <> struct FmtInfo<FMT_Q2_K> { static constexpr int BW = 256, BB = 84; };
template <> struct FmtInfo<FMT_Q3_K> { static constexpr int BW = 256, BB = 110; };
template <> struct FmtInfo<FMT_Q5_K> { static constexpr int BW = 256, BB = 176; };

// fp16 bit pattern (low 16 bits) -> exact fp32 (subnormals included).
__device__ __forceinline__ float h2f(u32 bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<u16>(bits & 0xFFFFu)));
}

// Byte b of v as a float (v_cvt_f32_ubyte{b}).
__device__ __forceinline__ float byte_f(u32 v, int b) {
  return static_cast<float>((v >> (8 * b)) & 0xFFu);
}

__device__ __forceinline__ u16 load_u16(const u8* p) {
  return *reinterpret_cast<const u16*>(p);
}

// NBYTES bytes at any alignment (NBYTES a multiple of 4), kept as the enclosing
// dword-aligned words and realigned with v_alignbit only when read: load() only
// issues loads, so the realignment -- and the wait for the data -- comes where
// the words are used.  The last load is the dword holding the range's last byte
// (a repeat of the one before it when src is dword aligned), so nothing past
// that dword is read and no branch guards a load.
template <int NBYTES>
struct RawBytes {
  static_assert(NBYTES % 4 == 0, "whole words");
  static constexpr int NW = NBYTES / 4;
  u32 raw[NW + 1];
  u32 sh;
  __device__ __forceinline__ void load(const u8* src) {
    // pointer arithmetic (not integer casts) keeps the global address space
    // known, so these stay global loads rather than flat ones
    const u32 mis = static_cast<u32>(reinterpret_cast<uintptr_t>(src) & 3u);
    const u32* p = reinterpret_cast<const u32*>(src - mis);
    sh = mis * 8u;
#pragma unroll
    for (int i = 0; i < NW; ++i) raw[i] = p[i];
    raw[NW] = p[(mis + NBYTES - 1) >> 2];
  }
  // bytes src[4j .. 4j+3] as a little-endian word
  __device__ __forceinline__ u32 word(int j) const { return __builtin_amdgcn_alignbit(raw[j + 1], raw[j], sh); }
};

// A decoded unit: 32 codes in 8 words, and w_k = fma(code_k, a, b) where the
// coefficient pair may change once, at weight 16 (Q6_K's two sub-blocks).
struct Unit {
  u32 c[8];      // code of weight 4j+b of the unit = byte b of c[j]
  float a0, b0;  // coefficients for weights 0..15
  float a1, b1;  // coefficients for weights 16..31
};

// Hides a value from the optimiser (emits nothing), so that byte extraction of a
// masked word is done with v_cvt_f32_ubyte{0..3} on the word rather than
// re-deriving each byte with a bit-field extract.
__device__ __forceinline__ u32 opaque(u32 v) {
  asm("" : "+v"(v));
  return v;
}

// ---------------------------------------------------------------------------------------------
// Loaders: base = start of a matrix (or of one expert's matrix), row_off = byte
// offset of the row from base (32 bits: a matrix is below 4 GiB), u = unit index
// within the row.  Q4_K and A4G64 read whole dwords directly: their blocks are
// 144 and 36 bytes, so with a 16-byte aligned tensor every super-block (group)
// of every expert is 16 (4) byte aligned.  The other formats realign.

template <int F> struct Decoder;

// Q4_0: block u; weight i (0..15) low nibble of qs[i], weight 16+i high nibble.
template <> struct Decoder<FMT_Q4_0> {
  static constexpr float kCodeBias = 0.0f;
  struct Raw { RawBytes<16> q; u32 d; };
  __device__ __forceinline__ static void load(const u8* base, u32 row_off, int u, Raw& r) {
    const u32 bo = row_off + 18u * u;
    r.q.load(base + bo + 2);
    r.d = load_u16(base + bo);
  }
  __device__ __forceinline__ static void unpack(const Raw& r, Unit& o) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32 q = r.q.word(j);
      o.c[j] = q & 0x0F0F0F0Fu;             // weights 4j .. 4j+3
      o.c[4 + j] = (q >> 4) & 0x0F0F0F0Fu;  // weights 16+4j .. 16+4j+3
    }
    const float d = h2f(r.d);
    o.a0 = o.a1 = d;
    o.b0 = o.b1 = -8.0f * d;
  }
};

// Q8_0: block u; int8 codes, biased by 128 so they convert as unsigned bytes.
template <> struct Decoder<FMT_Q8_0> {
  static constexpr float kCodeBias = 128.0f;  // code - 128 is the signed q
  struct Raw { RawBytes<32> q; u32 d; };
  __device__ __forceinline__ static void load(const u8* base, u32 row_off, int u, Raw& r) {
    const u32 bo = row_off + 34u * u;
    r.q.load(base + bo + 2);
    r.d = load_u16(base + bo);
  }
  __device__ __forceinline__ static void unpack(const Raw& r, Unit& o) {
#pragma unroll
    for (int j = 0; j < 8; ++j) o.c[j] = r.q.word(j) ^ 0x80808080u;
    const float d = h2f(r.d);
    o.a0 = o.a1 = d;
    o.b0 = o.b1 = 0.0f;
  }
};

// Q4_K: super-block u/8, sub-block j = u%8: codes are the (j odd ? high : low)
// nibbles of qs[32*(j/2) .. +31]; sc_j and m_j are 6-bit fields of the
// 96-bit string at bits 6j and 48+6j.  Super-blocks are 144 = 9*16 bytes, so
// with a 16-byte aligned base every super-block is 16-byte aligned.
template <> struct Decoder<FMT_Q4_K> {
  static constexpr float kCodeBias = 0.0f;
  struct Raw { u32 h[4]; u32 q[8]; int j; };
  __device__ __forceinline__ static void load(const u8* base, u32 row_off, int u, Raw& r) {
    const u32 so = row_off + 144u * (u >> 3);
    r.j = u & 7;
    const u32* h = reinterpret_cast<const u32*>(base + so);
    const u32* q = reinterpret_cast<const u32*>(base + so + 16 + 32 * (r.j >> 1));
#pragma unroll
    for (int k = 0; k < 4; ++k) r.h[k] = h[k];
#pragma unroll
    for (int k = 0; k < 8; ++k) r.q[k] = q[k];
  }
  // sc_j = bits [6j, 6j+6) and m_j = bits [48+6j, 54+6j) of the 96-bit string in
  // h[1] (bits 0..31), h[2] (32..63), h[3] (64..95).  Both candidate funnel shifts
  // are computed and one is selected, so no word is picked by a runtime index
  // (which the compiler would turn into a load from private memory).
  __device__ __forceinline__ static u32 field_sc(const Raw& r) {
    const u32 b = 6u * static_cast<u32>(r.j);  // 0..42
    const u32 t0 = __builtin_amdgcn_alignbit(r.h[2], r.h[1], b & 31u);
    const u32 t1 = __builtin_amdgcn_alignbit(r.h[3], r.h[2], b & 31u);
    return (b < 32 ? t0 : t1) & 63u;
  }
  __device__ __forceinline__ static u32 field_m(const Raw& r) {
    const u32 b = 48u + 6u * static_cast<u32>(r.j);  // 48..90
    const u32 t0 = __builtin_amdgcn_alignbit(r.h[3], r.h[2], b & 31u);
    const u32 t1 = r.h[3] >> (b & 31u);
    return (b < 64 ? t0 : t1) & 63u;
  }
  __device__ __forceinline__ static void unpack(const Raw& r, Unit& o) {
    const u32 sh = 4u * static_cast<u32>(r.j & 1);
#pragma unroll
    for (int k = 0; k < 8; ++k) o.c[k] = (r.q[k] >> sh) & 0x0F0F0F0Fu;
    const float d = h2f(r.h[0]);
    const float dmin = h2f(r.h[0] >> 16);
    const float sc = static_cast<float>(field_sc(r));
    const float m = static_cast<float>(field_m(r));
    o.a0 = o.a1 = d * sc;         // exact: 11-bit significand x 6-bit integer
    o.b0 = o.b1 = -(dmin * m);    // exact
  }
};

// Q6_K: super-block u/8, a = u%8 covers weights 32a .. 32a+31 (sub-blocks 2a, 2a+1).
// Low nibbles: ql[32*(a%4) + i], high nibble when a >= 4.  Top bits: bits
// 2*(a/2) .. +1 of qh[32*(a%2) + i].
template <> struct Decoder<FMT_Q6_K> {
  static constexpr float kCodeBias = 0.0f;
  struct Raw { RawBytes<32> ql, qh; u32 d; u32 sc; int a; };
  __device__ __forceinline__ static void load(const u8* base, u32 row_off, int u, Raw& r) {
    const u32 so = row_off + 210u * (u >> 3);
    r.a = u & 7;
    r.ql.load(base + so + 18 + 32 * (r.a & 3));
    r.qh.load(base + so + 146 + 32 * (r.a & 1));
    r.d = load_u16(base + so);
    r.sc = load_u16(base + so + 2 + 2 * r.a);
  }
  __device__ __forceinline__ static void unpack(const Raw& r, Unit& o) {
    const u32 lsh = 4u * static_cast<u32>(r.a >> 2);
    const u32 hsh = 2u * static_cast<u32>(r.a >> 1);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      o.c[k] = ((r.ql.word(k) >> lsh) & 0x0F0F0F0Fu) | (((r.qh.word(k) >> hsh) & 0x03030303u) << 4);
    const float d = h2f(r.d);
    const float s0 = static_cast<float>(static_cast<int8_t>(r.sc & 0xFFu));
    const float s1 = static_cast<float>(static_cast<int8_t>((r.sc >> 8) & 0xFFu));
    o.a0 = d * s0;                // exact: 11 + 7 significant bits
    o.a1 = d * s1;
    o.b0 = -32.0f * o.a0;         // exact (power of two)
    o.b1 = -32.0f * o.a1;
  }
};

// A4G64: group u/2, half h = u%2: codes are the (h ? high : low) nibbles of qs[0..31].
// Groups are 36 bytes, so every group is 4-byte aligned.
template <> struct Decoder<FMT_A4G64> {
  static constexpr float kCodeBias = 0.0f;
  struct Raw { u32 q[8]; u32 hdr; int h; };
  __device__ __forceinline__ static void load(const u8* base, u32 row_off, int u, Raw& r) {
    const u32 go = row_off + 36u * (u >> 1);
    r.h = u & 1;
    const u32* p = reinterpret_cast<const u32*>(base + go);
    r.hdr = p[0];
#pragma unroll
    for (int k = 0; k < 8; ++k) r.q[k] = p[1 + k];
  }
  __device__ __forceinline__ static void unpack(const Raw& r, Unit& o) {
    const u32 sh = 4u * static_cast<u32>(r.h);
#pragma unroll
    for (int k = 0; k < 8; ++k) o.c[k] = (r.q[k] >> sh) & 0x0F0F0F0Fu;
    o.a0 = o.a1 = h2f(r.hdr);
    o.b0 = o.b1 = h2f(r.hdr >> 16);
  }
};

// Four bits n (0..15) spread to bit 0 of the four bytes of a word: bit k of n to byte k.
__device__ __forceinline__ u32 spread4(u32 n) { return (n * 0x00204081u) & 0x01010101u; }

// Field f of a little-endian string of 6-bit fields held in words w1 (bits 0..31), w2, w3
// (the 96-bit string of the K-quants), for f < 16, without a runtime-indexed word.
__device__ __forceinline__ u32 six_bit_field(u32 w1, u32 w2, u32 w3, u32 f) {
  const u32 b = 6u * f;  // 0..90
  const u32 t0 = __builtin_amdgcn_alignbit(w2, w1, b & 31u);
  const u32 t1 = __builtin_amdgcn_alignbit(w3, w2, b & 31u);
  const u32 t2 = w3 >> (b & 31u);
  return (b < 32 ? t0 : (b < 64 ? t1 : t2)) & 63u;
}

// Q4_1: block u: fp16 d and m, codes as Q4_0.  20-byte blocks: every block is 4-byte aligned.
template <> struct Decoder<FMT_Q4_1> {
  static constexpr float kCodeBias = 0.0f;
  struct Raw { u32 hdr; u32 q[4]; };
  __device__ __forceinline__ static void load(const u8* base, u32 row_off, int u, Raw& r) {
    const u32* p = reinterpret_cast<const u32*>(base + row_off + 20u * u);
    r.hdr = p[0];
#pragma unroll
    for (int k = 0; k < 4; ++k) r.q[k] = p[1 + k];
  }
  __device__ __forceinline__ static void unpack(const Raw& r, Unit& o) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o.c[j] = r.q[j] & 0x0F0F0F0Fu;
      o.c[4 + j] = (r.q[j] >> 4) & 0x0F0F0F0Fu;
    }
    o.a0 = o.a1 = h2f(r.hdr);
    o.b0 = o.b1 = h2f(r.hdr >> 16);
  }
};

// The 32 five-bit codes of a Q5_0/Q5_1 block: low nibbles from the 16 code bytes as
// Q4_0, bit i of the 32-bit qh word on top of code i.
__device__ __forceinline__ void five_bit_codes(u32 qh, const u32 (&q)[4], Unit& o) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o.c[j] = (q[j] & 0x0F0F0F0Fu) | (spread4((qh >> (4 * j)) & 15u) << 4);
    o.c[4 + j] = ((q[j] >> 4) & 0x0F0F0F0Fu) | (spread4((qh >> (16 + 4 * j)) & 15u) << 4);
  }
}

// Q5_0: block u: fp16 d, qh, codes; 22-byte blocks are 2-byte aligned (realigned words).
template <> struct Decoder<FMT_Q5_0> {
  static constexpr float kCodeBias = 0.0f;
  struct Raw { RawBytes<20> b; u32 d; };  // bytes [2, 22): qh, then the 16 code bytes
  __device__ __forceinline__ static void load(const u8* base, u32 row_off, int u, Raw& r) {
    const u32 bo = row_off + 22u * u;
    r.b.load(base + bo + 2);
    r.d = load_u16(base + bo);
  }
  __device__ __forceinline__ static void unpack(const Raw& r, Unit& o) {
    const u32 q[4] = {r.b.word(1), r.b.word(2), r.b.word(3), r.b.word(4)};
    five_bit_codes(r.b.word(0), q, o);
    const float d = h2f(r.d);
    o.a0 = o.a1 = d;
    o.b0 = o.b1 = -16.0f * d;  // exact
  }
};

// Q5_1: block u: fp16 d and m, qh, codes; 24-byte blocks are 8-byte aligned.
template <> struct Decoder<FMT_Q5_1> {
  static constexpr float kCodeBias = 0.0f;
  struct Raw { u32 hdr, qh; u32 q[4]; };
  __device__ __forceinline__ static void load(const u8* base, u32 row_off, int u, Raw& r) {
    const u32* p = reinterpret_cast<const u32*>(base + row_off + 24u * u);
    r.hdr = p[0];
    r.qh = p[1];
#pragma unroll
    for (int k = 0; k < 4; ++k) r.q[k] = p[2 + k];
  }
  __device__ __forceinline__ static void unpack(const Raw& r, Unit& o) {
    five_bit_codes(r.qh, r.q, o);
    o.a0 = o.a1 = h2f(r.hdr);
    o.b0 = o.b1 = h2f(r.hdr >> 16);
  }
};

// Q2_K: super-block u/8, a = u%8 covers weights 32a .. 32a+31 (16-weight sub-blocks 2a,
// 2a+1): codes are bits 2(a/2) .. +1 of qs[32(a%2) + i]; sc and m of sub-block j are the
// nibbles of sm[j].  84-byte super-blocks are 4-byte aligned.
template <> struct Decoder<FMT_Q2_K> {
  static constexpr float kCodeBias = 0.0f;
  struct Raw { u32 hdr, sm; u32 q[8]; int a; };
  __device__ __forceinline__ static void load(const u8* base, u32 row_off, int u, Raw& r) {
    const u32 so = row_off + 84u * (u >> 3);
    r.a = u & 7;
    r.hdr = *reinterpret_cast<const u32*>(base + so);
    r.sm = load_u16(base + so + 4 + 2 * r.a);
    const u32* q = reinterpret_cast<const u32*>(base + so + 20 + 32 * (r.a & 1));
#pragma unroll
    for (int k = 0; k < 8; ++k) r.q[k] = q[k];
  }
  __device__ __forceinline__ static void unpack(const Raw& r, Unit& o) {
    const u32 sh = 2u * static_cast<u32>(r.a >> 1);
#pragma unroll
    for (int k = 0; k < 8; ++k) o.c[k] = (r.q[k] >> sh) & 0x03030303u;
    const float d = h2f(r.hdr), dmin = h2f(r.hdr >> 16);
    o.a0 = d * static_cast<float>(r.sm & 15u);          // exact
    o.b0 = -(dmin * static_cast<float>((r.sm >> 4) & 15u));
    o.a1 = d * static_cast<float>((r.sm >> 8) & 15u);
    o.b1 = -(dmin * static_cast<float>((r.sm >> 12) & 15u));
  }
};

// Q3_K: super-block u/8, a = u%8 covers weights 32a .. 32a+31 (sub-blocks 2a, 2a+1): low
// bits are bits 2(a/2) .. +1 of ql[32(a%2) + i], the top bit is bit a of qh[i]; the scale
// fields s_2a, s_2a+1 are the 12 bits at bit 12a of the 96-bit string.  110-byte
// super-blocks are 2-byte aligned (realigned words).
template <> struct Decoder<FMT_Q3_K> {
  static constexpr float kCodeBias = 0.0f;
  struct Raw { RawBytes<32> ql, qh; RawBytes<4> s; u32 d; int a; };
  __device__ __forceinline__ static void load(const u8* base, u32 row_off, int u, Raw& r) {
    const u32 so = row_off + 110u * (u >> 3);
    r.a = u & 7;
    r.ql.load(base + so + 14 + 32 * (r.a & 1));
    r.qh.load(base + so + 78);
    r.s.load(base + so + 2 + ((12 * r.a) >> 3));  // within the block: ends before byte 16
    r.d = load_u16(base + so);
  }
  __device__ __forceinline__ static void unpack(const Raw& r, Unit& o) {
    const u32 sh = 2u * static_cast<u32>(r.a >> 1);
    const u32 hb = static_cast<u32>(r.a);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      o.c[k] = ((r.ql.word(k) >> sh) & 0x03030303u) | (((r.qh.word(k) >> hb) & 0x01010101u) << 2);
    const u32 f = r.s.word(0) >> ((12u * hb) & 7u);
    const float d = h2f(r.d);
    o.a0 = d * static_cast<float>(static_cast<int>(f & 63u) - 32);         // exact
    o.a1 = d * static_cast<float>(static_cast<int>((f >> 6) & 63u) - 32);
    o.b0 = -4.0f * o.a0;  // exact (power of two)
    o.b1 = -4.0f * o.a1;
  }
};

// Q5_K: super-block u/8, sub-block j = u%8: low nibbles as Q4_K, the top bit is bit j of
// qh[i].  176-byte super-blocks are 16-byte aligned.
template <> struct Decoder<FMT_Q5_K> {
  static constexpr float kCodeBias = 0.0f;
  struct Raw { u32 h[4]; u32 qh[8]; u32 q[8]; int j; };
  __device__ __forceinline__ static void load(const u8* base, u32 row_off, int u, Raw& r) {
    const u32 so = row_off + 176u * (u >> 3);
    r.j = u & 7;
    const u32* h = reinterpret_cast<const u32*>(base + so);
    const u32* qh = reinterpret_cast<const u32*>(base + so + 16);
    const u32* q = reinterpret_cast<const u32*>(base + so + 48 + 32 * (r.j >> 1));
#pragma unroll
    for (int k = 0; k < 4; ++k) r.h[k] = h[k];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      r.qh[k] = qh[k];
      r.q[k] = q[k];
    }
  }
  __device__ __forceinline__ static void unpack(const Raw& r, Unit& o) {
    const u32 sh = 4u * static_cast<u32>(r.j & 1);
    const u32 hb = static_cast<u32>(r.j);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      o.c[k] = ((r.q[k] >> sh) & 0x0F0F0F0Fu) | (((r.qh[k] >> hb) & 0x01010101u) << 4);
    const float d = h2f(r.h[0]), dmin = h2f(r.h[0] >> 16);
    const u32 sc = six_bit_field(r.h[1], r.h[2], r.h[3], hb);
    const u32 m = six_bit_field(r.h[1], r.h[2], r.h[3], 8u + hb);
    o.a0 = o.a1 = d * static_cast<float>(sc);        // exact
    o.b0 = o.b1 = -(dmin * static_cast<float>(m));   // exact
  }
};

// The 32 codes of an unpacked unit as floats, in K order (weight i sits in byte
// i%4 of word i/4), with the format's code bias removed (exact: small integers).
template <int F>
__device__ __forceinline__ void unit_codes(const Unit& o, float (&q)[32]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const u32 m = opaque(o.c[k]);
#pragma unroll
    for (int b = 0; b < 4; ++b) q[4 * k + b] = byte_f(m, b) - Decoder<F>::kCodeBias;
  }
}

// The unit's 32 dequantized weights: w = fma(q, a, b), one rounding of an exact
// product and an exact addend, i.e. the fp32 rounding of the formula's value.
template <int F>
__device__ __forceinline__ void unit_weights(const Unit& o, float (&w)[32]) {
  float q[32];
  unit_codes<F>(o, q);
#pragma unroll
  for (int i = 0; i < 32; ++i) w[i] = i < 16 ? __builtin_fmaf(q[i], o.a0, o.b0) : __builtin_fmaf(q[i], o.a1, o.b1);
}

template <int F>
__device__ __forceinline__ void decode_unit(const u8* base, u32 row_off, int u, float (&w)[32]) {
  typename Decoder<F>::Raw r;
  Decoder<F>::load(base, row_off, u, r);
  Unit o;
  Decoder<F>::unpack(r, o);
  unit_weights<F>(o, w);
}

}  // namespace qmm

namespace qmm {

// ---------------------------------------------------------------------------------------------
// Matrix-vector work items: RUNS runs of 32 weights that share their bytes, so the
// scale fields and code bytes are fetched and unpacked once for all of them.
//   Q4_0, Q8_0  one block (1 run, unit i); the types read from their names
//               likewise take one unit per item.
//   Q4_K        sub-blocks 2p, 2p+1 of a super-block (units 2i, 2i+1): the low and
//               high nibbles of the same 32 code bytes, one 16-byte header.
//   Q6_K        runs a and a+4 of a super-block (units 8s+a, 8s+a+4, a = i%4): the
//               low and high nibbles of the same 32 ql bytes and two bit pairs of
//               the same 32 qh bytes.
//   A4G64       one group (units 2i, 2i+1): both nibbles of 32 code bytes.
// A high-nibble run keeps its codes in place (16*q in each byte) and carries
// a/16 instead of a: (a/16)*(16q) is the same fp32 value as a*q (power-of-two
// scalings are exact), and so is every partial sum of such products.
template <int F> struct Item;

template <> struct Item<FMT_Q4_0> {
  static constexpr int RUNS = 1;
  using Raw = Decoder<FMT_Q4_0>::Raw;
  __device__ __forceinline__ static int unit(int i, int) { return i; }
  __device__ __forceinline__ static void load(const u8* base, u32 row_off, int i, Raw& r) {
    Decoder<FMT_Q4_0>::load(base, row_off, i, r);
  }
  __device__ __forceinline__ static void unpack(const Raw& r, Unit (&o)[1]) { Decoder<FMT_Q4_0>::unpack(r, o[0]); }
};

template <> struct Item<FMT_Q8_0> {
  static constexpr int RUNS = 1;
  using Raw = Decoder<FMT_Q8_0>::Raw;
  __device__ __forceinline__ static int unit(int i, int) { return i; }
  __device__ __forceinline__ static void load(const u8* base, u32 row_off, int i, Raw& r) {
    Decoder<FMT_Q8_0>::load(base, row_off, i, r);
  }
  __device__ __forceinline__ static void unpack(const Raw& r, Unit (&o)[1]) { Decoder<FMT_Q8_0>::unpack(r, o[0]); }
};

// One-unit items of the other types: the unit's decoder as it is.
template <int F> struct ItemOne {
  static constexpr int RUNS = 1;
  using Raw = typename Decoder<F>::Raw;
  __device__ __forceinline__ static int unit(int i, int) { return i; }
  __device__ __forceinline__ static void load(const u8* base, u32 row_off, int i, Raw& r) {
    Decoder<F>::load(base, row_off, i, r);
  }
  __device__ __forceinline__ static void unpack(const Raw& r, Unit (&o)[1]) { Decoder<F>::unpack(r, o[0]); }
};
template <> struct Item<FMT_Q4_1> : ItemOne<FMT_Q4_1> {};
template <> struct Item<FMT_Q5_0> : ItemOne<FMT_Q5_0> {};
template <> struct Item<FMT_Q5_1> : ItemOne<FMT_Q5_1> {};
template <> struct Item<FMT_Q2_K> : ItemOne<FMT_Q2_K> {};
template <> struct Item<FMT_Q3_K> : ItemOne<FMT_Q3_K> {};
template <> struct Item<FMT_Q5_K> : ItemOne<FMT_Q5_K> {};

template <> struct Item<FMT_Q4_K> {
  static constexpr int RUNS = 2;
  struct Raw { u32 h[4]; u32 q[8]; int p; };
  __device__ __forceinline__ static int unit(int i, int run) { return 2 * i + run; }
  __device__ __forceinline__ static void load(const u8* base, u32 row_off, int i, Raw& r) {
    const u32 so = row_off + 144u * static_cast<u32>(i >> 2);
    r.p = i & 3;
    const u32* h = reinterpret_cast<const u32*>(base + so);
    const u32* q = reinterpret_cast<const u32*>(base + so + 16 + 32 * r.p);
#pragma unroll
    for (int k = 0; k < 4; ++k) r.h[k] = h[k];
#pragma unroll
    for (int k = 0; k < 8; ++k) r.q[k] = q[k];
  }
  // 12-bit field pairs (sc_{2p}, sc_{2p+1}) at bit 12p and (m_{2p}, m_{2p+1}) at
  // bit 48+12p of the bit string h[1..3]; candidates computed, then selected (no
  // runtime-indexed word, see Decoder<FMT_Q4_K>).
  __device__ __forceinline__ static u32 sc_pair(const Raw& r) {
    const u32 b = 12u * static_cast<u32>(r.p);  // 0..36
    const u32 t0 = __builtin_amdgcn_alignbit(r.h[2], r.h[1], b & 31u);
    const u32 t1 = __builtin_amdgcn_alignbit(r.h[3], r.h[2], b & 31u);
    return (b < 32 ? t0 : t1) & 0xFFFu;
  }
  __device__ __forceinline__ static u32 m_pair(const Raw& r) {
    const u32 b = 48u + 12u * static_cast<u32>(r.p);  // 48..84
    const u32 t0 = __builtin_amdgcn_alignbit(r.h[3], r.h[2], b & 31u);
    const u32 t1 = r.h[3] >> (b & 31u);
    return (b < 64 ? t0 : t1) & 0xFFFu;
  }
  __device__ __forceinline__ static void unpack(const Raw& r, Unit (&o)[2]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      o[0].c[k] = r.q[k] & 0x0F0F0F0Fu;
      o[1].c[k] = r.q[k] & 0xF0F0F0F0u;  // 16 * code
    }
    const float d = h2f(r.h[0]);
    const float dmin = h2f(r.h[0] >> 16);
    const u32 sc = sc_pair(r);
    const u32 m = m_pair(r);
    o[0].a0 = o[0].a1 = d * static_cast<float>(sc & 63u);
    o[0].b0 = o[0].b1 = -(dmin * static_cast<float>(m & 63u));
    o[1].a0 = o[1].a1 = d * static_cast<float>(sc >> 6) * 0.0625f;
    o[1].b0 = o[1].b1 = -(dmin * static_cast<float>(m >> 6));
  }
};

template <> struct Item<FMT_Q6_K> {
  static constexpr int RUNS = 2;
  struct Raw { RawBytes<32> ql, qh; u32 d; u32 sc0, sc1; int a; };
  __device__ __forceinline__ static int unit(int i, int run) { return 8 * (i >> 2) + (i & 3) + 4 * run; }
  __device__ __forceinline__ static void load(const u8* base, u32 row_off, int i, Raw& r) {
    const u32 so = row_off + 210u * static_cast<u32>(i >> 2);
    r.a = i & 3;
    r.ql.load(base + so + 18 + 32 * r.a);
    r.qh.load(base + so + 146 + 32 * (r.a & 1));
    r.d = load_u16(base + so);
    r.sc0 = load_u16(base + so + 2 + 2 * r.a);    // sub-blocks 2a, 2a+1
    r.sc1 = load_u16(base + so + 10 + 2 * r.a);   // sub-blocks 2a+8, 2a+9
  }
  __device__ __forceinline__ static void unpack(const Raw& r, Unit (&o)[2]) {
    const u32 hs = 2u * static_cast<u32>(r.a >> 1);  // run a: bits hs, run a+4: bits hs+4
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const u32 ql = r.ql.word(k), qh = r.qh.word(k);
      o[0].c[k] = (ql & 0x0F0F0F0Fu) | (((qh >> hs) & 0x03030303u) << 4);
      o[1].c[k] = ((ql >> 4) & 0x0F0F0F0Fu) | (((qh >> (hs + 4)) & 0x03030303u) << 4);
    }
    const float d = h2f(r.d);
    const u32 sc[2] = {r.sc0, r.sc1};
#pragma unroll
    for (int run = 0; run < 2; ++run) {
      o[run].a0 = d * static_cast<float>(static_cast<int8_t>(sc[run] & 0xFFu));
      o[run].a1 = d * static_cast<float>(static_cast<int8_t>((sc[run] >> 8) & 0xFFu));
      o[run].b0 = -32.0f * o[run].a0;
      o[run].b1 = -32.0f * o[run].a1;
    }
  }
};

template <> struct Item<FMT_A4G64> {
  static constexpr int RUNS = 2;
  struct Raw { u32 q[8]; u32 hdr; };
  __device__ __forceinline__ static int unit(int i, int run) { return 2 * i + run; }
  __device__ __forceinline__ static void load(const u8* base, u32 row_off, int i, Raw& r) {
    const u32* p = reinterpret_cast<const u32*>(base + row_off + 36u * static_cast<u32>(i));
    r.hdr = p[0];
#pragma unroll
    for (int k = 0; k < 8; ++k) r.q[k] = p[1 + k];
  }
  __device__ __forceinline__ static void unpack(const Raw& r, Unit (&o)[2]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      o[0].c[k] = r.q[k] & 0x0F0F0F0Fu;
      o[1].c[k] = r.q[k] & 0xF0F0F0F0u;  // 16 * code
    }
    const float scale = h2f(r.hdr), bias = h2f(r.hdr >> 16);
    o[0].a0 = o[0].a1 = scale;
    o[1].a0 = o[1].a1 = scale * 0.0625f;
    o[0].b0 = o[0].b1 = o[1].b0 = o[1].b1 = bias;
  }
};

}  // namespace qmm
