/*
 * qmm.h -- fused dequantize-and-multiply of block-quantized weights on MI355X (gfx950).
 *
 * y = x . W^T, where W (M rows x K) is stored as packed quantized blocks that the
 * kernels decode themselves, x holds N activation tokens of K values, and y is
 * N x M fp32.  This is the operation all three source pages optimise:
 *   - candle pull request "Metal: 64-token tile for the quantized matrix-matrix
 *     kernel" (sections "What changes" and "Why the tile sets the weight reuse"):
 *     the matrix-matrix path over 32- or 64-token tiles, and the one-token
 *     matrix-vector path;
 *   - llama.cpp pull request "metal : fix idle threads in mul_mv_iq3_xxs for
 *     ne00 < 1024" (sections "Overview" and "Additional information"): the
 *     matrix-vector path at narrow K and its expert-indexed (MUL_MAT_ID) form;
 *   - tiny-llm pull request "perf: Optimize quantized matmul for small decode
 *     batches" (section "Summary"): the matrix-vector path at 1..16 tokens.
 *
 * Conventions for every call
 * --------------------------
 *  - Pointers named "device" must point to device memory of the current HIP
 *    device; the library never dereferences them on the host.
 *  - The library never allocates or frees device memory and never synchronises.
 *    Every call that launches work is asynchronous on the given stream; a device
 *    fault surfaces at the caller's next synchronisation.
 *  - Argument checks happen before any launch.  On error nothing is launched,
 *    the call returns a negative qmm_status, and qmm_last_error() holds a
 *    thread-local description.  No C++ exception crosses this interface.
 *  - Buffers passed in (blocks, x, ids) are borrowed: they must stay alive and
 *    unmodified until the stream has passed the launched work.  y must not
 *    alias x, ids or the blocks.
 *  - A handle is immutable after qmm_create, so concurrent calls with one handle
 *    on different streams are safe.
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t; NULL is the default stream. */
typedef struct ihipStream_t *qmm_stream_t;

/*
 * Block formats (byte layouts are this library's; the pages print none).
 * fp16 fields are little-endian IEEE binary16.  Row r of a matrix starts at byte
 * r * qmm_row_bytes(type, K); expert e of a stacked tensor at e * M * row_bytes.
 *
 *  QMM_Q4_0   32 weights / 18 B: [0,2) d | [2,18) qs[16]; weight i = low nibble of
 *             qs[i], weight i+16 = high nibble.  w = d * (q - 8).
 *  QMM_Q8_0   32 weights / 34 B: [0,2) d | [2,34) int8 q[32].  w = d * q.
 *  QMM_Q4_K   256 weights / 144 B: [0,2) d | [2,4) dmin | [4,16) 96-bit little-endian
 *             string of sixteen 6-bit fields (field f at bit 6f: sc_0..sc_7, then
 *             m_0..m_7) | [16,144) qs[128]: weight 64p+i = low nibble of qs[32p+i],
 *             weight 64p+32+i = high nibble (p = 0..3, i = 0..31).
 *             w = d * sc_j * q - dmin * m_j with j = weight / 32.
 *  QMM_Q6_K   256 weights / 210 B: [0,2) d | [2,18) int8 sc[16] | [18,146) ql[128]:
 *             weight i (< 128) low nibble of ql[i], weight i+128 high nibble |
 *             [146,210) qh[64]: bits 2b..2b+1 of qh[i] are the top two bits of
 *             weight i+64b.  q = low4 | high2 << 4.  w = d * sc_j * (q - 32), j = weight / 16.
 *  QMM_A4G64  64 weights / 36 B: [0,2) scale | [2,4) bias | [4,36) qs[32]; weight i =
 *             low nibble of qs[i], weight i+32 = high nibble.  w = scale * q + bias.
 *
 * The other types the candle pull request lists (section "What changes"); the
 * pages give no formula for them, so they are read from their names ("_0": a
 * scale times a zero-centred code, "_1": a scale and a minimum, K-quants:
 * 256-weight super-blocks with per-sub-block scales and minimums):
 *  QMM_Q4_1   32 weights / 20 B: [0,2) d | [2,4) m | [4,20) qs[16] as Q4_0.  w = d * q + m.
 *  QMM_Q5_0   32 weights / 22 B: [0,2) d | [2,6) qh, 32-bit little-endian, bit i the top
 *             (fifth) bit of weight i | [6,22) qs[16], low nibbles as Q4_0.  w = d * (q - 16).
 *  QMM_Q5_1   32 weights / 24 B: [0,2) d | [2,4) m | [4,8) qh | [8,24) qs[16] as Q5_0.
 *             w = d * q + m.
 *  QMM_Q2_K   256 weights / 84 B: [0,2) d | [2,4) dmin | [4,20) sm[16]: sc_j low nibble,
 *             m_j high nibble of sm[j] | [20,84) qs[64]: weight i is bits 2(i/64)..+1 of
 *             qs[i % 64].  w = d * sc_j * q - dmin * m_j with j = weight / 16.
 *  QMM_Q3_K   256 weights / 110 B: [0,2) d | [2,14) 96-bit string of sixteen 6-bit s_j |
 *             [14,78) ql[64]: low two bits of weight i are bits 2(i/64)..+1 of ql[i % 64] |
 *             [78,110) qh[32]: top bit of weight i is bit i/32 of qh[i % 32].
 *             w = d * (s_j - 32) * (q - 4) with j = weight / 16.
 *  QMM_Q5_K   256 weights / 176 B: [0,2) d | [2,4) dmin | [4,16) sc/m string as Q4_K |
 *             [16,48) qh[32]: top bit of weight i is bit i/32 of qh[i % 32] | [48,176)
 *             qs[128], low nibbles as Q4_K.  w = d * sc_j * q - dmin * m_j, j = weight / 32.
 *
 * Every product in these formulas is exact in fp32, so the dequantized weight is
 * the fp32 round-to-nearest-even of the formula's exact value.
 */
typedef enum {
  QMM_Q4_0 = 0,
  QMM_Q8_0 = 1,
  QMM_Q4_K = 2,
  QMM_Q6_K = 3,
  QMM_A4G64 = 4,
  QMM_Q4_1 = 5,
  QMM_Q5_0 = 6,
  QMM_Q5_1 = 7,
  QMM_Q2_K = 8,
  QMM_Q3_K = 9,
  QMM_Q5_K = 10
} qmm_type;

/* Element type of activations (x) and of qmm_dequantize's output. */
typedef enum { QMM_F32 = 0, QMM_F16 = 1 } qmm_dtype;

/* Token tile of the matrix-matrix path (candle pull request, sections "What
 * changes" and "Where the 64-token tile is used"): AUTO applies
 * qmm_tile_for_tokens(N); 32 and 64 force a tile. */
typedef enum { QMM_TILE_AUTO = 0, QMM_TILE_32 = 32, QMM_TILE_64 = 64 } qmm_tile;

typedef int qmm_status;
#define QMM_OK 0
#define QMM_E_ARG (-1)    /* null pointer or invalid value */
#define QMM_E_TYPE (-2)   /* unknown qmm_type or qmm_dtype */
#define QMM_E_SHAPE (-3)  /* M, K, N, S or expert out of range */
#define QMM_E_ALIGN (-4)  /* a pointer is not aligned as required */
#define QMM_E_DEVICE (-5) /* no HIP device, or the current device is not gfx950 */
#define QMM_E_HIP (-6)    /* a HIP runtime error (text in qmm_last_error) */

typedef struct qmm_matrix qmm_matrix;

/*
 * qmm_create -- describe a quantized weight tensor: the block buffer, its format
 * and its shape, the operand every page's kernel reads (candle pull request,
 * section "Why the tile sets the weight reuse": a weight tile read from the
 * quantized blocks; llama.cpp pull request, section "Overview": rows of
 * 32-weight chunks; tiny-llm pull request, section "Benchmark setup": 4-bit
 * groups with a scale and a bias).  For the expert-indexed path the tensor is
 * the experts' matrices stacked (llama.cpp pull request, section "Additional
 * information": MUL_MAT_ID picks one expert's matrix per token and slot).
 *   out        receives the handle (host memory owned by the library; free it with
 *              qmm_destroy).
 *   type       block format.
 *   blocks     DEVICE pointer, 16-byte aligned, holding n_experts * M * row_bytes(K)
 *              bytes in the layout above.  Borrowed, not copied: it must outlive
 *              the handle and stay unmodified.
 *   n_experts  1 for a plain matrix; E for the stacked experts of qmm_gemm_id.
 *   M, K       rows and reduction length; K a positive multiple of the block's
 *              weight count (32 for the 32-weight types, 64 for A4G64, 256 for the
 *              K-quants); M >= 1; one matrix
 *              (M * row_bytes(K)) below 4 GiB.
 * Checks that the current device is gfx950 (QMM_E_DEVICE otherwise) and records it.
 */
qmm_status qmm_create(qmm_matrix **out, qmm_type type, const void *blocks,
                      int64_t n_experts, int64_t M, int64_t K);

/* qmm_destroy -- free a handle's host metadata (the blocks stay the caller's; see
 * qmm_create).  NULL is accepted.  Returns QMM_OK. */
qmm_status qmm_destroy(qmm_matrix *h);

/*
 * qmm_gemv -- matrix-vector path for 1..32 tokens (llama.cpp and tiny-llm pull
 * requests above): y[t, r] = sum_k x[t, k] * w[r, k], fp32 accumulation.
 *   h   a handle with n_experts == 1.
 *   x   DEVICE, [N, K] contiguous, element type xt (fp32 or fp16), 16-byte aligned.
 *   N   0..32; 0 launches nothing and returns QMM_OK; above 32 -> QMM_E_SHAPE.
 *   y   DEVICE, [N, M] contiguous fp32, 4-byte aligned; every element is written.
 * Lanes of each 64-wide wavefront are spread over (row, 32-weight chunk) pairs so
 * none idles at narrow K, and the token count picks a kernel instance that gives
 * no register to absent tokens.  fp16 calls of 5 to 32 tokens take the matrix cores
 * with exact products: there a token's outputs depend on its activations and K only
 * (the same bits at any token count from 5), and differ in summation order, not in
 * the weights, from the vector kernels, whose N-token outputs are the bits of N
 * one-token calls.
 */
qmm_status qmm_gemv(const qmm_matrix *h, const void *x, qmm_dtype xt, int64_t N,
                    float *y, qmm_stream_t stream);

/*
 * qmm_gemv_group -- qmm_gemv on `count` independent matrices in one call: the
 * matrix-vector product of the llama.cpp and tiny-llm pull requests above, for the
 * projections of one decode step that read no output of each other (a layer's
 * query, key and value projections; its gate and up projections).
 *   hs, xs, ys  HOST arrays of `count` entries: handle i (n_experts == 1), its
 *               activations ([N, K_i], element type xt, 16-byte aligned DEVICE
 *               pointer) and its output ([N, M_i] fp32, 4-byte aligned DEVICE
 *               pointer), as for qmm_gemv.  No output may overlap another output
 *               or any activation.  The arrays are read during the call only.
 *   N           0..32 tokens, the same for every matrix; 0 launches nothing.
 *   count       0..QMM_GEMV_GROUP_MAX.
 * Every output holds the bits qmm_gemv would give it.  At one token, matrices of
 * the same format and K share launches (up to four matrices per launch, one kernel
 * launch per such set); other matrices, and every matrix at N > 1, take a launch
 * of their own.  All arguments are checked before anything is launched; errors as
 * for qmm_gemv (QMM_E_ARG for a NULL array or a count out of range).
 */
#define QMM_GEMV_GROUP_MAX 64
qmm_status qmm_gemv_group(const qmm_matrix *const *hs, const void *const *xs, qmm_dtype xt,
                          int64_t N, float *const *ys, int count, qmm_stream_t stream);

/*
 * qmm_gemm -- matrix-matrix path for any N (candle pull request above).  Each
 * workgroup dequantizes a tile of weight rows once per K step into LDS as fp16
 * (round to nearest even of the fp32 weight) and multiplies it on the matrix
 * cores, with fp32 accumulation, by a tile of 32 or 64 tokens.
 *   x     DEVICE, [N, K] contiguous fp32 or fp16, 16-byte aligned; fp32 values are
 *         rounded to fp16 (nearest even) when staged.
 *   N     >= 0; a batch of sequences is passed flattened (N = batch * tokens).
 *         The handle's K must be below 2^22 (QMM_E_SHAPE otherwise).
 *   y     DEVICE, [N, M] fp32, 4-byte aligned.
 *   tile  QMM_TILE_AUTO, QMM_TILE_32 or QMM_TILE_64.  Results are bit-identical
 *         for either tile: every output is accumulated in the same order.
 */
qmm_status qmm_gemm(const qmm_matrix *h, const void *x, qmm_dtype xt, int64_t N,
                    float *y, qmm_tile tile, qmm_stream_t stream);

/*
 * qmm_gemm_workspace_bytes -- device bytes qmm_gemm_ws needs for N tokens on this
 * handle, with either activation type (the larger of the two needs); 0 when it
 * needs none: up to 16 tokens (K is divided among the waves of a workgroup), and
 * above when the call is not split (then qmm_gemm_ws computes exactly as qmm_gemm).
 * Also 0 for a NULL or expert handle and for N outside 1..2^24.
 */
size_t qmm_gemm_workspace_bytes(const qmm_matrix *h, int64_t N);

/*
 * qmm_gemm_ws -- qmm_gemm with a caller-owned workspace (same operation, tile
 * rule and arguments; candle pull request above).  Up to 16 tokens the K range is
 * divided among the waves of a workgroup of 16 weight rows, which sum their partial
 * products in LDS (no workspace).  Above, when N tokens make too few (row, token)
 * tiles to fill the GPU, or the GPU is filled better that way, the K range is divided
 * among more workgroups: each writes its partial products to its own [N, M] fp32 slab
 * of `ws`, and a second kernel sums the slabs in split order into y.  Either split
 * depends only on the handle's shape, N and the activation type, so the result is
 * deterministic and bit-identical for either tile; it can differ from qmm_gemm's in
 * rounding (both within the same error bound).  The staged operands are qmm_gemm's:
 * the fp16 weights and activations, so one-hot tokens give the staged weights.
 *   ws        DEVICE, 16-byte aligned, ws_bytes >= qmm_gemm_workspace_bytes(h, N)
 *             (QMM_E_ARG otherwise; may be NULL when that is 0).  Borrowed until
 *             the stream passes the call; must not alias x, y or the blocks.
 *             Concurrent calls need separate workspaces.
 */
qmm_status qmm_gemm_ws(const qmm_matrix *h, const void *x, qmm_dtype xt, int64_t N,
                       float *y, qmm_tile tile, void *ws, size_t ws_bytes,
                       qmm_stream_t stream);

/*
 * qmm_gemm_noalloc -- qmm_gemm_ws for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same operation, arguments, tile rule, K split and results, bit for
 * bit, as qmm_gemm_ws, with the split's partial products in a scratch array the
 * library holds in device memory (QMM_NOALLOC_SCRATCH_BYTES per GPU, reserved when the
 * library's code is loaded on that GPU and kept until the process ends).  The call
 * allocates nothing, on the device or the host.
 *   x, xt, N, y, tile  as qmm_gemm.
 * Errors: as qmm_gemm, and QMM_E_SHAPE when the call's split needs more than
 * QMM_NOALLOC_SCRATCH_BYTES, i.e. qmm_gemm_workspace_bytes(h, N) above it (nothing is
 * launched; use qmm_gemm_ws or qmm_gemm).  QMM_E_HIP if the scratch's
 * device address cannot be found.
 * Every call on one GPU shares that GPU's scratch: calls that overlap in time on one
 * GPU (different streams, or host threads) race and must be serialised by the
 * caller, e.g. by issuing them on one stream.  The scratch keeps the last call's
 * partial products; each split call overwrites every element it reads.
 */
#define QMM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
qmm_status qmm_gemm_noalloc(const qmm_matrix *h, const void *x, qmm_dtype xt, int64_t N,
                            float *y, qmm_tile tile, qmm_stream_t stream);

/*
 * qmm_gemm_id -- expert-indexed matrix-vector path (MUL_MAT_ID in the llama.cpp
 * pull request above): y[t, s, r] = sum_k x_ts[k] * w_{ids[t, s]}[r, k].
 *   h           handle with n_experts = E >= 1 (experts stacked in `blocks`).
 *   x           DEVICE, fp32 or fp16, 16-byte aligned.  x_per_slot = 1: [N, S, K],
 *               slot (t, s) reads row t*S + s.  x_per_slot = 0: [N, K], every slot
 *               of token t reads row t.
 *   N           0..32 tokens (0: no launch); S 1..64 slots per token.
 *   ids         DEVICE int32 [N, S], 4-byte aligned.  Duplicate ids are computed
 *               independently; an id outside [0, E) makes its output row all NaN.
 *   y           DEVICE fp32 [N, S, M].
 * The (token, slot) pairs are grouped by expert on the device, and each active
 * expert's rows are swept once per group of its pairs (two at a time on Q4_0 rows
 * of K = 512, more on the other paths); no host synchronisation, no device memory
 * beyond the arguments.
 */
qmm_status qmm_gemm_id(const qmm_matrix *h, const void *x, qmm_dtype xt, int64_t N,
                       int64_t S, int x_per_slot, const int32_t *ids, float *y,
                       qmm_stream_t stream);

/*
 * qmm_gemm_id_tiled -- expert-indexed matrix-matrix path for prefill-sized calls
 * (MUL_MAT_ID in the llama.cpp pull request above, on the token-tiled matrix
 * cores of the candle pull request): the same operation, arguments and NaN rule
 * as qmm_gemm_id, with qmm_gemm's arithmetic (weights staged as fp16, fp32
 * activations rounded to fp16, fp32 accumulation; bound 2e-3 * S).  Each
 * workgroup finds its expert, gathers the pairs routed to it in ascending pair
 * order, and multiplies that expert's rows by them tile by tile; each expert's
 * pairs are padded to the token tile on their own.
 *   N, S   N * S <= 2^18 (token, slot) pairs; S 1..64.  Any N >= 0.
 *   x      activation rows below 4 GiB in all.
 *   tile   QMM_TILE_AUTO (the tile rule on each expert's pair count), 32 or 64.
 *          Results are bit-identical for either tile, and every output row equals,
 *          bit for bit, qmm_gemm of its expert on its activation row.
 */
qmm_status qmm_gemm_id_tiled(const qmm_matrix *h, const void *x, qmm_dtype xt, int64_t N,
                             int64_t S, int x_per_slot, const int32_t *ids, float *y,
                             qmm_tile tile, qmm_stream_t stream);

/*
 * qmm_dequantize -- decode one expert's matrix (expert 0 for a plain matrix): the
 * per-block decode step of every path, written out.  The candle pull request
 * (section "Why the tile sets the weight reuse") decodes each weight tile once
 * into threadgroup memory before the matrix product; QMM_F16 returns exactly those
 * staged values, QMM_F32 the exact dequantized weights the matrix-vector paths
 * multiply by (llama.cpp pull request, section "Additional information", checks
 * both paths against a CPU backend working from the same weights).
 *   expert  0 .. n_experts - 1 (QMM_E_SHAPE otherwise).
 *   out     DEVICE [M, K] of type ot, 16-byte aligned, every element written.
 *           QMM_F32: the exact dequantized weights (the fp32 round-to-nearest-even
 *           of each formula above).  QMM_F16: round-to-nearest-even of those fp32
 *           values, as the matrix-matrix path stages them (an fp16 overflow gives
 *           an infinity).
 * Errors: QMM_E_ARG (NULL handle or out), QMM_E_TYPE (ot), QMM_E_ALIGN, QMM_E_DEVICE
 * (not the handle's device), QMM_E_HIP (launch).
 */
qmm_status qmm_dequantize(const qmm_matrix *h, int64_t expert, void *out, qmm_dtype ot,
                          qmm_stream_t stream);

/*
 * qmm_quantize -- encode fp32 weights into blocks of `type` on the GPU (the step
 * before the path), for Q4_0, Q8_0, Q4_K, Q6_K and A4G64 (QMM_E_TYPE for the others).  The pages quantize random weights to each type before
 * timing (candle pull request above, section "Numbers") but print no quantizer;
 * these are this library's closed forms, evaluated in fp64 on the exact fp32
 * inputs in the order written.  rne/up/down round to the nearest fp16 (ties to
 * even), the least fp16 >= the value, the greatest fp16 <= it; rha rounds half
 * away from zero:
 *   Q4_0   w* = element of largest |w| (first on a tie), d = rne(w* / -8),
 *          q = min(15, floor(w / d + 8.5)) (8 when d = 0).
 *   Q8_0   d = rne(max|w| / 127), q = clamp(rha(w / d), -127, 127) (0 when d = 0).
 *   Q4_K   per 32-weight sub-block j: lo_j = min(0, min w), hi_j = max w;
 *          dmin = up(max_j(-lo_j) / 63), m_j = clamp(ceil(-lo_j / dmin), 0, 63),
 *          span_j = hi_j + dmin * m_j, d = up(max_j(span_j / 15) / 63),
 *          sc_j = clamp(ceil(span_j / (15 d)), 0, 63),
 *          q = clamp(rha((w + dmin m_j) / (d sc_j)), 0, 15) (0 when d sc_j = 0);
 *          a zero divisor gives 0 before a ceil.
 *   Q6_K   a_j = max|w| per 16-weight sub-block, d = up(max_j a_j / 3937),
 *          sc_j = clamp(ceil(a_j / (31 d)), 0, 127),
 *          q = clamp(rha(w / (d sc_j)) + 32, 0, 63) (32 when d sc_j = 0).
 *   A4G64  bias = down(min w), scale = up((max w - bias) / 15),
 *          q = clamp(rha((w - bias) / scale), 0, 15) (0 when scale = 0).
 *   w       DEVICE fp32 [M, K] contiguous, 4-byte aligned; finite values whose
 *           scales fit fp16.
 *   blocks  DEVICE, 16-byte aligned, M * qmm_row_bytes(type, K) bytes, written in
 *           the block layout above (rows back to back).  M = 0: no launch.
 * Deterministic: the bytes depend only on w.
 */
qmm_status qmm_quantize(qmm_type type, const float *w, int64_t M, int64_t K, void *blocks,
                        qmm_stream_t stream);

/* qmm_tile_for_tokens -- 64 when a 64-token tile pads no more tokens than a
 * 32-token tile, else 32 (candle pull request, section "Where the 64-token tile
 * is used").  Host-only and pure; N < 0 returns 0. */
int qmm_tile_for_tokens(int64_t N);

/* Helpers.  qmm_row_bytes returns 0 for an unknown type or a K that is not a
 * positive multiple of the block; the block queries return 0 for an unknown type. */
size_t qmm_row_bytes(qmm_type type, int64_t K);
int qmm_block_weights(qmm_type type);
int qmm_block_bytes(qmm_type type);
const char *qmm_status_string(qmm_status s);
const char *qmm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
