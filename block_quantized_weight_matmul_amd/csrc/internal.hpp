// internal.hpp -- launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

struct MatDesc {
  const uint8_t* blocks;  // device, 16-byte aligned
  int fmt;                // FMT_*
  int64_t n_experts, M, K;
  uint64_t row_bytes;
  int cus;                // compute units of the device (launch shapes are sized to fill them)
};

// Largest expert count the expert-indexed path accepts (its presence bitmap
// lives in LDS), and the largest token / slot counts of the matrix-vector paths.
constexpr int64_t kMaxExperts = 8192;
constexpr int64_t kMaxGemvTokens = 32;
constexpr int64_t kMaxSlots = 64;
// The matrix-matrix path addresses a 256-token slab of fp32 activations with
// 32-bit offsets: K * 4 bytes * 256 must stay below 4 GiB.
constexpr int64_t kMaxGemmK = int64_t(1) << 22;
// The expert-indexed matrix-matrix path scans every (token, slot) id in each
// workgroup's routing prologue: at most this many pairs per call.
constexpr int64_t kMaxGemmIdPairs = int64_t(1) << 18;

hipError_t launch_dequant(const MatDesc& m, int64_t expert, void* out, int out_f16, hipStream_t s);
hipError_t launch_quantize(int fmt, const float* w, int64_t M, int64_t K, void* out, hipStream_t s);
hipError_t launch_gemv(const MatDesc& m, const void* x, int x_f16, int N, float* y, hipStream_t s);
// Matrix-vector products of N tokens (1 .. 32) on up to kGemvGroupMax matrices of one
// format and K in one launch (y_i = x_i W_i^T, the bits of separate launch_gemv
// calls).  Returns hipErrorNotSupported, launching nothing, when the matrices cannot
// share the one-token or few-token kernel's launch shape; the caller then makes
// separate calls.
constexpr int kGemvGroupMax = 4;
hipError_t launch_gemv_group(const MatDesc* const* ms, const void* const* xs, float* const* ys, int n, int N,
                             int x_f16, hipStream_t s);
hipError_t launch_gemv_id(const MatDesc& m, const void* x, int x_f16, int N, int S, int x_per_slot,
                          const int32_t* ids, float* y, hipStream_t s);
// K splits of the matrix-matrix path for N tokens (splits = 1: unsplit)
struct GemmSplit {
  int splits;  // workgroups along K
  int stages;  // 64-deep K stages per split
};
GemmSplit gemm_split(const MatDesc& m, int64_t N);
size_t gemm_workspace_bytes(const MatDesc& m, int64_t N);
// split_ok: the call may divide K (qmm_gemm_ws, qmm_gemm_noalloc): among the waves of
// a workgroup up to 16 tokens, among workgroups above (ws: workspace of
// gemm_workspace_bytes(m, N) bytes when that is not 0); otherwise every K stage runs in
// one workgroup (qmm_gemm)
hipError_t launch_gemm(const MatDesc& m, const void* x, int x_f16, int64_t N, float* y, int tile, float* ws,
                       bool split_ok, hipStream_t s);
// The allocation-free entry point's scratch: its size, the once-per-device lookup of its
// device address (call with dev current), and that address (nullptr before the lookup).
size_t gemm_scratch_bytes();
hipError_t gemm_scratch_init(int dev);
float* gemm_scratch(int dev);
// tile: 32 or 64, or 0 for the tile rule on each expert's pair count
hipError_t launch_gemm_id(const MatDesc& m, const void* x, int x_f16, int64_t N, int64_t S, int x_per_slot,
                          const int32_t* ids, float* y, int tile, hipStream_t s);

}  // namespace qmm
