// api.hip -- the C ABI declared in include/qmm.h: argument checks, device checks
// and dispatch to the kernels.  No device memory is allocated here and nothing
// synchronises; every launch goes on the caller's stream.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <climits>
#include <new>

#include "qmm.h"
#include "decode.hpp"
#include "internal.hpp"

struct qmm_matrix {
  qmm::MatDesc d;
  int device;
};

namespace {

thread_local char g_err[512] = "";

qmm_status fail(qmm_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

qmm_status ok() {
  g_err[0] = '\0';
  return QMM_OK;
}

constexpr int kBW[qmm::kNumFormats] = {32, 32, 256, 256, 64, 32, 32, 32, 256, 256, 256};
constexpr int kBB[qmm::kNumFormats] = {18, 34, 144, 210, 36, 20, 22, 24, 84, 110, 176};

bool valid_type(int t) { return t >= 0 && t < qmm::kNumFormats; }
// the types qmm_quantize encodes (the others have no quantizer here)
bool quantizable_type(int t) { return t >= 0 && t <= QMM_A4G64; }
bool valid_dtype(int t) { return t == QMM_F32 || t == QMM_F16; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

qmm_status hip_fail(hipError_t e, const char* what) {
  return fail(QMM_E_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
}

// The current device must be the handle's device.
qmm_status check_device(const qmm_matrix* h) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != h->device)
    return fail(QMM_E_DEVICE, "current device %d is not the handle's device %d", dev, h->device);
  return QMM_OK;
}

qmm_status check_x(const void* x, int xt) {
  if (!valid_dtype(xt)) return fail(QMM_E_TYPE, "unknown activation dtype %d", xt);
  if (!x) return fail(QMM_E_ARG, "x is NULL");
  if (!aligned(x, 16)) return fail(QMM_E_ALIGN, "x must be 16-byte aligned");
  return QMM_OK;
}

qmm_status check_y(const float* y) {
  if (!y) return fail(QMM_E_ARG, "y is NULL");
  if (!aligned(y, 4)) return fail(QMM_E_ALIGN, "y must be 4-byte aligned");
  return QMM_OK;
}

}  // namespace

extern "C" {

size_t qmm_row_bytes(qmm_type t, int64_t K) {
  if (!valid_type(t) || K <= 0 || K % kBW[t] != 0) return 0;
  return static_cast<size_t>(K / kBW[t]) * kBB[t];
}

int qmm_block_weights(qmm_type t) { return valid_type(t) ? kBW[t] : 0; }
int qmm_block_bytes(qmm_type t) { return valid_type(t) ? kBB[t] : 0; }

int qmm_tile_for_tokens(int64_t N) {
  if (N < 0) return 0;
  const int64_t pad64 = (N + 63) / 64 * 64 - N;
  const int64_t pad32 = (N + 31) / 32 * 32 - N;
  return pad64 <= pad32 ? 64 : 32;
}

const char* qmm_status_string(qmm_status s) {
  switch (s) {
    case QMM_OK: return "QMM_OK";
    case QMM_E_ARG: return "QMM_E_ARG";
    case QMM_E_TYPE: return "QMM_E_TYPE";
    case QMM_E_SHAPE: return "QMM_E_SHAPE";
    case QMM_E_ALIGN: return "QMM_E_ALIGN";
    case QMM_E_DEVICE: return "QMM_E_DEVICE";
    case QMM_E_HIP: return "QMM_E_HIP";
    default: return "QMM_E_UNKNOWN";
  }
}

const char* qmm_last_error(void) { return g_err; }

qmm_status qmm_create(qmm_matrix** out, qmm_type type, const void* blocks, int64_t n_experts,
                      int64_t M, int64_t K) {
  if (!out) return fail(QMM_E_ARG, "out is NULL");
  *out = nullptr;
  if (!valid_type(type)) return fail(QMM_E_TYPE, "unknown block type %d", static_cast<int>(type));
  if (!blocks) return fail(QMM_E_ARG, "blocks is NULL");
  if (!aligned(blocks, 16)) return fail(QMM_E_ALIGN, "blocks must be 16-byte aligned");
  if (n_experts < 1 || M < 1 || M > INT_MAX / 2)
    return fail(QMM_E_SHAPE, "need n_experts >= 1 and 1 <= M < 2^30 (got %lld, %lld)",
                static_cast<long long>(n_experts), static_cast<long long>(M));
  const size_t rb = qmm_row_bytes(type, K);
  if (rb == 0 || K > INT_MAX / 2)
    return fail(QMM_E_SHAPE, "K=%lld is not a positive multiple of %d (or too large)",
                static_cast<long long>(K), kBW[type]);
  if (static_cast<double>(M) * static_cast<double>(rb) >= 4294967296.0)
    return fail(QMM_E_SHAPE, "one matrix (M * row bytes) must be below 4 GiB");
  if (static_cast<double>(n_experts) * static_cast<double>(M) * static_cast<double>(rb) > 9.0e18)
    return fail(QMM_E_SHAPE, "tensor too large");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(QMM_E_DEVICE, "no HIP device: %s", hipGetErrorString(e));
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return fail(QMM_E_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(QMM_E_DEVICE, "device %d is %s, this library is built for gfx950", dev, prop.gcnArchName);
  qmm_matrix* h = new (std::nothrow) qmm_matrix;
  if (!h) return fail(QMM_E_ARG, "out of host memory");
  h->d.blocks = static_cast<const uint8_t*>(blocks);
  h->d.fmt = static_cast<int>(type);
  h->d.n_experts = n_experts;
  h->d.M = M;
  h->d.K = K;
  h->d.row_bytes = rb;
  h->d.cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  h->device = dev;
  // set-up of qmm_gemm_noalloc's scratch on this device (once per device); a failure
  // is reported by that entry point, the others do not need it
  (void)qmm::gemm_scratch_init(dev);
  *out = h;
  return ok();
}

qmm_status qmm_destroy(qmm_matrix* h) {
  delete h;
  return ok();
}

qmm_status qmm_gemv(const qmm_matrix* h, const void* x, qmm_dtype xt, int64_t N, float* y,
                    qmm_stream_t stream) {
  if (!h) return fail(QMM_E_ARG, "handle is NULL");
  if (h->d.n_experts != 1) return fail(QMM_E_ARG, "qmm_gemv needs a handle with n_experts == 1");
  if (N < 0 || N > qmm::kMaxGemvTokens)
    return fail(QMM_E_SHAPE, "qmm_gemv takes 0..%lld tokens (got %lld)",
                static_cast<long long>(qmm::kMaxGemvTokens), static_cast<long long>(N));
  qmm_status s;
  if ((s = check_x(x, xt)) != QMM_OK || (s = check_y(y)) != QMM_OK) return s;
  if (N == 0) return ok();
  if ((s = check_device(h)) != QMM_OK) return s;
  const hipError_t e = qmm::launch_gemv(h->d, x, xt == QMM_F16, static_cast<int>(N), y,
                                        reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gemv launch");
  return ok();
}

qmm_status qmm_gemv_group(const qmm_matrix* const* hs, const void* const* xs, qmm_dtype xt, int64_t N,
                          float* const* ys, int count, qmm_stream_t stream) {
  if (count < 0 || count > QMM_GEMV_GROUP_MAX)
    return fail(QMM_E_ARG, "qmm_gemv_group takes 0..%d matrices (got %d)", QMM_GEMV_GROUP_MAX, count);
  if (count == 0) return ok();
  if (!hs || !xs || !ys) return fail(QMM_E_ARG, "handle, activation and output arrays must not be NULL");
  if (N < 0 || N > qmm::kMaxGemvTokens)
    return fail(QMM_E_SHAPE, "qmm_gemv_group takes 0..%lld tokens (got %lld)",
                static_cast<long long>(qmm::kMaxGemvTokens), static_cast<long long>(N));
  qmm_status s;
  for (int i = 0; i < count; ++i) {
    if (!hs[i]) return fail(QMM_E_ARG, "handle %d is NULL", i);
    if (hs[i]->d.n_experts != 1) return fail(QMM_E_ARG, "qmm_gemv_group needs handles with n_experts == 1 (handle %d)", i);
    if ((s = check_x(xs[i], xt)) != QMM_OK || (s = check_y(ys[i])) != QMM_OK) return s;
  }
  if (N == 0) return ok();
  for (int i = 0; i < count; ++i)
    if ((s = check_device(hs[i])) != QMM_OK) return s;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int xf = xt == QMM_F16;
  // in order of first appearance: up to kGemvGroupMax not yet launched matrices of
  // the same K in one launch (the kernels take one format, or Q4_K with Q6_K at one
  // token), else those of the same format and K, else the matrix alone
  bool done[QMM_GEMV_GROUP_MAX] = {};
  for (int i = 0; i < count; ++i) {
    if (done[i]) continue;
    hipError_t e = hipErrorNotSupported;
    for (int same_fmt = 0; same_fmt < 2 && e == hipErrorNotSupported; ++same_fmt) {
      const qmm::MatDesc* ms[qmm::kGemvGroupMax];
      const void* gx[qmm::kGemvGroupMax];
      float* gy[qmm::kGemvGroupMax];
      int idx[qmm::kGemvGroupMax];
      int n = 0;
      for (int j = i; j < count && n < qmm::kGemvGroupMax; ++j)
        if (!done[j] && hs[j]->d.K == hs[i]->d.K && (!same_fmt || hs[j]->d.fmt == hs[i]->d.fmt)) {
          ms[n] = &hs[j]->d;
          gx[n] = xs[j];
          gy[n] = ys[j];
          idx[n++] = j;
        }
      if (n < 2) continue;
      e = qmm::launch_gemv_group(ms, gx, gy, n, static_cast<int>(N), xf, st);
      if (e == hipSuccess)
        for (int k = 0; k < n; ++k) done[idx[k]] = true;
    }
    if (e == hipSuccess) continue;
    if (e != hipErrorNotSupported) return hip_fail(e, "gemv group launch");
    e = qmm::launch_gemv(hs[i]->d, xs[i], xf, static_cast<int>(N), ys[i], st);
    if (e != hipSuccess) return hip_fail(e, "gemv launch");
    done[i] = true;
  }
  return ok();
}

qmm_status qmm_gemm(const qmm_matrix* h, const void* x, qmm_dtype xt, int64_t N, float* y, qmm_tile tile,
                    qmm_stream_t stream) {
  if (!h) return fail(QMM_E_ARG, "handle is NULL");
  if (h->d.n_experts != 1) return fail(QMM_E_ARG, "qmm_gemm needs a handle with n_experts == 1");
  if (tile != QMM_TILE_AUTO && tile != QMM_TILE_32 && tile != QMM_TILE_64)
    return fail(QMM_E_ARG, "tile must be QMM_TILE_AUTO, QMM_TILE_32 or QMM_TILE_64 (got %d)", static_cast<int>(tile));
  if (N < 0 || N > (1LL << 24))
    return fail(QMM_E_SHAPE, "qmm_gemm takes 0..2^24 tokens (got %lld)", static_cast<long long>(N));
  if (h->d.K >= qmm::kMaxGemmK)
    return fail(QMM_E_SHAPE, "qmm_gemm takes K below %lld (handle has K=%lld)",
                static_cast<long long>(qmm::kMaxGemmK), static_cast<long long>(h->d.K));
  qmm_status s;
  if ((s = check_x(x, xt)) != QMM_OK || (s = check_y(y)) != QMM_OK) return s;
  if (N == 0) return ok();
  if ((s = check_device(h)) != QMM_OK) return s;
  const int T = tile == QMM_TILE_AUTO ? qmm_tile_for_tokens(N) : static_cast<int>(tile);
  const hipError_t e =
      qmm::launch_gemm(h->d, x, xt == QMM_F16, N, y, T, nullptr, false, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gemm launch");
  return ok();
}

size_t qmm_gemm_workspace_bytes(const qmm_matrix* h, int64_t N) {
  if (!h || h->d.n_experts != 1 || N <= 0 || N > (1LL << 24) || h->d.K >= qmm::kMaxGemmK) return 0;
  return qmm::gemm_workspace_bytes(h->d, N);
}

qmm_status qmm_gemm_ws(const qmm_matrix* h, const void* x, qmm_dtype xt, int64_t N, float* y, qmm_tile tile,
                       void* ws, size_t ws_bytes, qmm_stream_t stream) {
  if (!h) return fail(QMM_E_ARG, "handle is NULL");
  if (h->d.n_experts != 1) return fail(QMM_E_ARG, "qmm_gemm_ws needs a handle with n_experts == 1");
  if (tile != QMM_TILE_AUTO && tile != QMM_TILE_32 && tile != QMM_TILE_64)
    return fail(QMM_E_ARG, "tile must be QMM_TILE_AUTO, QMM_TILE_32 or QMM_TILE_64 (got %d)", static_cast<int>(tile));
  if (N < 0 || N > (1LL << 24))
    return fail(QMM_E_SHAPE, "qmm_gemm_ws takes 0..2^24 tokens (got %lld)", static_cast<long long>(N));
  if (h->d.K >= qmm::kMaxGemmK)
    return fail(QMM_E_SHAPE, "qmm_gemm_ws takes K below %lld (handle has K=%lld)",
                static_cast<long long>(qmm::kMaxGemmK), static_cast<long long>(h->d.K));
  qmm_status s;
  if ((s = check_x(x, xt)) != QMM_OK || (s = check_y(y)) != QMM_OK) return s;
  if (N == 0) return ok();
  const size_t need = qmm::gemm_workspace_bytes(h->d, N);
  if (need > 0) {
    if (!ws) return fail(QMM_E_ARG, "ws is NULL; this call needs %zu bytes", need);
    if (ws_bytes < need) return fail(QMM_E_ARG, "ws holds %zu bytes; this call needs %zu", ws_bytes, need);
    if (!aligned(ws, 16)) return fail(QMM_E_ALIGN, "ws must be 16-byte aligned");
  }
  if ((s = check_device(h)) != QMM_OK) return s;
  const int T = tile == QMM_TILE_AUTO ? qmm_tile_for_tokens(N) : static_cast<int>(tile);
  const hipError_t e = qmm::launch_gemm(h->d, x, xt == QMM_F16, N, y, T, need > 0 ? static_cast<float*>(ws) : nullptr, true,
                                        reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gemm launch");
  return ok();
}

qmm_status qmm_gemm_noalloc(const qmm_matrix* h, const void* x, qmm_dtype xt, int64_t N, float* y, qmm_tile tile,
                            qmm_stream_t stream) {
  if (!h) return fail(QMM_E_ARG, "handle is NULL");
  if (h->d.n_experts != 1) return fail(QMM_E_ARG, "qmm_gemm_noalloc needs a handle with n_experts == 1");
  if (tile != QMM_TILE_AUTO && tile != QMM_TILE_32 && tile != QMM_TILE_64)
    return fail(QMM_E_ARG, "tile must be QMM_TILE_AUTO, QMM_TILE_32 or QMM_TILE_64 (got %d)", static_cast<int>(tile));
  if (N < 0 || N > (1LL << 24))
    return fail(QMM_E_SHAPE, "qmm_gemm_noalloc takes 0..2^24 tokens (got %lld)", static_cast<long long>(N));
  if (h->d.K >= qmm::kMaxGemmK)
    return fail(QMM_E_SHAPE, "qmm_gemm_noalloc takes K below %lld (handle has K=%lld)",
                static_cast<long long>(qmm::kMaxGemmK), static_cast<long long>(h->d.K));
  qmm_status s;
  if ((s = check_x(x, xt)) != QMM_OK || (s = check_y(y)) != QMM_OK) return s;
  if (N == 0) return ok();
  const size_t need = qmm::gemm_workspace_bytes(h->d, N);
  if (need > qmm::gemm_scratch_bytes())
    return fail(QMM_E_SHAPE,
                "qmm_gemm_noalloc: this call's K split needs %zu bytes of scratch, above the library's %zu "
                "(use qmm_gemm_ws with a workspace, or qmm_gemm)", need, qmm::gemm_scratch_bytes());
  if ((s = check_device(h)) != QMM_OK) return s;
  float* scratch = nullptr;
  if (need > 0) {
    const hipError_t ei = qmm::gemm_scratch_init(h->device);  // no-op after qmm_create's
    if (ei != hipSuccess) return hip_fail(ei, "hipGetSymbolAddress(scratch)");
    scratch = qmm::gemm_scratch(h->device);
  }
  const int T = tile == QMM_TILE_AUTO ? qmm_tile_for_tokens(N) : static_cast<int>(tile);
  const hipError_t e = qmm::launch_gemm(h->d, x, xt == QMM_F16, N, y, T, scratch, true, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gemm launch");
  return ok();
}

qmm_status qmm_gemm_id(const qmm_matrix* h, const void* x, qmm_dtype xt, int64_t N, int64_t S,
                       int x_per_slot, const int32_t* ids, float* y, qmm_stream_t stream) {
  if (!h) return fail(QMM_E_ARG, "handle is NULL");
  if (h->d.n_experts > qmm::kMaxExperts)
    return fail(QMM_E_SHAPE, "qmm_gemm_id takes at most %lld experts (handle has %lld)",
                static_cast<long long>(qmm::kMaxExperts), static_cast<long long>(h->d.n_experts));
  if (N < 0 || N > qmm::kMaxGemvTokens)
    return fail(QMM_E_SHAPE, "qmm_gemm_id takes 0..%lld tokens (got %lld)",
                static_cast<long long>(qmm::kMaxGemvTokens), static_cast<long long>(N));
  if (S < 1 || S > qmm::kMaxSlots)
    return fail(QMM_E_SHAPE, "qmm_gemm_id takes 1..%lld slots per token (got %lld)",
                static_cast<long long>(qmm::kMaxSlots), static_cast<long long>(S));
  if (x_per_slot != 0 && x_per_slot != 1) return fail(QMM_E_ARG, "x_per_slot must be 0 or 1");
  qmm_status s;
  if ((s = check_x(x, xt)) != QMM_OK || (s = check_y(y)) != QMM_OK) return s;
  if (!ids) return fail(QMM_E_ARG, "ids is NULL");
  if (!aligned(ids, 4)) return fail(QMM_E_ALIGN, "ids must be 4-byte aligned");
  if (N == 0) return ok();
  if ((s = check_device(h)) != QMM_OK) return s;
  const hipError_t e = qmm::launch_gemv_id(h->d, x, xt == QMM_F16, static_cast<int>(N), static_cast<int>(S),
                                           x_per_slot, ids, y, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gemm_id launch");
  return ok();
}

qmm_status qmm_gemm_id_tiled(const qmm_matrix* h, const void* x, qmm_dtype xt, int64_t N, int64_t S,
                             int x_per_slot, const int32_t* ids, float* y, qmm_tile tile, qmm_stream_t stream) {
  if (!h) return fail(QMM_E_ARG, "handle is NULL");
  if (h->d.n_experts > qmm::kMaxExperts)
    return fail(QMM_E_SHAPE, "qmm_gemm_id_tiled takes at most %lld experts (handle has %lld)",
                static_cast<long long>(qmm::kMaxExperts), static_cast<long long>(h->d.n_experts));
  if (tile != QMM_TILE_AUTO && tile != QMM_TILE_32 && tile != QMM_TILE_64)
    return fail(QMM_E_ARG, "tile must be QMM_TILE_AUTO, QMM_TILE_32 or QMM_TILE_64 (got %d)", static_cast<int>(tile));
  if (S < 1 || S > qmm::kMaxSlots)
    return fail(QMM_E_SHAPE, "qmm_gemm_id_tiled takes 1..%lld slots per token (got %lld)",
                static_cast<long long>(qmm::kMaxSlots), static_cast<long long>(S));
  if (N < 0 || N * S > qmm::kMaxGemmIdPairs)
    return fail(QMM_E_SHAPE, "qmm_gemm_id_tiled takes 0..%lld (token, slot) pairs (got %lld x %lld)",
                static_cast<long long>(qmm::kMaxGemmIdPairs), static_cast<long long>(N), static_cast<long long>(S));
  if (h->d.K >= qmm::kMaxGemmK)
    return fail(QMM_E_SHAPE, "qmm_gemm_id_tiled takes K below %lld (handle has K=%lld)",
                static_cast<long long>(qmm::kMaxGemmK), static_cast<long long>(h->d.K));
  if (x_per_slot != 0 && x_per_slot != 1) return fail(QMM_E_ARG, "x_per_slot must be 0 or 1");
  const int64_t xrows = x_per_slot ? N * S : N;
  if (xrows * h->d.K * (xt == QMM_F16 ? 2 : 4) >= (int64_t(1) << 32))
    return fail(QMM_E_SHAPE, "qmm_gemm_id_tiled takes activations below 4 GiB");
  qmm_status s;
  if ((s = check_x(x, xt)) != QMM_OK || (s = check_y(y)) != QMM_OK) return s;
  if (!ids) return fail(QMM_E_ARG, "ids is NULL");
  if (!aligned(ids, 4)) return fail(QMM_E_ALIGN, "ids must be 4-byte aligned");
  if (N == 0) return ok();
  if ((s = check_device(h)) != QMM_OK) return s;
  const hipError_t e = qmm::launch_gemm_id(h->d, x, xt == QMM_F16, N, S, x_per_slot, ids, y, static_cast<int>(tile),
                                           reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gemm_id_tiled launch");
  return ok();
}

qmm_status qmm_quantize(qmm_type type, const float* w, int64_t M, int64_t K, void* blocks, qmm_stream_t stream) {
  if (!valid_type(type)) return fail(QMM_E_TYPE, "unknown block type %d", static_cast<int>(type));
  if (!quantizable_type(type))
    return fail(QMM_E_TYPE, "qmm_quantize encodes Q4_0, Q8_0, Q4_K, Q6_K and A4G64 only (got type %d)",
                static_cast<int>(type));
  if (M < 0 || M > INT_MAX / 2) return fail(QMM_E_SHAPE, "M=%lld out of range", static_cast<long long>(M));
  const size_t rb = qmm_row_bytes(type, K);
  if (rb == 0 || K > INT_MAX / 2)
    return fail(QMM_E_SHAPE, "K=%lld is not a positive multiple of %d (or too large)",
                static_cast<long long>(K), kBW[type]);
  if (!w) return fail(QMM_E_ARG, "w is NULL");
  if (!blocks) return fail(QMM_E_ARG, "blocks is NULL");
  if (!aligned(w, 4)) return fail(QMM_E_ALIGN, "w must be 4-byte aligned");
  if (!aligned(blocks, 16)) return fail(QMM_E_ALIGN, "blocks must be 16-byte aligned");
  if (M == 0) return ok();
  const hipError_t e = qmm::launch_quantize(static_cast<int>(type), w, M, K, blocks,
                                            reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "quantize launch");
  return ok();
}

qmm_status qmm_dequantize(const qmm_matrix* h, int64_t expert, void* out, qmm_dtype ot, qmm_stream_t stream) {
  if (!h) return fail(QMM_E_ARG, "handle is NULL");
  if (expert < 0 || expert >= h->d.n_experts)
    return fail(QMM_E_SHAPE, "expert %lld outside [0, %lld)", static_cast<long long>(expert),
                static_cast<long long>(h->d.n_experts));
  if (!valid_dtype(ot)) return fail(QMM_E_TYPE, "unknown output dtype %d", static_cast<int>(ot));
  if (!out) return fail(QMM_E_ARG, "out is NULL");
  if (!aligned(out, 16)) return fail(QMM_E_ALIGN, "out must be 16-byte aligned");
  qmm_status s;
  if ((s = check_device(h)) != QMM_OK) return s;
  const hipError_t e = qmm::launch_dequant(h->d, expert, out, ot == QMM_F16, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "dequantize launch");
  return ok();
}

}  // extern "C"
