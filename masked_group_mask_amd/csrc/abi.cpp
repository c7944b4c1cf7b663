// C ABI of libwide.so: host-side argument validation and dispatch.
// Every check runs before any HIP call, so an invalid request returns an
// error without touching the device or the caller's buffers.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "launch.hpp"

namespace {

constexpr int64_t kI32Max = 2147483647;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Half-open byte ranges [p, p + n) and [q, q + m) intersect.
bool overlap(const void *p, size_t n, const void *q, size_t m) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + m && b < a + n;
}

size_t span_bytes(int64_t rows, int64_t cols, int64_t ld, size_t esize) {
  return (size_t)((rows - 1) * ld + cols) * esize;
}

// 1 = device present, 0 = none; probed once.
int device_ok() {
  static std::atomic<int> state{-1};
  int s = state.load();
  if (s < 0) {
    int n = 0;
    s = (hipGetDeviceCount(&n) == hipSuccess && n > 0) ? 1 : 0;
    state.store(s);
  }
  return s;
}

bool valid_dtype(int t) { return t == WIDE_DTYPE_BF16 || t == WIDE_DTYPE_F32; }

int check_mn(const wide_bf16 *A, int64_t lda, const wide_bf16 *B0, const wide_bf16 *B1,
             int64_t ldb, const void *C, int64_t ldc, int c_dtype, int64_t M, int64_t N,
             int64_t K, int64_t G, const int32_t *perm, const int32_t *counts,
             const uint8_t *mask) {
  if (!A || !B0 || !C) return WIDE_ERR_INVALID_ARG;
  if (M < 1 || N < 1 || K < 1 || G < 1) return WIDE_ERR_INVALID_ARG;
  if (M > kI32Max || N > kI32Max || K > kI32Max) return WIDE_ERR_INVALID_ARG;
  if (N % G != 0 || K % 8 != 0) return WIDE_ERR_INVALID_ARG;
  if (lda < K || ldb < K || lda % 8 != 0 || ldb % 8 != 0 || ldc < N) return WIDE_ERR_INVALID_ARG;
  if (!valid_dtype(c_dtype)) return WIDE_ERR_INVALID_ARG;
  if (!aligned16(A) || !aligned16(B0) || !aligned16(C) || (B1 && !aligned16(B1)))
    return WIDE_ERR_INVALID_ARG;
  if (perm == nullptr) {
    if (mask == nullptr || M > 4) return WIDE_ERR_INVALID_ARG;
  } else if (counts == nullptr) {
    return WIDE_ERR_INVALID_ARG;
  }
  const size_t cb = span_bytes(M, N, ldc, c_dtype == WIDE_DTYPE_F32 ? 4 : 2);
  if (overlap(C, cb, A, span_bytes(M, K, lda, 2)) || overlap(C, cb, B0, span_bytes(N, K, ldb, 2)) ||
      (B1 && overlap(C, cb, B1, span_bytes(N, K, ldb, 2))))
    return WIDE_ERR_INVALID_ARG;
  if (G % 16 != 0) return WIDE_ERR_UNSUPPORTED;
  // Gathered rows are addressed with 32-bit byte offsets into A, a tile's
  // (at most 256) weight rows with 32-bit offsets into B.
  if ((uint64_t)M * (uint64_t)lda * 2u > 0x7fffffffull || (uint64_t)ldb * 512u > 0x7fffffffull)
    return WIDE_ERR_UNSUPPORTED;
  return WIDE_OK;
}

// Validates a GEMM-MN workspace; on success `ws` is the pointer the launcher
// takes (null when no workspace applies: no perm, or a plan that splits
// nothing).
int check_mn_ws(const wide_bf16 *A, int64_t lda, const wide_bf16 *B0, const wide_bf16 *B1,
                int64_t ldb, const void *C, int64_t ldc, int c_dtype, int64_t M, int64_t N,
                int64_t K, int64_t G, const int32_t *perm, const int32_t *counts, void *&ws,
                size_t ws_bytes) {
  if (ws == nullptr) return WIDE_OK;
  if (perm == nullptr) {
    ws = nullptr;
    return WIDE_OK;
  }
  const size_t need = wide::gemm_mn_workspace_bytes((int)M, (int)N, (int)K, (int)G, B1 != nullptr);
  if (ws_bytes < need || !aligned16(ws)) return WIDE_ERR_INVALID_ARG;
  if (need == 0) {
    ws = nullptr;
    return WIDE_OK;
  }
  const size_t cb = span_bytes(M, N, ldc, c_dtype == WIDE_DTYPE_F32 ? 4 : 2);
  const size_t ng = (size_t)(N / G);
  if (overlap(ws, need, A, span_bytes(M, K, lda, 2)) || overlap(ws, need, B0, span_bytes(N, K, ldb, 2)) ||
      (B1 && overlap(ws, need, B1, span_bytes(N, K, ldb, 2))) || overlap(ws, need, C, cb) ||
      overlap(ws, need, perm, ng * (size_t)M * 4) || overlap(ws, need, counts, ng * 4))
    return WIDE_ERR_INVALID_ARG;
  return WIDE_OK;
}

int gemm_mn_impl(const wide_bf16 *A, int64_t lda, const wide_bf16 *B0, const wide_bf16 *B1, int64_t ldb,
                 void *C, int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K, int64_t G,
                 const int32_t *perm, const int32_t *counts, const uint8_t *mask, void *ws,
                 size_t ws_bytes, wide_stream_t stream) {
  int st = check_mn(A, lda, B0, B1, ldb, C, ldc, c_dtype, M, N, K, G, perm, counts, mask);
  if (st != WIDE_OK) return st;
  st = check_mn_ws(A, lda, B0, B1, ldb, C, ldc, c_dtype, M, N, K, G, perm, counts, ws, ws_bytes);
  if (st != WIDE_OK) return st;
  if (!device_ok()) return WIDE_ERR_NO_DEVICE;
  wide::MnArgs a{A, lda, B0, B1, ldb, C, ldc, c_dtype == WIDE_DTYPE_F32, (int)M, (int)N,
                 (int)K, (int)G, perm, counts, mask};
  a.ws = ws;
  a.ws_bytes = ws_bytes;
  return wide::launch_gemm_mn(a, reinterpret_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

int wide_abi_version(void) { return 2; }

const char *wide_status_string(int status) {
  switch (status) {
    case WIDE_OK: return "ok";
    case WIDE_ERR_INVALID_ARG: return "invalid argument";
    case WIDE_ERR_UNSUPPORTED: return "unsupported shape or mode";
    case WIDE_ERR_NO_DEVICE: return "no HIP device";
    case WIDE_ERR_LAUNCH: return "kernel launch failed";
    case WIDE_ERR_TOO_LARGE: return "needs more scratch than the built-in buffer holds";
    default: return "unknown status";
  }
}

int wide_reorder(const uint8_t *mask, int64_t batch, int64_t rows, int64_t groups,
                 int32_t *perm, int32_t *counts, wide_stream_t stream) {
  if (!mask || !perm || !counts) return WIDE_ERR_INVALID_ARG;
  if (batch < 1 || rows < 1 || groups < 1) return WIDE_ERR_INVALID_ARG;
  if (rows > kI32Max || groups > kI32Max || batch > 65535) return WIDE_ERR_INVALID_ARG;
  if ((groups + 7) / 8 > kI32Max) return WIDE_ERR_INVALID_ARG;
  const size_t mb = (size_t)batch * rows * groups;
  if (overlap(perm, mb * 4, mask, mb) || overlap(counts, (size_t)batch * groups * 4, mask, mb) ||
      overlap(counts, (size_t)batch * groups * 4, perm, mb * 4))
    return WIDE_ERR_INVALID_ARG;
  if (!device_ok()) return WIDE_ERR_NO_DEVICE;
  return wide::launch_reorder(mask, (int)batch, (int)rows, (int)groups, perm, counts,
                              reinterpret_cast<hipStream_t>(stream));
}

int wide_gemm_mn(const wide_bf16 *A, int64_t lda, const wide_bf16 *B, int64_t ldb, void *C,
                 int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K, int64_t G,
                 const int32_t *perm, const int32_t *counts, const uint8_t *mask,
                 wide_stream_t stream) {
  return gemm_mn_impl(A, lda, B, nullptr, ldb, C, ldc, c_dtype, M, N, K, G, perm, counts, mask, nullptr, 0,
                      stream);
}

int wide_gemm_mn_swiglu(const wide_bf16 *A, int64_t lda, const wide_bf16 *Wg, const wide_bf16 *Wu,
                        int64_t ldb, void *H, int64_t ldh, int h_dtype, int64_t M, int64_t N,
                        int64_t K, int64_t G, const int32_t *perm, const int32_t *counts,
                        const uint8_t *mask, wide_stream_t stream) {
  if (!Wu) return WIDE_ERR_INVALID_ARG;
  return gemm_mn_impl(A, lda, Wg, Wu, ldb, H, ldh, h_dtype, M, N, K, G, perm, counts, mask, nullptr, 0, stream);
}

size_t wide_gemm_mn_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t G, int swiglu) {
  if (M < 1 || N < 1 || K < 1 || G < 1 || M > kI32Max || N > kI32Max || K > kI32Max || N % G != 0) return 0;
  return wide::gemm_mn_workspace_bytes((int)M, (int)N, (int)K, (int)G, swiglu != 0);
}

int wide_gemm_mn_ws(const wide_bf16 *A, int64_t lda, const wide_bf16 *B, int64_t ldb, void *C,
                    int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K, int64_t G,
                    const int32_t *perm, const int32_t *counts, const uint8_t *mask, void *workspace,
                    size_t workspace_bytes, wide_stream_t stream) {
  return gemm_mn_impl(A, lda, B, nullptr, ldb, C, ldc, c_dtype, M, N, K, G, perm, counts, mask, workspace,
                      workspace_bytes, stream);
}

int wide_gemm_mn_swiglu_ws(const wide_bf16 *A, int64_t lda, const wide_bf16 *Wg, const wide_bf16 *Wu,
                           int64_t ldb, void *H, int64_t ldh, int h_dtype, int64_t M, int64_t N,
                           int64_t K, int64_t G, const int32_t *perm, const int32_t *counts,
                           const uint8_t *mask, void *workspace, size_t workspace_bytes,
                           wide_stream_t stream) {
  if (!Wu) return WIDE_ERR_INVALID_ARG;
  return gemm_mn_impl(A, lda, Wg, Wu, ldb, H, ldh, h_dtype, M, N, K, G, perm, counts, mask, workspace,
                      workspace_bytes, stream);
}

int wide_order_by_pattern(const uint8_t *mask, int64_t rows, int64_t groups, int32_t *order,
                          wide_stream_t stream) {
  if (!mask || !order) return WIDE_ERR_INVALID_ARG;
  if (rows < 1 || groups < 1 || rows > kI32Max || groups > kI32Max) return WIDE_ERR_INVALID_ARG;
  if (overlap(order, (size_t)rows * 4, mask, (size_t)rows * groups)) return WIDE_ERR_INVALID_ARG;
  if (!device_ok()) return WIDE_ERR_NO_DEVICE;
  return wide::launch_pattern_order(mask, (int)rows, (int)groups, order, reinterpret_cast<hipStream_t>(stream));
}

int wide_gemm_k(const wide_bf16 *A, int64_t lda, const wide_bf16 *B, int64_t ldb, float *C,
                int64_t ldc, int beta, int64_t M, int64_t N, int64_t K, int64_t G,
                const int32_t *order, const uint8_t *mask, wide_stream_t stream) {
  return wide_gemm_k_ws(A, lda, B, ldb, C, ldc, beta, M, N, K, G, order, mask, nullptr, 0, stream);
}

size_t wide_gemm_k_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1 || M > kI32Max || N > kI32Max || K > kI32Max) return 0;
  return wide::gemm_k_workspace_bytes((int)M, (int)N, (int)K);
}

int wide_gemm_k_ws(const wide_bf16 *A, int64_t lda, const wide_bf16 *B, int64_t ldb, float *C,
                   int64_t ldc, int beta, int64_t M, int64_t N, int64_t K, int64_t G,
                   const int32_t *order, const uint8_t *mask, void *workspace, size_t workspace_bytes,
                   wide_stream_t stream) {
  if (!A || !B || !C || !mask) return WIDE_ERR_INVALID_ARG;
  if (M < 1 || N < 1 || K < 1 || G < 1) return WIDE_ERR_INVALID_ARG;
  if (M > kI32Max || N > kI32Max || K > kI32Max) return WIDE_ERR_INVALID_ARG;
  if (K % G != 0 || lda < K || ldb < K || lda % 8 != 0 || ldb % 8 != 0) return WIDE_ERR_INVALID_ARG;
  if (ldc < N || ldc % 4 != 0 || (beta != 0 && beta != 1)) return WIDE_ERR_INVALID_ARG;
  if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return WIDE_ERR_INVALID_ARG;
  const size_t cb = span_bytes(M, N, ldc, 4);
  if (overlap(C, cb, A, span_bytes(M, K, lda, 2)) || overlap(C, cb, B, span_bytes(N, K, ldb, 2)) ||
      overlap(C, cb, mask, (size_t)M * (K / G)) || (order && overlap(C, cb, order, (size_t)M * 4)))
    return WIDE_ERR_INVALID_ARG;
  if (G % 16 != 0 || K / G > 512 || N % 128 != 0) return WIDE_ERR_UNSUPPORTED;
  // A tile of 256 rows and a B tile of 128 rows are addressed with 32-bit byte offsets.
  if ((uint64_t)lda * 512u > 0x7fffffffull || (uint64_t)ldb * 512u > 0x7fffffffull)
    return WIDE_ERR_UNSUPPORTED;
  if (workspace != nullptr) {
    const size_t need = wide::gemm_k_workspace_bytes((int)M, (int)N, (int)K);
    if (workspace_bytes < need || !aligned16(workspace)) return WIDE_ERR_INVALID_ARG;
    if (need > 0 && (overlap(workspace, need, A, span_bytes(M, K, lda, 2)) ||
                     overlap(workspace, need, B, span_bytes(N, K, ldb, 2)) || overlap(workspace, need, C, cb) ||
                     overlap(workspace, need, mask, (size_t)M * (K / G)) ||
                     (order && overlap(workspace, need, order, (size_t)M * 4))))
      return WIDE_ERR_INVALID_ARG;
    if (need == 0) workspace = nullptr;
  }
  if (!device_ok()) return WIDE_ERR_NO_DEVICE;
  wide::KArgs a{A, lda, B, ldb, C, ldc, beta, (int)M, (int)N, (int)K, (int)G, mask, order,
                static_cast<float *>(workspace), workspace_bytes, 0, 0, 0, 1};
  return wide::launch_gemm_k(a, reinterpret_cast<hipStream_t>(stream));
}

int wide_gemm_k_grouped(const wide_bf16 *A, int64_t lda, const wide_bf16 *B, int64_t ldb, float *C,
                        int64_t ldc, int beta, int64_t M, int64_t N, int64_t K, int64_t G,
                        const int32_t *perm, const int32_t *counts, wide_stream_t stream) {
  if (!A || !B || !C || !perm || !counts) return WIDE_ERR_INVALID_ARG;
  if (M < 1 || N < 1 || K < 1 || G < 1) return WIDE_ERR_INVALID_ARG;
  if (M > kI32Max || N > kI32Max || K > kI32Max) return WIDE_ERR_INVALID_ARG;
  if (K % G != 0 || lda < K || ldb < K || lda % 8 != 0 || ldb % 8 != 0) return WIDE_ERR_INVALID_ARG;
  if (ldc < N || ldc % 4 != 0 || (beta != 0 && beta != 1)) return WIDE_ERR_INVALID_ARG;
  if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return WIDE_ERR_INVALID_ARG;
  const int64_t NG = K / G;
  const size_t cb = span_bytes(M, N, ldc, 4);
  if (overlap(C, cb, A, span_bytes(M, K, lda, 2)) || overlap(C, cb, B, span_bytes(N, K, ldb, 2)) ||
      overlap(C, cb, perm, (size_t)NG * M * 4) || overlap(C, cb, counts, (size_t)NG * 4))
    return WIDE_ERR_INVALID_ARG;
  if (G % 64 != 0 || N % 128 != 0) return WIDE_ERR_UNSUPPORTED;
  // Gathered rows are addressed with 32-bit byte offsets into A, a tile's
  // (at most 256) weight rows with 32-bit offsets into B; one workgroup per
  // (group, row tile, column tile).
  if ((uint64_t)M * (uint64_t)lda * 2u > 0x7fffffffull || (uint64_t)ldb * 512u > 0x7fffffffull)
    return WIDE_ERR_UNSUPPORTED;
  if ((uint64_t)NG * (uint64_t)((M + 255) / 256) * (uint64_t)(N / 128) > 0x7fffffffull)
    return WIDE_ERR_UNSUPPORTED;
  if (!device_ok()) return WIDE_ERR_NO_DEVICE;
  wide::KgArgs a{A, lda, B, ldb, C, ldc, beta, (int)M, (int)N, (int)K, (int)G, perm, counts};
  return wide::launch_gemm_kg(a, reinterpret_cast<hipStream_t>(stream));
}

int wide_router(const wide_bf16 *X, int64_t ldx, const wide_bf16 *W1, const wide_bf16 *W2,
                int64_t batch, int64_t rows, int64_t D, int64_t r, int64_t groups, uint8_t *mask,
                float *logits, int32_t *perm, int32_t *counts, wide_stream_t stream) {
  if (!X || !W1 || !W2 || !mask || (perm == nullptr) != (counts == nullptr)) return WIDE_ERR_INVALID_ARG;
  if (batch < 1 || rows < 1 || D < 1 || groups < 1 || batch > 65535) return WIDE_ERR_INVALID_ARG;
  if (rows > kI32Max || D > kI32Max || groups > kI32Max) return WIDE_ERR_INVALID_ARG;
  const int64_t M = batch * rows;
  if (M > kI32Max || D % 8 != 0 || ldx < D || ldx % 8 != 0) return WIDE_ERR_INVALID_ARG;
  if (r != 16 && r != 32 && r != 48 && r != 64) return WIDE_ERR_UNSUPPORTED;
  if (!aligned16(X) || !aligned16(W1) || !aligned16(W2) || (logits && !aligned16(logits)))
    return WIDE_ERR_INVALID_ARG;
  if (groups * r > 16384) return WIDE_ERR_UNSUPPORTED;  // W2 staged in 64 KB of LDS
  if ((uint64_t)M * (uint64_t)ldx * 2u > 0x7fffffffull || (uint64_t)r * (uint64_t)D * 2u > 0x7fffffffull)
    return WIDE_ERR_UNSUPPORTED;  // 32-bit byte offsets
  const size_t xb = span_bytes(M, D, ldx, 2), w1b = (size_t)r * D * 2, w2b = (size_t)2 * groups * r * 2;
  const size_t mb = (size_t)M * groups, lb = (size_t)M * groups * 2 * 4;
  const size_t pb = (size_t)M * groups * 4, cb = (size_t)batch * groups * 4;
  const void *ins[3] = {X, W1, W2};
  const size_t insz[3] = {xb, w1b, w2b};
  for (int i = 0; i < 3; ++i) {
    if (overlap(mask, mb, ins[i], insz[i]) || (logits && overlap(logits, lb, ins[i], insz[i])) ||
        (perm && (overlap(perm, pb, ins[i], insz[i]) || overlap(counts, cb, ins[i], insz[i]))))
      return WIDE_ERR_INVALID_ARG;
  }
  if ((logits && overlap(logits, lb, mask, mb)) ||
      (perm && (overlap(perm, pb, mask, mb) || overlap(counts, cb, mask, mb) || overlap(counts, cb, perm, pb) ||
                (logits && (overlap(perm, pb, logits, lb) || overlap(counts, cb, logits, lb))))))
    return WIDE_ERR_INVALID_ARG;
  if (!device_ok()) return WIDE_ERR_NO_DEVICE;
  wide::RouterArgs a{X, ldx, W1, W2, (int)M, (int)D, (int)r, (int)groups, (int)batch, (int)rows,
                     mask, logits, perm, counts};
  return wide::launch_router(a, reinterpret_cast<hipStream_t>(stream));
}

int wide_mfma_probe(int64_t blocks, int64_t iters, float *sink, wide_stream_t stream) {
  if (!sink || blocks < 1 || iters < 1 || blocks > 65535 || iters > (1 << 24)) return WIDE_ERR_INVALID_ARG;
  if (!device_ok()) return WIDE_ERR_NO_DEVICE;
  return wide::launch_mfma_probe((int)blocks, (int)iters, sink, reinterpret_cast<hipStream_t>(stream));
}

size_t wide_attn_workspace_bytes(int64_t B, int64_t Tq, int64_t Tk, int64_t Hq, int64_t Hk,
                                 int64_t d) {
  if (B < 1 || Tq < 1 || Tk < 1 || Hq < 1 || Hk < 1 || d < 1) return 0;
  return wide::attn_workspace_bytes(B, Tq, Tk, Hq, Hk, d);
}

}  // extern "C"

namespace {

// Validates and launches attention. builtin: the decode scratch is this
// device's built-in array (workspace arguments ignored); sizes that need more
// than it holds are refused.
int attn_impl(const wide_bf16 *Q, const wide_bf16 *K, const wide_bf16 *V, void *O, int o_dtype, int64_t B,
              int64_t Tq, int64_t Tk, int64_t Hq, int64_t Hk, int64_t groups, int64_t d, int causal, float scale,
              const int32_t *leftpad, const int32_t *perm, const int32_t *counts, const uint8_t *mask,
              void *workspace, size_t workspace_bytes, bool builtin, wide_stream_t stream) {
  if (!Q || !K || !V || !O) return WIDE_ERR_INVALID_ARG;
  if (B < 1 || Tq < 1 || Tk < 1 || Hq < 1 || Hk < 1 || d < 1) return WIDE_ERR_INVALID_ARG;
  if (B > 65535 || Hq > 65535 || Tq > kI32Max || Tk > kI32Max) return WIDE_ERR_INVALID_ARG;
  if (Hq % Hk != 0 || Tk < Tq || !valid_dtype(o_dtype)) return WIDE_ERR_INVALID_ARG;
  if (groups < Hk || groups % Hk != 0 || Hq % groups != 0) return WIDE_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return WIDE_ERR_INVALID_ARG;
  if (!(scale >= 0.f) || !isfinite(scale)) return WIDE_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return WIDE_ERR_INVALID_ARG;
  if (Tq > 1 && (!perm || !counts)) return WIDE_ERR_INVALID_ARG;
  if (Tq == 1 && !perm && !mask) return WIDE_ERR_INVALID_ARG;
  if (Tq == 1 && perm && !counts) return WIDE_ERR_INVALID_ARG;
  const size_t need = wide::attn_workspace_bytes(B, Tq, Tk, Hq, Hk, d);
  if (builtin) {
    if (need > wide::kAttnScratchBytes) return WIDE_ERR_TOO_LARGE;
    workspace = nullptr;  // taken below, once every other argument has passed
  } else if (need > 0 && (workspace == nullptr || workspace_bytes < need)) {
    return WIDE_ERR_INVALID_ARG;
  }
  const size_t ob = (size_t)B * Tq * Hq * d * (o_dtype == WIDE_DTYPE_F32 ? 4 : 2);
  const size_t qb = (size_t)B * Tq * Hq * d * 2, kb = (size_t)B * Tk * Hk * d * 2;
  if (overlap(O, ob, Q, qb) || overlap(O, ob, K, kb) || overlap(O, ob, V, kb))
    return WIDE_ERR_INVALID_ARG;
  if (!builtin && need > 0 &&
      (overlap(workspace, need, O, ob) || overlap(workspace, need, Q, qb) || overlap(workspace, need, K, kb) ||
       overlap(workspace, need, V, kb)))
    return WIDE_ERR_INVALID_ARG;
  if (d != 128) return WIDE_ERR_UNSUPPORTED;
  // Per-sequence Q/K/V are addressed with 32-bit byte offsets.
  if ((uint64_t)Tq * Hq * d * 2u > 0x7fffffffull || (uint64_t)Tk * Hk * d * 2u > 0x7fffffffull)
    return WIDE_ERR_UNSUPPORTED;
  // Decoding merges at most 4096 splits of 64 keys.
  if (Tq == 1 && (Hq / Hk > 16 || Tk > 4096 * 64)) return WIDE_ERR_UNSUPPORTED;
  if (!device_ok()) return WIDE_ERR_NO_DEVICE;
  if (builtin && need > 0) {
    int st = WIDE_OK;
    workspace = wide::attn_scratch(&st);
    if (st != WIDE_OK) return st;
  }
  wide::AttnArgs a{};
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.o_f32 = o_dtype == WIDE_DTYPE_F32;
  a.B = (int)B;
  a.Tq = (int)Tq;
  a.Tk = (int)Tk;
  a.Hq = (int)Hq;
  a.Hk = (int)Hk;
  a.NG = (int)groups;
  a.d = (int)d;
  a.causal = causal;
  a.scale = scale == 0.f ? 1.0f / sqrtf((float)d) : scale;
  a.leftpad = leftpad;
  a.perm = perm;
  a.counts = counts;
  a.mask = perm ? nullptr : mask;
  a.workspace = workspace;
  return wide::launch_attn(a, reinterpret_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

int wide_attn_grouped(const wide_bf16 *Q, const wide_bf16 *K, const wide_bf16 *V, void *O, int o_dtype,
                      int64_t B, int64_t Tq, int64_t Tk, int64_t Hq, int64_t Hk, int64_t groups, int64_t d,
                      int causal, float scale, const int32_t *leftpad, const int32_t *perm,
                      const int32_t *counts, const uint8_t *mask, void *workspace, size_t workspace_bytes,
                      wide_stream_t stream) {
  return attn_impl(Q, K, V, O, o_dtype, B, Tq, Tk, Hq, Hk, groups, d, causal, scale, leftpad, perm, counts, mask,
                   workspace, workspace_bytes, false, stream);
}

int wide_attn_noalloc(const wide_bf16 *Q, const wide_bf16 *K, const wide_bf16 *V, void *O, int o_dtype,
                      int64_t B, int64_t Tq, int64_t Tk, int64_t Hq, int64_t Hk, int64_t d, int causal,
                      float scale, const int32_t *leftpad, const int32_t *perm, const int32_t *counts,
                      const uint8_t *mask, wide_stream_t stream) {
  return attn_impl(Q, K, V, O, o_dtype, B, Tq, Tk, Hq, Hk, Hk, d, causal, scale, leftpad, perm, counts, mask,
                   nullptr, 0, true, stream);
}

int wide_attn(const wide_bf16 *Q, const wide_bf16 *K, const wide_bf16 *V, void *O, int o_dtype,
              int64_t B, int64_t Tq, int64_t Tk, int64_t Hq, int64_t Hk, int64_t d, int causal,
              float scale, const int32_t *leftpad, const int32_t *perm, const int32_t *counts,
              const uint8_t *mask, void *workspace, size_t workspace_bytes,
              wide_stream_t stream) {
  return wide_attn_grouped(Q, K, V, O, o_dtype, B, Tq, Tk, Hq, Hk, Hk, d, causal, scale, leftpad, perm,
                           counts, mask, workspace, workspace_bytes, stream);
}

}  // extern "C"
