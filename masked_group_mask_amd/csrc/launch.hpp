// Internal launcher declarations shared by the kernels and the C ABI layer.
// Launchers assume the C ABI layer has validated every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/wide.h"

namespace wide {

// Compute units of the current device (cached per device).
int cu_count();

inline int check_launch() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? WIDE_OK : WIDE_ERR_LAUNCH;
}

// Workgroup id -> logical tile id such that consecutive logical ids run on the
// same XCD (the dispatcher deals workgroups to the 8 XCDs round-robin), so
// tiles that share an operand share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int p, int total) {
  const int per = total / 8, rem = total % 8;
  const int x = p % 8, i = p / 8;
  return x * per + (x < rem ? x : rem) + i;
}

int launch_reorder(const uint8_t *mask, int batch, int rows, int groups, int32_t *perm,
                   int32_t *counts, hipStream_t stream);
// Stable sort of the rows by the Gray-code rank of their pattern over the
// first min(groups, 8) groups.
int launch_pattern_order(const uint8_t *mask, int rows, int groups, int32_t *order, hipStream_t stream);

struct MnArgs {
  const uint16_t *A;
  int64_t lda;
  const uint16_t *B0;  // [N][K] weights (gate for the SwiGLU variant)
  const uint16_t *B1;  // up weights for the SwiGLU variant, else null
  int64_t ldb;
  void *C;
  int64_t ldc;
  int c_f32;           // output is fp32 (else bf16)
  int M, N, K, G;
  const int32_t *perm;
  const int32_t *counts;
  const uint8_t *mask;
  // Caller's workspace (may be null). With one, the tiled path schedules the
  // active tiles on the device and splits a partly filled last round along K.
  void *ws = nullptr;
  size_t ws_bytes = 0;
  int cus = 0;  // set by the launcher: compute units of the device
};
int launch_gemm_mn(const MnArgs &a, hipStream_t stream);
// Bytes of workspace the scheduled GEMM-MN path needs on the current device
// (0 when it would never split a tile: the path then runs without one).
size_t gemm_mn_workspace_bytes(int M, int N, int K, int G, bool swiglu);

struct KArgs {
  const uint16_t *A;
  int64_t lda;
  const uint16_t *B;
  int64_t ldb;
  float *C;
  int64_t ldc;
  int beta;
  int M, N, K, G;
  const uint8_t *mask;
  // Optional permutation of the token rows (rows with equal routing patterns
  // adjacent); with it the tiles cover sorted positions and skip the work of
  // groups their rows do not keep.
  const int32_t *order;
  // Caller's workspace for the K-split tiles (may be null: then no K split).
  float *ws;
  size_t ws_bytes;
  // Set by the launcher: the tiled kernels cover logical 256 x 256 tiles
  // tile_base, tile_base + 1, ... of the raster; with split_tail each one is
  // covered by two 256 x 128 workgroups. With ksplit > 1 the tiles from
  // `head` on are each covered by ksplit workgroups that own consecutive
  // slices of the K range.
  int tile_base;
  int split_tail;
  int head;
  int ksplit;
};
int launch_gemm_k(const KArgs &a, hipStream_t stream);
// Bytes of workspace the K-split plan of an M x N x K product needs on the
// current device (0 when the plan splits nothing).
size_t gemm_k_workspace_bytes(int M, int N, int K);

// GEMM-K by K-groups: every active (group, sorted row tile) pair multiplies
// its rows over the group's G columns and adds the partial into C with
// atomics (C zeroed first when beta = 0). Needs G % 64 == 0, N % 128 == 0.
struct KgArgs {
  const uint16_t *A;
  int64_t lda;
  const uint16_t *B;
  int64_t ldb;
  float *C;
  int64_t ldc;
  int beta;
  int M, N, K, G;
  const int32_t *perm;    // [K/G][M]
  const int32_t *counts;  // [K/G]
};
int launch_gemm_kg(const KgArgs &a, hipStream_t stream);

struct AttnArgs {
  const uint16_t *Q, *K, *V;
  void *O;
  int o_f32;
  int B, Tq, Tk, Hq, Hk, d;
  int NG;  // routing groups: a multiple of Hk dividing Hq; head h is gated by group h / (Hq / NG)
  int causal;
  float scale;
  const int32_t *leftpad;
  const int32_t *perm, *counts;
  const uint8_t *mask;
  void *workspace;
};
int launch_attn(const AttnArgs &a, hipStream_t stream);
// Size of the built-in decode scratch of wide_attn_noalloc (one per device).
constexpr size_t kAttnScratchBytes = size_t(32) << 20;
// Device address of this device's built-in scratch (queried once per device);
// null with *status set on failure.
void *attn_scratch(int *status);

struct RouterArgs {
  const uint16_t *X;   // [M][ldx] bf16
  int64_t ldx;
  const uint16_t *W1;  // [r][D] bf16
  const uint16_t *W2;  // [2 groups][r] bf16
  int M, D, r, groups;
  int batch, rows;     // M = batch * rows (for the reorder)
  uint8_t *mask;       // [M][groups]
  float *logits;       // [M][2 groups] or NULL
  int32_t *perm;       // [batch][groups][rows] or NULL
  int32_t *counts;     // [batch][groups] (with perm)
};
int launch_router(const RouterArgs &a, hipStream_t stream);
size_t attn_workspace_bytes(int64_t B, int64_t Tq, int64_t Tk, int64_t Hq, int64_t Hk,
                            int64_t d);

// MFMA rate probe: `blocks` workgroups of 4 waves, `iters` rounds of 8 MFMAs
// per wave; one float per wave to sink[blocks * 4].
int launch_mfma_probe(int blocks, int iters, float *sink, hipStream_t stream);

}  // namespace wide
