// GEMM-MN on gfx950: the N-axis routed projection (W_q, W_gate, W_up).
//
// WIDE (arXiv 2607.28418) Figure 1 and Appendix B, Algorithm 2: C = A B^T with
// N cut into groups of G output features; token m computes group g only if its
// mask says so. After the reorder, the rows that keep group g are the first
// counts[g] entries of perm[g], so a workgroup owning the tile (sorted rows
// m0..m0+BM, features n0..n0+BN) with BN | G sees one group and, except for
// at most one boundary tile per group, only fully active rows:
//   level 0: a tile with m0 >= counts[g] exits before touching memory;
//   level 1: A rows past counts[g] are not loaded (zero-filled in LDS);
//   level 2: 16-row MFMA fragments past counts[g] are not issued (the test is
//            on a scalar, so it is a uniform branch, not a lane vote).
// The A rows are gathered through perm straight from the original layout and
// the outputs scattered back through it, so no activation is ever copied.
//
// Tile: 128 sorted rows x 128 B rows (BN = 128 features, or 64 gate + 64 up
// features for the fused SwiGLU variant), BK = 64, 4 waves in a 2 x 2 layout,
// v_mfma_f32_16x16x32_bf16, LDS double-buffered with one barrier per K step.
// Workgroups are remapped so that the row tiles of one feature tile run on the
// same XCD and share its B tile in that XCD's L2.
//
// For M <= 4 with no reorder (one decode step), a matrix-vector kernel reads
// the mask bytes directly and streams only the active groups' weight rows.
#include "common.hpp"
#include "launch.hpp"

namespace wide {

constexpr int kMnBM = 128;
constexpr int kMnBK = 64;
constexpr int kMnLds = kMnBK + 8;  // LDS row stride in bf16 (16-byte pad)
constexpr int kMnThreads = 256;

template <bool OUT_F32>
__device__ __forceinline__ void store_out(void *C, size_t idx, float v) {
  if (OUT_F32)
    reinterpret_cast<float *>(C)[idx] = v;
  else
    reinterpret_cast<uint16_t *>(C)[idx] = f2bf(v);
}

template <int BNT, bool SWIGLU, bool OUT_F32>
__global__ __launch_bounds__(kMnThreads, 2) void gemm_mn_kernel(MnArgs a) {
  constexpr int BN_OUT = SWIGLU ? BNT / 2 : BNT;
  constexpr int WN = BNT / 2;                 // B-tile rows per wave
  constexpr int NF = WN / 16;                 // column fragments per wave
  constexpr int MF = 4;                       // row fragments per wave (64 rows)
  constexpr int A_PASSES = kMnBM * 8 / kMnThreads;
  constexpr int B_PASSES = BNT * 8 / kMnThreads;
  static_assert(!SWIGLU || BNT == 128, "SwiGLU tiles pair 64 gate and 64 up rows");

  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kMnBM * kMnLds];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BNT * kMnLds];
  __shared__ int sRows[kMnBM];

  const int n_tiles = a.N / BN_OUT;
  const int m_tiles = (a.M + kMnBM - 1) / kMnBM;
  const int L = xcd_remap(blockIdx.x, n_tiles * m_tiles);
  const int n0 = (L / m_tiles) * BN_OUT;
  const int m0 = (L % m_tiles) * kMnBM;
  const int g = n0 / a.G;
  const int cnt = a.counts[g];
  if (m0 >= cnt) return;  // level 0: this tile and every later one of group g are inactive
  const int rows = min(kMnBM, cnt - m0);

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;

  if (tid < kMnBM) sRows[tid] = tid < rows ? a.perm[(size_t)g * a.M + m0 + tid] : 0;
  __syncthreads();

  const int chunk = tid % 8;
  const int rbase = tid / 8;
  // Gathered A rows and the B tile as buffer resources: rows past the count
  // and the K tail get out-of-range offsets (zeros, no memory traffic), so
  // every load is issued unconditionally.
  const rsrc_t ra_rsrc = make_rsrc(a.A, (uint64_t)a.M * a.lda * 2);
  uint32_t a_off[A_PASSES];
#pragma unroll
  for (int p = 0; p < A_PASSES; ++p) {
    const int r = rbase + 32 * p;
    // level 1: rows past the count are never fetched
    a_off[p] = r < rows ? (uint32_t)(sRows[r] * a.lda + chunk * 8) * 2u : kOffNone;
  }
  rsrc_t rb_rsrc[2];
  rb_rsrc[0] = make_rsrc(a.B0 + (size_t)n0 * a.ldb, (uint64_t)(SWIGLU ? BNT / 2 : BNT) * a.ldb * 2);
  rb_rsrc[1] = SWIGLU ? make_rsrc(a.B1 + (size_t)n0 * a.ldb, (uint64_t)(BNT / 2) * a.ldb * 2) : rb_rsrc[0];
  uint32_t b_off[B_PASSES];
#pragma unroll
  for (int p = 0; p < B_PASSES; ++p) {
    const int br = rbase + 32 * p;
    const int lr = (SWIGLU && br >= BNT / 2) ? br - BNT / 2 : br;
    b_off[p] = (uint32_t)(lr * a.ldb + chunk * 8) * 2u;
  }

  const int nk = (a.K + kMnBK - 1) / kMnBK;
  u32x4 ra[A_PASSES], rb[B_PASSES];
  auto gload = [&](int kt) {
    const bool kin = kt * kMnBK + chunk * 8 < a.K;
    const uint32_t kb = (uint32_t)(kt * kMnBK) * 2u;
#pragma unroll
    for (int p = 0; p < A_PASSES; ++p) ra[p] = buf_ld16(ra_rsrc, kin ? a_off[p] + kb : kOffNone);
#pragma unroll
    for (int p = 0; p < B_PASSES; ++p) {
      const int which = (SWIGLU && rbase + 32 * p >= BNT / 2) ? 1 : 0;
      rb[p] = buf_ld16(which ? rb_rsrc[1] : rb_rsrc[0], kin ? b_off[p] + kb : kOffNone);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < A_PASSES; ++p) st16(&sA[buf][(rbase + 32 * p) * kMnLds + chunk * 8], ra[p]);
#pragma unroll
    for (int p = 0; p < B_PASSES; ++p) st16(&sB[buf][(rbase + 32 * p) * kMnLds + chunk * 8], rb[p]);
  };
  auto brow = [&](int j) -> int {
    if (SWIGLU) return (j < NF / 2) ? wn * 32 + 16 * j : 64 + wn * 32 + 16 * (j - NF / 2);
    return wn * WN + 16 * j;
  };

  f32x4 acc[MF][NF];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // number of live 16-row fragments of this wave (uniform)
  const int live = uniform(min(MF, max(0, (rows - wm * 64 + 15) / 16)));

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int koff = kk * 32 + (lane / 16) * 8;
      u32x4 bf[NF];
#pragma unroll
      for (int j = 0; j < NF; ++j) bf[j] = ld16(&sB[cur][(brow(j) + lane % 16) * kMnLds + koff]);
      if (live == MF) {
        // Fully active rows (every tile of a group but the last): no
        // predicate, all fragment reads issued together.
        u32x4 af[MF];
#pragma unroll
        for (int i = 0; i < MF; ++i) af[i] = ld16(&sA[cur][(wm * 64 + 16 * i + lane % 16) * kMnLds + koff]);
#pragma unroll
        for (int i = 0; i < MF; ++i)
#pragma unroll
          for (int j = 0; j < NF; ++j) acc[i][j] = mfma16x16x32(af[i], bf[j], acc[i][j]);
      } else {
#pragma unroll
        for (int i = 0; i < MF; ++i) {
          if (i < live) {  // level 2: skip fragments past the count
            const u32x4 af = ld16(&sA[cur][(wm * 64 + 16 * i + lane % 16) * kMnLds + koff]);
#pragma unroll
            for (int j = 0; j < NF; ++j) acc[i][j] = mfma16x16x32(af, bf[j], acc[i][j]);
          }
        }
      }
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: scatter active rows back to their physical positions.
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    if (i >= live) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int rl = wm * 64 + 16 * i + 4 * (lane / 16) + v;
      if (rl >= rows) continue;
      const size_t rowoff = (size_t)sRows[rl] * a.ldc;
      if (SWIGLU) {
#pragma unroll
        for (int j = 0; j < NF / 2; ++j) {
          const float gt = acc[i][j][v], up = acc[i][j + NF / 2][v];
          store_out<OUT_F32>(a.C, rowoff + n0 + wn * 32 + 16 * j + lane % 16, silu(gt) * up);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NF; ++j)
          store_out<OUT_F32>(a.C, rowoff + n0 + wn * WN + 16 * j + lane % 16, acc[i][j][v]);
      }
    }
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float dot8(const u32x4 &w, const u32x4 &x, float acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc = fmaf(bf_lo(w[e]), bf_lo(x[e]), acc);
    acc = fmaf(bf_hi(w[e]), bf_hi(x[e]), acc);
  }
  return acc;
}

// Matrix-vector GEMM-MN for M <= 4 reading the mask directly (no reorder).
// One wave per output feature n (four per workgroup, all in one group). A
// workgroup whose group is off for every token exits without reading its
// weights. The weight row is streamed in 16-byte chunks (consecutive lanes,
// consecutive chunks: whole cache lines), with a whole block of chunks per
// lane issued before any is used, so each wave keeps 8 KB per row in flight.
template <bool SWIGLU, bool OUT_F32>
__global__ __launch_bounds__(256) void gemv_mn_kernel(MnArgs a) {
  constexpr int U = 8;                // 16-byte chunks per lane per block
  constexpr int BLK = kWave * 8 * U;  // bf16 elements per block
  const int n = blockIdx.x * 4 + threadIdx.x / kWave;
  const int g = (blockIdx.x * 4) / a.G;
  const int NG = a.N / a.G;
  bool act[4];
  bool any = false;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    act[m] = m < a.M && a.mask[(size_t)m * NG + g] != 0;
    any |= act[m];
  }
  if (!any) return;  // the whole group is off for every token: its weights are never read
  const int lane = threadIdx.x % kWave;
  const rsrc_t w0r = make_rsrc(a.B0 + (size_t)n * a.ldb, (uint64_t)a.K * 2);
  const rsrc_t w1r = make_rsrc((SWIGLU ? a.B1 : a.B0) + (size_t)n * a.ldb, (uint64_t)a.K * 2);
  float s0[4] = {0.f, 0.f, 0.f, 0.f}, s1[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < a.K; k0 += BLK) {
    u32x4 w0[U], w1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + (u * kWave + lane) * 8;
      const uint32_t off = k < a.K ? (uint32_t)k * 2u : kOffNone;
      w0[u] = buf_ld16(w0r, off);
      if (SWIGLU) w1[u] = buf_ld16(w1r, off);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (!act[m]) continue;
      const rsrc_t xr = make_rsrc(a.A + (size_t)m * a.lda, (uint64_t)a.K * 2);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = k0 + (u * kWave + lane) * 8;
        const u32x4 x = buf_ld16(xr, k < a.K ? (uint32_t)k * 2u : kOffNone);
        s0[m] = dot8(w0[u], x, s0[m]);
        if (SWIGLU) s1[m] = dot8(w1[u], x, s1[m]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (!act[m]) continue;
    const float g0 = wave_sum(s0[m]);
    float out = g0;
    if (SWIGLU) out = silu(g0) * wave_sum(s1[m]);
    if (lane == 0) store_out<OUT_F32>(a.C, (size_t)m * a.ldc + n, out);
  }
}

template <int BNT, bool SWIGLU, bool F32>
static void launch_tiled(const MnArgs &a, hipStream_t s) {
  constexpr int BN_OUT = SWIGLU ? BNT / 2 : BNT;
  const int tiles = (a.N / BN_OUT) * ((a.M + kMnBM - 1) / kMnBM);
  hipLaunchKernelGGL((gemm_mn_kernel<BNT, SWIGLU, F32>), dim3(tiles), dim3(kMnThreads), 0, s, a);
}

template <bool SWIGLU, bool F32>
static void launch_gemv(const MnArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((gemv_mn_kernel<SWIGLU, F32>), dim3(a.N / 4), dim3(256), 0, s, a);
}

int launch_gemm_mn(const MnArgs &a, hipStream_t s) {
  const bool swiglu = a.B1 != nullptr;
  if (a.perm == nullptr) {
    if (swiglu) {
      if (a.c_f32) launch_gemv<true, true>(a, s); else launch_gemv<true, false>(a, s);
    } else {
      if (a.c_f32) launch_gemv<false, true>(a, s); else launch_gemv<false, false>(a, s);
    }
  } else if (swiglu) {
    if (a.c_f32) launch_tiled<128, true, true>(a, s); else launch_tiled<128, true, false>(a, s);
  } else if (a.G % 128 == 0) {
    if (a.c_f32) launch_tiled<128, false, true>(a, s); else launch_tiled<128, false, false>(a, s);
  } else {
    if (a.c_f32) launch_tiled<64, false, true>(a, s); else launch_tiled<64, false, false>(a, s);
  }
  return check_launch();
}

}  // namespace wide
