// GEMM-MN on gfx950: the N-axis routed projections (W_q, W_gate, W_up).
//
// WIDE (arXiv 2607.28418), Figure 1 and Appendix B, Algorithm 2: C = A B^T
// with N cut into groups of G output features; token m computes group g only
// if its mask keeps it. After the reorder the rows that keep group g are the
// first counts[g] entries of perm[g], so a workgroup owning the tile (sorted
// rows s0 .. s0+256 of group g, features n0 .. n0+BN) sees only active rows
// except in the last tile of the group:
//   level 0: a tile with s0 >= counts[g] exits before touching memory;
//   level 1: A rows past counts[g] are never loaded (their offsets are out of
//            range, so the buffer loads move no data and leave zeros);
// and every other row is a full MFMA row. The rows are gathered through perm
// straight from the original activation layout (the gather is just the
// per-lane load offset) and the outputs scattered back through it, so no
// activation is ever copied. Level 2 (skipping MFMA fragments) only matters
// in the one partial tile per group and is not taken.
//
// The tile runs on the shared MFMA main loop: 256 sorted rows x BN weight
// rows, BN = 256 or 320 (8 waves) when the group size is a multiple of it,
// else 128 or 64 (4 waves); the scheduled 256-wide tiles take 320 sorted rows.
// The fused SwiGLU variant stages BN/2 gate rows and the matching BN/2 up
// rows (BN = 256 when G is a multiple of 128) and writes BN/2 outputs.
//
// With a caller workspace the active tiles are scheduled on the device: every
// workgroup derives the same numbering of the active tiles from counts
// (group by group, each XCD a contiguous range), and when they leave a last
// round on the compute units at most half full, the tiles of that round are
// split along K (the page's split-K variant of Algorithm 2) and a fixup
// kernel sums the slices in a fixed order before the epilogue.
//
// For M <= 4 with no reorder (decode steps of up to four sequences), a
// matrix-vector kernel reads the mask bytes directly and streams only the
// active groups' weight rows, with x shared through LDS.
#include "common.hpp"
#include "launch.hpp"
#include "mma_engine.hpp"

namespace wide {

template <bool OUT_F32>
__device__ __forceinline__ void store_out(void *C, size_t idx, float v) {
  if (OUT_F32)
    reinterpret_cast<float *>(C)[idx] = v;
  else
    reinterpret_cast<uint16_t *>(C)[idx] = f2bf(v);
}

// Four consecutive outputs; vector stores when the row start allows them.
template <bool OUT_F32>
__device__ __forceinline__ void store_out4(void *C, size_t idx, const f32x4 &v, bool vec) {
  if (vec) {
    if (OUT_F32)
      *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(C) + idx) = v;
    else
      *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(C) + idx) =
          u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) store_out<OUT_F32>(C, idx + e, v[e]);
  }
}

template <class S, bool SPLIT>
struct MnLoader {
  static constexpr int kDsReads = 0;
  // SwiGLU tiles run faster with the next stage's loads packed at the start
  // of the step; plain tiles with them spread (both measured)
  static constexpr int kLoadGap = SPLIT ? 1 : 0;
  static constexpr int kWideAGroups = 2;
  rsrc_t ar, br0, br1, none;
  uint32_t aoff[S::AI], boff[S::BI];
  int nk, kb, K, wave;  // steps kb .. kb + nk - 1 of K
  int kchunk;  // first k (elements) of this lane's 16-byte chunk within a stage

  __device__ __forceinline__ void prefetch(int) const {}

  __device__ __forceinline__ void operator()(int t, eng::lds_u16 *sa, eng::lds_u16 *sb) const {
    const bool live = t < nk;
    const uint32_t k0 = (uint32_t)(t + kb) * eng::kBK * 2u;
    // K tail: a chunk at or past K is loaded out of range (zeros)
    const bool in = (t + kb) * eng::kBK + kchunk < K;
    const rsrc_t ra = live ? ar : none;
#pragma unroll
    for (int i = 0; i < S::AI; ++i) eng::load_lds(ra, eng::load_dst<S::WAVES>(sa, wave, i), in ? aoff[i] : kOffNone, k0);
#pragma unroll
    for (int i = 0; i < S::BI; ++i) {
      // split tiles: the first half of the B rows are gate rows, the rest up rows
      const rsrc_t rb = live ? ((SPLIT && i >= S::BI / 2) ? br1 : br0) : none;
      eng::load_lds(rb, eng::load_dst<S::WAVES>(sb, wave, i), in ? boff[i] : kOffNone, k0);
    }
  }
};

// ---- Device-side schedule of the active tiles (workspace path) ----------
//
// The active tiles are known only on the device (counts are never read on the
// host), so every workgroup derives the same schedule from counts: group g
// has ceil(counts[g] / BM) row tiles (BM = 256 or 320 rows) times
// ceil(G / BN_OUT) column tiles, numbered group by group (row tile major,
// column tile minor, so the column tiles of one row tile, which gather the
// same rows, are neighbours). With A active
// tiles on C compute units (one tile workgroup per CU), the A mod C tiles of
// the last round (all A when A < C) are split into S = min(C / L, 8,
// K-steps / 8) slices of K when they fill at most half of it (S >= 2), so
// that round takes about 1/S of a tile's time. Workgroup p < W (W whole
// tiles) takes whole tile xcd_remap(p, W) (each XCD a contiguous range);
// workgroup W + q takes slice q % S of split tile W + q / S. Every slice
// writes its fp32 partial tile to the workspace, and gemm_mn_fixup_kernel
// sums the slices in slice order and applies the epilogue.
//
// Workspace layout: int4 header {L, S, W, 0}; int4 {g, s0, n0, counts[g]}
// per split tile; from kMnHdrBytes on, the partial tiles [slot][slice][BM][BN].
constexpr int kMnHdrInts = 4 * (1 + 1024);
constexpr int kMaxSlices = 8;  // K slices per split tile
constexpr int kFixRows = 16;   // rows of a split tile per fixup workgroup
constexpr size_t kMnHdrBytes = kMnHdrInts * sizeof(int);

struct MnPlan {
  int A, W, L, S;
};

// Exclusive prefix of v over the workgroup; `total` receives the sum.
// `tmp` holds one int per wave.
template <int THREADS>
__device__ __forceinline__ int block_excl_scan(int v, int &total, int *tmp) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) tmp[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < THREADS / kWave; ++w) {
    const int t = tmp[w];
    before += w < wave ? t : 0;
    tot += t;
  }
  total = tot;
  __syncthreads();
  return before + x - v;
}

// Thread t owns groups [t per, (t + 1) per); returns the schedule and this
// thread's (first tile, tile count).
template <int THREADS, int BM>
__device__ __forceinline__ MnPlan mn_plan(const MnArgs &a, int ntg, int nk, int *tmp, int &first, int &mine) {
  const int NG = a.N / a.G;
  const int per = (NG + THREADS - 1) / THREADS;
  const int g0 = min((int)threadIdx.x * per, NG), g1 = min(g0 + per, NG);
  mine = 0;
  for (int g = g0; g < g1; ++g) mine += (a.counts[g] + BM - 1) / BM * ntg;
  MnPlan p;
  first = block_excl_scan<THREADS>(mine, p.A, tmp);
  const int C = a.cus;
  p.L = p.A % C;
  p.S = 1;
  if (p.L > 0 && 2 * p.L <= C) p.S = min(min(C / p.L, kMaxSlices), nk / 8);
  if (p.S < 2) {
    p.S = 1;
    p.L = 0;
  }
  p.W = p.A - p.L;
  return p;
}

// The (group, index within the group) of logical tile j < A; one thread finds
// it, the result is read back from LDS.
template <int BM>
__device__ __forceinline__ void mn_find(const MnArgs &a, int ntg, int j, int first, int mine, int *out) {
  if (j >= first && j < first + mine) {
    const int NG = a.N / a.G;
    const int per = (NG + blockDim.x - 1) / blockDim.x;
    int acc = first;
    for (int g = min((int)threadIdx.x * per, NG); g < NG; ++g) {
      const int tg = (a.counts[g] + BM - 1) / BM * ntg;
      if (j < acc + tg) {
        out[0] = g;
        out[1] = j - acc;
        break;
      }
      acc += tg;
    }
  }
  __syncthreads();
}

template <int BN, int W, int BM, bool SWIGLU, bool OUT_F32, bool SCHED>
__global__ __launch_bounds__(64 * W) void gemm_mn_kernel(MnArgs a) {
  using S = eng::Shape<BN, W, BM>;
  constexpr int BN_OUT = SWIGLU ? BN / 2 : BN;
  constexpr int A3 = S::STAGES == 3 ? S::A_ELEMS : 8, B3 = S::STAGES == 3 ? S::B_ELEMS : 8;
  __shared__ __attribute__((aligned(1024))) uint16_t sA0[S::A_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sB0[S::B_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sA1[S::A_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sB1[S::B_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sA2[A3];
  __shared__ __attribute__((aligned(1024))) uint16_t sB2[B3];
  __shared__ int sRows[BM];

  const int nk_all = (a.K + eng::kBK - 1) / eng::kBK;
  int n0, g, mt;
  int part = 0, nparts = 1, slot = 0;  // K slice of this workgroup; slot: split tile index
  if constexpr (SCHED) {
    __shared__ int sTmp[W + 2];
    const int ntg = (a.G + BN_OUT - 1) / BN_OUT;
    int first, mine;
    const MnPlan p = mn_plan<S::THREADS, BM>(a, ntg, nk_all, sTmp, first, mine);
    int *hdr = static_cast<int *>(a.ws);
    if (blockIdx.x == 0 && threadIdx.x == 0) *reinterpret_cast<int4 *>(hdr) = int4{p.L, p.S, p.W, 0};
    const int p_id = blockIdx.x;
    if (p_id >= p.W + p.L * p.S) return;  // no work left for this workgroup
    int j;
    if (p_id < p.W) {
      j = xcd_remap(p_id, p.W);
    } else {
      slot = (p_id - p.W) / p.S;
      part = (p_id - p.W) % p.S;
      nparts = p.S;
      j = p.W + slot;
    }
    mn_find<BM>(a, ntg, j, first, mine, sTmp + W);
    g = sTmp[W];
    const int local = sTmp[W + 1];
    mt = local / ntg;
    n0 = g * a.G + (local % ntg) * BN_OUT;
    if (nparts > 1 && part == 0 && threadIdx.x == 0)
      reinterpret_cast<int4 *>(hdr)[1 + slot] = int4{g, mt * BM, n0, a.counts[g]};
  } else {
    // column tiles: ntg per group (a group narrower than a tile gets one)
    const int ntg = (a.G + BN_OUT - 1) / BN_OUT;
    const int MT = (a.M + BM - 1) / BM, NT = (a.N / a.G) * ntg;
    int tn;
    eng::tile_of<8>(blockIdx.x, MT, NT, mt, tn);  // 8 m-tiles per raster group
    g = tn / ntg;
    n0 = g * a.G + (tn % ntg) * BN_OUT;
  }
  // outputs of this tile that belong to its group (fewer than BN_OUT when
  // the group is narrower than the tile, or in a group's last column tile)
  const int ncols = min(BN_OUT, (g + 1) * a.G - n0);
  const int cnt = a.counts[g];
  const int s0 = mt * BM;
  if (s0 >= cnt) return;  // level 0 (never taken by a scheduled tile)
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / S::WNW, wn = wave % S::WNW;
  if (tid < BM) sRows[tid] = s0 + tid < cnt ? a.perm[(size_t)g * a.M + s0 + tid] : -1;
  __syncthreads();

  MnLoader<S, SWIGLU> ld;
  ld.ar = make_rsrc(a.A, (uint64_t)a.M * a.lda * 2);
  const int brows = SWIGLU ? BN / 2 : BN;
  // weight rows past N (a narrow last group) read as zeros
  const uint64_t brange = (uint64_t)min(brows, a.N - n0) * a.ldb * 2;
  ld.br0 = make_rsrc(a.B0 + (size_t)n0 * a.ldb, brange);
  ld.br1 = make_rsrc((SWIGLU ? a.B1 : a.B0) + (size_t)n0 * a.ldb, brange);
  ld.none = make_rsrc(a.A, 0);
#pragma unroll
  for (int i = 0; i < S::AI; ++i) {
    const int r = eng::load_row<W>(wave, i, lane);
    const int phys = sRows[r];
    ld.aoff[i] = phys >= 0 ? (uint32_t)phys * (uint32_t)a.lda * 2u + eng::load_chunk_bytes(r, lane) : kOffNone;
  }
#pragma unroll
  for (int i = 0; i < S::BI; ++i) {
    const int r = eng::load_row<W>(wave, i, lane);
    const int rb = SWIGLU ? r % (BN / 2) : r;
    ld.boff[i] = (uint32_t)rb * (uint32_t)a.ldb * 2u + eng::load_chunk_bytes(r, lane);
  }
  ld.kb = part * nk_all / nparts;
  ld.nk = (part + 1) * nk_all / nparts - ld.kb;
  ld.K = a.K;
  ld.wave = wave;
  ld.kchunk = (int)(eng::load_chunk_bytes(eng::load_row<W>(wave, 0, lane), lane) / 2);

  eng::Acc<S> acc;
#pragma unroll
  for (int i = 0; i < S::FN; ++i)
#pragma unroll
    for (int j = 0; j < S::FM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  eng::mainloop<S, BN, SWIGLU>(ld.nk, ld, (eng::lds_u16 *)sA0, (eng::lds_u16 *)sB0, (eng::lds_u16 *)sA1,
                               (eng::lds_u16 *)sB1, (eng::lds_u16 *)sA2, (eng::lds_u16 *)sB2, acc, wm, wn, lane);

  // A lane holds sorted row (lane % 16) of A fragment j and features
  // 4 (lane / 16) .. +3 of B fragment i.
  if (nparts > 1) {
    // A K slice: the fp32 partial tile (stage-row order of B, gate then up
    // rows for SwiGLU) goes to the workspace for the fixup kernel.
    float *wt = reinterpret_cast<float *>(static_cast<char *>(a.ws) + kMnHdrBytes) +
                ((size_t)slot * nparts + part) * (size_t)(BM * BN);
#pragma unroll
    for (int j = 0; j < S::FM; ++j) {
      float *wrow = wt + (size_t)(wm * S::TM + j * 16 + lane % 16) * BN + 4 * (lane / 16);
#pragma unroll
      for (int i = 0; i < S::FN; ++i)
        *reinterpret_cast<f32x4 *>(wrow + eng::b_frag_row<S, BN, SWIGLU>(wn, i)) = acc[i][j];
    }
    return;
  }
  // Scatter through perm.
  const bool vec = a.ldc % 4 == 0 && reinterpret_cast<uintptr_t>(a.C) % 16 == 0;
#pragma unroll
  for (int j = 0; j < S::FM; ++j) {
    const int phys = sRows[wm * S::TM + j * 16 + lane % 16];
    if (phys < 0) continue;
    const size_t rowoff = (size_t)phys * a.ldc;
    if (SWIGLU) {
#pragma unroll
      for (int i = 0; i < S::FN / 2; ++i) {
        const int col = wn * (S::TN / 2) + i * 16 + 4 * (lane / 16);
        if (col >= ncols) continue;
        const f32x4 gt = acc[i][j], up = acc[i + S::FN / 2][j];
        const f32x4 h = {silu(gt[0]) * up[0], silu(gt[1]) * up[1], silu(gt[2]) * up[2], silu(gt[3]) * up[3]};
        store_out4<OUT_F32>(a.C, rowoff + n0 + col, h, vec);
      }
    } else {
#pragma unroll
      for (int i = 0; i < S::FN; ++i) {
        const int col = wn * S::TN + i * 16 + 4 * (lane / 16);
        if (col >= ncols) continue;
        store_out4<OUT_F32>(a.C, rowoff + n0 + col, acc[i][j], vec);
      }
    }
  }
}

// Second pass of the K-split tiles: for every active row of a split tile,
// sums the slices' partials in slice order, applies the epilogue (SwiGLU or
// none) and scatters through perm. kFixRows rows per workgroup (16
// workgroups per split tile), one thread per 4 consecutive outputs, the
// loads of all slices issued before the sum.
template <int BN, int BM, bool SWIGLU, bool OUT_F32>
__global__ __launch_bounds__(256) void gemm_mn_fixup_kernel(MnArgs a) {
  constexpr int BN_OUT = SWIGLU ? BN / 2 : BN, Q = BN_OUT / 4, PER_TILE = BM / kFixRows;
  constexpr size_t TILE = (size_t)BM * BN;
  const int *hdr = static_cast<const int *>(a.ws);
  const int4 h = *reinterpret_cast<const int4 *>(hdr);
  const int L = h.x, S = h.y;
  const int slot = blockIdx.x / PER_TILE, rb = blockIdx.x % PER_TILE;
  if (slot >= L) return;
  const int4 info = reinterpret_cast<const int4 *>(hdr)[1 + slot];
  const int g = info.x, s0 = info.y, n0 = info.z, cnt = info.w;
  const int ncols = min(BN_OUT, (g + 1) * a.G - n0);
  const float *base = reinterpret_cast<const float *>(static_cast<const char *>(a.ws) + kMnHdrBytes) +
                      (size_t)slot * S * TILE;
  const bool vec = a.ldc % 4 == 0 && reinterpret_cast<uintptr_t>(a.C) % 16 == 0;
  for (int e = threadIdx.x; e < kFixRows * Q; e += 256) {
    const int r = rb * kFixRows + e / Q, q = e % Q;
    if (s0 + r >= cnt || 4 * q >= ncols) continue;
    const int phys = a.perm[(size_t)g * a.M + s0 + r];
    const float *src = base + (size_t)r * BN + 4 * q;
    f32x4 pv[kMaxSlices], pu[kMaxSlices];
#pragma unroll
    for (int p = 0; p < kMaxSlices; ++p) {
      if (p < S) {
        pv[p] = *reinterpret_cast<const f32x4 *>(src + p * TILE);
        if (SWIGLU) pu[p] = *reinterpret_cast<const f32x4 *>(src + p * TILE + BN / 2);
      }
    }
    f32x4 v = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < kMaxSlices; ++p) {
      if (p < S) {
        v += pv[p];
        if (SWIGLU) u += pu[p];
      }
    }
    if (SWIGLU) v = f32x4{silu(v[0]) * u[0], silu(v[1]) * u[1], silu(v[2]) * u[2], silu(v[3]) * u[3]};
    store_out4<OUT_F32>(a.C, (size_t)phys * a.ldc + n0 + 4 * q, v, vec);
  }
}

// Matrix-vector GEMM-MN for M = MT <= 4 tokens, reading the mask directly
// (no reorder). One wave per output feature n (four per workgroup, all in one
// group). A workgroup whose group is off for every token exits without
// reading its weights. Per block of 4096 reduction elements: the block of x
// of every token goes to LDS once per workgroup (direct loads, shared by the
// four waves), then each lane issues its 8 16-byte weight chunks per matrix
// (consecutive lanes, consecutive chunks: whole cache lines), and the
// products read x from LDS once it has landed. The token count is a template
// argument.
template <bool SWIGLU, bool OUT_F32, int MT>
__global__ __launch_bounds__(256) void gemv_mn_kernel(MnArgs a) {
  constexpr int U = 8;                // 16-byte chunks per lane per block
  constexpr int BLK = kWave * 8 * U;  // bf16 elements per block
  constexpr int NW = SWIGLU ? 2 * U : U;  // weight loads per block
  __shared__ __attribute__((aligned(16))) uint16_t sx[MT][BLK];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int n = blockIdx.x * 4 + wave;
  const int g = (blockIdx.x * 4) / a.G;
  const int NG = a.N / a.G;
  bool act[MT];
  bool any = false;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    act[m] = a.mask[(size_t)m * NG + g] != 0;
    any |= act[m];
  }
  if (!any) return;  // the whole group is off for every token: its weights are never read
  const int lane = threadIdx.x % kWave;
  const rsrc_t w0r = make_rsrc(a.B0 + (size_t)n * a.ldb, (uint64_t)a.K * 2);
  const rsrc_t w1r = make_rsrc((SWIGLU ? a.B1 : a.B0) + (size_t)n * a.ldb, (uint64_t)a.K * 2);
  float s0[MT], s1[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) s0[m] = s1[m] = 0.f;
  for (int k0 = 0; k0 < a.K; k0 += BLK) {
    if (k0 > 0) __syncthreads();  // every wave is done with the previous block of x
    // x -> LDS: instruction (m, u), u = wave, wave + 4, moves chunks 64 u .. 64 u + 63
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const rsrc_t xr = make_rsrc(a.A + (size_t)m * a.lda, (uint64_t)a.K * 2);
#pragma unroll
      for (int i = 0; i < U / 4; ++i) {
        const int u = wave + 4 * i;
        const int k = k0 + (u * kWave + lane) * 8;
        eng::load_lds(xr, (eng::lds_u16 *)&sx[m][u * kWave * 8], act[m] && k < a.K ? (uint32_t)k * 2u : kOffNone,
                      0u);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    u32x4 w0[U], w1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + (u * kWave + lane) * 8;
      const uint32_t off = k < a.K ? (uint32_t)k * 2u : kOffNone;
      w0[u] = buf_ld16(w0r, off);
      if (SWIGLU) w1[u] = buf_ld16(w1r, off);
    }
    __builtin_amdgcn_sched_barrier(0);
    WIDE_WAIT_VM_LGKM0(NW);  // this wave's x loads have landed; its weights may still be in flight
    __syncthreads();         // and every other wave's
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const u32x4 x = *(const WIDE_LDS u32x4 *)((const WIDE_LDS uint16_t *)&sx[m][0] + (u * kWave + lane) * 8);
        s0[m] = dot8(w0[u], x, s0[m]);
        if (SWIGLU) s1[m] = dot8(w1[u], x, s1[m]);
      }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (!act[m]) continue;
    const float g0 = wave_sum(s0[m]);
    float out = g0;
    if (SWIGLU) out = silu(g0) * wave_sum(s1[m]);
    if (lane == 0) store_out<OUT_F32>(a.C, (size_t)m * a.ldc + n, out);
  }
}

// Rows of the scheduled tile: 320 for the 256-wide 8-wave tiles (1.25x the
// MFMAs of a 256-row step for 1.125x its stage loads; measured on MI355X:
// fused gate/up of the Qwen3-14B layer 1.34 -> 1.27 ms), else 256. The
// unscheduled raster keeps 256 rows (measured 1.34 against 1.36 ms there).
constexpr int sched_bm(int BN, int W) { return BN == 256 && W == 8 ? 320 : 256; }

template <int BN, int W, bool SWIGLU, bool F32>
static void launch_tiled(const MnArgs &a, hipStream_t s) {
  constexpr int BN_OUT = SWIGLU ? BN / 2 : BN;
  const int ntg = (a.G + BN_OUT - 1) / BN_OUT;
  if (a.ws != nullptr) {
    // every schedule has at most tiles - L + C <= tiles + C work items, and
    // at most C / 2 split tiles
    constexpr int BM = sched_bm(BN, W);
    const int tiles = (a.N / a.G) * ntg * ((a.M + BM - 1) / BM);
    hipLaunchKernelGGL((gemm_mn_kernel<BN, W, BM, SWIGLU, F32, true>), dim3(tiles + a.cus), dim3(64 * W), 0, s, a);
    hipLaunchKernelGGL((gemm_mn_fixup_kernel<BN, BM, SWIGLU, F32>), dim3((BM / kFixRows) * max(a.cus / 2, 1)),
                       dim3(256), 0, s, a);
  } else {
    const int tiles = (a.N / a.G) * ntg * ((a.M + eng::kBM - 1) / eng::kBM);
    hipLaunchKernelGGL((gemm_mn_kernel<BN, W, eng::kBM, SWIGLU, F32, false>), dim3(tiles), dim3(64 * W), 0, s, a);
  }
}

template <bool SWIGLU, bool F32>
static void launch_gemv(const MnArgs &a, hipStream_t s) {
  const dim3 grid(a.N / 4), block(256);
  switch (a.M) {
    case 1: hipLaunchKernelGGL((gemv_mn_kernel<SWIGLU, F32, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((gemv_mn_kernel<SWIGLU, F32, 2>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((gemv_mn_kernel<SWIGLU, F32, 3>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((gemv_mn_kernel<SWIGLU, F32, 4>), grid, block, 0, s, a); break;
  }
}

// Output tile width BN of the tiled kernel chosen for a group size.
static int tile_bn(int G, bool swiglu) {
  if (swiglu) return G % 128 == 0 ? 256 : 128;
  if (G % 256 == 0) return 256;
  if (G % 320 == 0) return 320;
  return G % 128 == 0 ? 128 : 64;
}


// Fused SwiGLU over groups that are a multiple of 64 but not of 128 features
// runs the static raster even with a workspace: a group's row tiles then span
// about the same token windows as the other groups', and the raster runs
// tiles of several groups over one window together, which share those X rows
// in L2 (measured on MI355X, Qwen3-14B gate/up at G = 64 and 50%: 1.51 ms
// against 1.70 scheduled; a scheduled 8-wave 448 x 128 tile took 1.62).
static bool raster_only(int G, bool swiglu) { return swiglu && G % 128 != 0 && G % 64 == 0; }

size_t gemm_mn_workspace_bytes(int M, int N, int K, int G, bool swiglu) {
  (void)M;
  (void)N;
  const int nk = (K + eng::kBK - 1) / eng::kBK;
  const int cus = cu_count();
  if (nk / 8 < 2 || cus > 1024) return 0;  // no slice plan: the unscheduled path runs
  if (raster_only(G, swiglu)) return 0;
  const int bn = tile_bn(G, swiglu);
  return kMnHdrBytes + (size_t)cus * sched_bm(bn, bn >= 256 ? 8 : 4) * bn * sizeof(float);
}

int launch_gemm_mn(const MnArgs &a0, hipStream_t s) {
  MnArgs a = a0;
  const bool swiglu = a.B1 != nullptr;
  a.cus = cu_count();
  const size_t need = gemm_mn_workspace_bytes(a.M, a.N, a.K, a.G, swiglu);
  if (need == 0 || a.ws_bytes < need) a.ws = nullptr;  // also for raster_only shapes
  if (a.perm == nullptr) {
    if (swiglu) {
      if (a.c_f32) launch_gemv<true, true>(a, s); else launch_gemv<true, false>(a, s);
    } else {
      if (a.c_f32) launch_gemv<false, true>(a, s); else launch_gemv<false, false>(a, s);
    }
  } else if (swiglu && a.G % 128 == 0) {  // 128 gate + 128 up rows: one group per tile
    if (a.c_f32) launch_tiled<256, 8, true, true>(a, s); else launch_tiled<256, 8, true, false>(a, s);
  } else if (swiglu) {
    if (a.c_f32) launch_tiled<128, 4, true, true>(a, s); else launch_tiled<128, 4, true, false>(a, s);
  } else if (a.G % 256 == 0) {
    if (a.c_f32) launch_tiled<256, 8, false, true>(a, s); else launch_tiled<256, 8, false, false>(a, s);
  } else if (a.G % 320 == 0) {
    if (a.c_f32) launch_tiled<320, 8, false, true>(a, s); else launch_tiled<320, 8, false, false>(a, s);
  } else if (a.G % 128 == 0) {
    if (a.c_f32) launch_tiled<128, 4, false, true>(a, s); else launch_tiled<128, 4, false, false>(a, s);
  } else {
    if (a.c_f32) launch_tiled<64, 4, false, true>(a, s); else launch_tiled<64, 4, false, false>(a, s);
  }
  return check_launch();
}

}  // namespace wide
