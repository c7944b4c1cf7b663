// GEMM-K by K-groups on gfx950: the K-axis routed projections (W_o, W_down)
// computed one active K-group at a time.
//
// WIDE (arXiv 2607.28418), Appendix B, Eq. 21 and Algorithm 3: for every
// K-group g the rows that keep it are the first counts[g] entries of perm[g]
// (the reorder of the [M][K/G] mask), so the product restricted to group g,
//   P_g = A[perm_g, K_g] B[:, K_g]^T,
// is a dense GEMM over those rows and the G columns of the group, and
// C = sum_g scatter(P_g). A workgroup owns one tile (group g, sorted rows
// s0 .. s0+255 of that group, output features n0 .. n0+BN):
//   level 0: a tile with s0 >= counts[g] exits before touching memory, so an
//            inactive (row, group) pair costs nothing;
//   level 1: rows past counts[g] in the group's last tile are never loaded
//            (out-of-range offsets: the loads move no data, leave zeros);
// and its main loop covers only the G / 64 stages of the group, on the shared
// MFMA pipeline (the pipeline is local to the group: it starts and drains
// within the tile, as in the page). The partial tile is then added into C at
// the gathered rows with fp32 atomic adds, since the tiles of different groups
// reach the same entries of C in no fixed order.
//
// Workgroups are numbered group by group, so the tiles running at one time
// belong to one or two groups, whose rows rarely coincide: few atomic adds
// meet on the same entry at once (the page packs several groups into one
// workgroup for the same purpose). Within a group the raster is the XCD-aware
// one of the other tiled GEMMs.
//
// Epilogue: each wave passes its 128 x 64 block through LDS, 64 rows at a
// time, so that one atomic instruction covers 64 consecutive features of one
// row (256 contiguous bytes) rather than 4 features of 16 rows.
//
// With beta = 0 a fill kernel first zeroes C (the page's zero-initialised
// output); rows that keep no group are left at zero.
//
// Measured on MI355X (Qwen3-14B prefill, M = 8192, N = 5120, half of the
// groups kept): the partial writes bound this path. Every kept (row, group)
// pair adds N fp32 values into C, and the device sustains about 1.7 TB/s of
// such atomic adds, so o_proj (G = 640, 4 partials per row) takes 0.61 ms and
// down_proj 4.3 ms at G = 256 (34 per row), against 0.41 and 1.16 ms for the
// mask-driven kernel of gemm_k.hip, which keeps each output tile in
// registers across all groups.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"
#include "mma_engine.hpp"

namespace wide {

namespace {

constexpr int kKgGM = 8;  // m-tiles per raster group

template <class S>
struct KgLoader {
  static constexpr int kDsReads = 0;
  static constexpr int kLoadGap = 0;
  static constexpr int kWideAGroups = 2;
  rsrc_t ar, br, none;
  uint32_t aoff[S::AI], boff[S::BI];
  uint32_t kbyte0;  // byte offset of the group's first column
  int nk, wave;

  __device__ __forceinline__ void prefetch(int) const {}

  __device__ __forceinline__ void operator()(int t, eng::lds_u16 *sa, eng::lds_u16 *sb) const {
    const bool live = t < nk;
    const uint32_t k0 = kbyte0 + (uint32_t)t * eng::kBK * 2u;
    const rsrc_t ra = live ? ar : none, rb = live ? br : none;
#pragma unroll
    for (int i = 0; i < S::AI; ++i) eng::load_lds(ra, eng::load_dst<S::WAVES>(sa, wave, i), aoff[i], k0);
#pragma unroll
    for (int i = 0; i < S::BI; ++i) eng::load_lds(rb, eng::load_dst<S::WAVES>(sb, wave, i), boff[i], k0);
  }
};

// C[0:M][0:N] = 0, four features per thread (N % 4 == 0, ldc % 4 == 0).
__global__ __launch_bounds__(256) void fill_zero_kernel(float *C, int64_t ldc, int M, int N) {
  const int64_t q = N / 4, total = (int64_t)M * q;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256)
    *reinterpret_cast<f32x4 *>(C + (i / q) * ldc + (i % q) * 4) = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <int BN, int W>
__global__ __launch_bounds__(64 * W) void gemm_kg_kernel(KgArgs a) {
  using S = eng::Shape<BN, W>;
  static_assert(S::TN == 64 && S::FN == 4 && S::FM == 8, "epilogue assumes 128 x 64 wave blocks");
  constexpr int A3 = S::STAGES == 3 ? S::A_ELEMS : 8, B3 = S::STAGES == 3 ? S::B_ELEMS : 8;
  __shared__ __attribute__((aligned(1024))) uint16_t sA0[S::A_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sB0[S::B_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sA1[S::A_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sB1[S::B_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sA2[A3];
  __shared__ __attribute__((aligned(1024))) uint16_t sB2[B3];
  __shared__ int sRows[eng::kBM];

  const int MT = (a.M + eng::kBM - 1) / eng::kBM, NT = a.N / BN;
  const int per_group = MT * NT;
  const int g = blockIdx.x / per_group;
  int mt, tn;
  eng::tile_of<kKgGM>(blockIdx.x % per_group, MT, NT, mt, tn);
  const int cnt = min(a.counts[g], a.M);
  const int s0 = mt * eng::kBM;
  if (s0 >= cnt) return;  // level 0
  const int n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / S::WNW, wn = wave % S::WNW;
  // a perm entry outside [0, M) is dropped, never dereferenced
  if (tid < eng::kBM) {
    const int p = s0 + tid < cnt ? a.perm[(size_t)g * a.M + s0 + tid] : -1;
    sRows[tid] = (unsigned)p < (unsigned)a.M ? p : -1;
  }
  __syncthreads();

  KgLoader<S> ld;
  ld.ar = make_rsrc(a.A, (uint64_t)a.M * a.lda * 2);
  ld.br = make_rsrc(a.B + (size_t)n0 * a.ldb, (uint64_t)BN * a.ldb * 2);
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
    ld.boff[i] = (uint32_t)r * (uint32_t)a.ldb * 2u + eng::load_chunk_bytes(r, lane);
  }
  ld.kbyte0 = (uint32_t)g * (uint32_t)a.G * 2u;
  ld.nk = a.G / eng::kBK;
  ld.wave = wave;

  eng::Acc<S> acc;
#pragma unroll
  for (int i = 0; i < S::FN; ++i)
#pragma unroll
    for (int j = 0; j < S::FM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  eng::mainloop<S, BN, false>(ld.nk, ld, (eng::lds_u16 *)sA0, (eng::lds_u16 *)sB0, (eng::lds_u16 *)sA1,
                              (eng::lds_u16 *)sB1, (eng::lds_u16 *)sA2, (eng::lds_u16 *)sB2, acc, wm, wn, lane);

  // Every wave is done with the stage buffers; each wave now owns 16 KB of
  // them (64 rows x 64 fp32 features, row-major, 16-byte chunk c of row r at
  // position c ^ (r % 16)).
  __syncthreads();
  const int pair = wave / 2;
  uint16_t *base;
  if constexpr (W == 8)
    base = pair == 0 ? sA0 : pair == 1 ? sB0 : pair == 2 ? sA1 : sB1;
  else
    base = pair == 0 ? sA0 : sA1;
  WIDE_LDS float *buf = (WIDE_LDS float *)(eng::lds_u16 *)base + (wave % 2) * 4096;
  float *crow = a.C + n0 + wn * S::TN + lane;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // A lane holds row lane % 16 of A fragment j and features
    // 4 (lane / 16) .. +3 of B fragment i.
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = jj * 16 + lane % 16;
#pragma unroll
      for (int i = 0; i < S::FN; ++i) {
        const int chunk = i * 4 + lane / 16;
        *(WIDE_LDS f32x4 *)(buf + r * 64 + ((chunk ^ (r & 15)) * 4)) = acc[i][4 * h + jj];
      }
    }
    // row r of the half: lane l takes feature l
    const int rbase = wm * S::TM + h * 64;
#pragma unroll 8
    for (int r = 0; r < 64; ++r) {
      const float v = buf[r * 64 + ((((lane / 4) ^ (r & 15))) * 4) + lane % 4];
      const int phys = sRows[rbase + r];
      if (phys >= 0) unsafeAtomicAdd(crow + (size_t)phys * a.ldc, v);
    }
  }
}

template <int BN, int W>
int launch_kg(const KgArgs &a, hipStream_t s) {
  const int MT = (a.M + eng::kBM - 1) / eng::kBM, NT = a.N / BN;
  const int64_t blocks = (int64_t)(a.K / a.G) * MT * NT;
  hipLaunchKernelGGL((gemm_kg_kernel<BN, W>), dim3((unsigned)blocks), dim3(64 * W), 0, s, a);
  return check_launch();
}

}  // namespace

int launch_gemm_kg(const KgArgs &a, hipStream_t s) {
  if (a.beta == 0) {
    const int64_t quads = (int64_t)a.M * (a.N / 4);
    const int blocks = (int)std::min<int64_t>((quads + 255) / 256, 8 * 1024);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, s, a.C, a.ldc, a.M, a.N);
    const int st = check_launch();
    if (st != WIDE_OK) return st;
  }
  return a.N % 256 == 0 ? launch_kg<256, 8>(a, s) : launch_kg<128, 4>(a, s);
}

}  // namespace wide
