// GEMM-K on gfx950: the K-axis routed projections (W_o, W_down).
//
// WIDE (arXiv 2607.28418), Appendix B, Eq. 21 and Algorithm 3:
//   C[m][n] = sum_g mask[m][g] * sum_{k in group g} A[m][k] * B[n][k].
// The page gives every (sorted row tile, K-group) pair its own pipeline and
// scatters each fp32 partial into C with atomics. Under token-level masks the
// rows a group keeps differ from group to group, so on MI355X that scatter
// (one fp32 read-add-write per active row and feature per group, through LDS
// or L2 atomics) costs more than the multiply-adds it saves while the group
// is short (G = 128 needs 2G = 256 MFMA flops per scattered value; the LDS
// moves a value in and out more slowly than that). Here C stays in registers:
//   - a workgroup owns C[m0:m0+256, n0:n0+128] in original row order and runs
//     the shared 3-stage MFMA main loop over the whole K range;
//   - the A slice of a row whose group is off for that token is never read
//     (level 1): its load offset is set out of range, the buffer load moves
//     no data and the stage holds zeros there, so the product adds exactly 0;
//   - a tile none of whose rows keeps any group writes beta*C and exits
//     (level 0);
//   - the per-row predicates come from a bit table built once per tile from
//     the mask bytes: bit r of word i of group g = row 32i + r keeps group g;
//   - the summation order is fixed, so results are reproducible bit for bit.
// For M <= 4 a matrix-vector kernel streams only the K-groups some token
// keeps.
#include "common.hpp"
#include "launch.hpp"
#include "mma_engine.hpp"

namespace wide {

constexpr int kKMaxGroups = 512;
constexpr int kKBN = 128;  // output features per tile
using KShape = eng::Shape<kKBN>;

// Builds the tile's bit table: thread t reads the mask row of tile row t and
// each wave turns one group column of its 64 rows into two words by ballot.
// Returns whether any row of the tile keeps any group. `flag` is one word of
// LDS that is free during the prologue.
__device__ __forceinline__ bool build_bits(const KArgs &a, int m0, WIDE_LDS uint32_t *bits, WIDE_LDS int *flag) {
  const int NG = a.K / a.G;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int m = m0 + tid;
  const uint8_t *row = a.mask + (size_t)m * NG;
  const bool valid = m < a.M;
  if (tid == 0) *flag = 0;
  __syncthreads();
  int any = 0;
  auto put = [&](int g, bool on) {
    const uint64_t bal = __ballot(on);
    any |= bal != 0;
    if (lane == 0) {
      bits[g * 8 + wave * 2] = (uint32_t)bal;
      bits[g * 8 + wave * 2 + 1] = (uint32_t)(bal >> 32);
    }
  };
  if (NG % 4 == 0 && reinterpret_cast<uintptr_t>(a.mask) % 4 == 0) {
    const uint32_t *row4 = reinterpret_cast<const uint32_t *>(row);
    for (int g0 = 0; g0 < NG; g0 += 32) {
      uint32_t w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = (valid && g0 + 4 * u < NG) ? row4[g0 / 4 + u] : 0u;
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (g0 + 4 * u + e < NG) put(g0 + 4 * u + e, ((w[u] >> (8 * e)) & 0xffu) != 0);
    }
  } else {
    for (int g0 = 0; g0 < NG; g0 += 8) {
      uint8_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = (valid && g0 + u < NG) ? row[g0 + u] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (g0 + u < NG) put(g0 + u, v[u] != 0);
    }
  }
  if (any && lane == 0) *flag = 1;
  __syncthreads();
  return *flag != 0;
}

// Stage loader of the tile: A rows predicated by the bit table (the
// predicates of the next stage are read one stage ahead), B rows dense.
struct KLoader {
  rsrc_t ar, br, none;
  uint32_t aoff[KShape::AI], boff[KShape::BI];
  const WIDE_LDS uint32_t *bits;
  int nk, steps_per_group, NG, wave, lane;
  uint32_t pred;  // bit i: A row of load instruction i is live at stage `next`
  int next;

  __device__ __forceinline__ uint32_t read_pred(int t) const {
    const int g = min(t / steps_per_group, NG - 1);
    const u32x4 lo = *(const WIDE_LDS u32x4 *)(bits + g * 8);
    const u32x4 hi = *(const WIDE_LDS u32x4 *)(bits + g * 8 + 4);
    const int sh = wave * 8 + lane / 8;  // row % 32 of every load instruction of this lane
    uint32_t p = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) p |= ((lo[i] >> sh) & 1u) << i;
#pragma unroll
    for (int i = 0; i < 4; ++i) p |= ((hi[i] >> sh) & 1u) << (i + 4);
    return p;
  }

  __device__ __forceinline__ void operator()(int t, eng::lds_u16 *sa, eng::lds_u16 *sb) {
    const bool live = t < nk;
    const rsrc_t ra = live ? ar : none, rb = live ? br : none;
    const uint32_t k0 = (uint32_t)t * eng::kBK * 2u;
    const uint32_t p = pred;
#pragma unroll
    for (int i = 0; i < KShape::AI; ++i)
      eng::load_lds(ra, sa + (wave + 4 * i) * 512, ((p >> i) & 1u) ? aoff[i] : kOffNone, k0);
#pragma unroll
    for (int i = 0; i < KShape::BI; ++i) eng::load_lds(rb, sb + (wave + 4 * i) * 512, boff[i], k0);
    next = t + 1;
    pred = read_pred(next);
  }
};

__global__ __launch_bounds__(eng::kThreads) void gemm_k_kernel(KArgs a) {
  __shared__ __attribute__((aligned(1024))) uint16_t sA0[eng::kBM * eng::kBK];
  __shared__ __attribute__((aligned(1024))) uint16_t sB0[kKBN * eng::kBK];
  __shared__ __attribute__((aligned(1024))) uint16_t sA1[eng::kBM * eng::kBK];
  __shared__ __attribute__((aligned(1024))) uint16_t sB1[kKBN * eng::kBK];
  __shared__ __attribute__((aligned(1024))) uint16_t sA2[eng::kBM * eng::kBK];
  __shared__ __attribute__((aligned(1024))) uint16_t sB2[kKBN * eng::kBK];
  __shared__ __attribute__((aligned(16))) uint32_t sBits[kKMaxGroups][8];

  const int MT = (a.M + eng::kBM - 1) / eng::kBM, NT = a.N / kKBN;
  int mt, tn;
  eng::tile_of(blockIdx.x, MT, NT, mt, tn);
  const int m0 = mt * eng::kBM, n0 = tn * kKBN;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int wm = wave / 2, wn = wave % 2;
  using S = KShape;

  const bool any = build_bits(a, m0, (WIDE_LDS uint32_t *)&sBits[0][0], (WIDE_LDS int *)sA2);
  f32x4 acc[S::FN][S::FM];
#pragma unroll
  for (int i = 0; i < S::FN; ++i)
#pragma unroll
    for (int j = 0; j < S::FM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (any) {  // level 0: otherwise the tile's product is exactly zero
    KLoader ld;
    const int rows = min(eng::kBM, a.M - m0);
    ld.ar = make_rsrc(a.A + (size_t)m0 * a.lda, (uint64_t)rows * a.lda * 2);  // rows past M: out of range
    ld.br = make_rsrc(a.B + (size_t)n0 * a.ldb, (uint64_t)kKBN * a.ldb * 2);
    ld.none = make_rsrc(a.A, 0);
#pragma unroll
    for (int i = 0; i < S::AI; ++i) {
      const int r = eng::load_row(wave, i, lane);
      ld.aoff[i] = (uint32_t)r * (uint32_t)a.lda * 2u + eng::load_chunk_bytes(r, lane);
    }
#pragma unroll
    for (int i = 0; i < S::BI; ++i) {
      const int r = eng::load_row(wave, i, lane);
      ld.boff[i] = (uint32_t)r * (uint32_t)a.ldb * 2u + eng::load_chunk_bytes(r, lane);
    }
    ld.bits = (const WIDE_LDS uint32_t *)&sBits[0][0];
    ld.nk = a.K / eng::kBK;
    ld.steps_per_group = a.G / eng::kBK;
    ld.NG = a.K / a.G;
    ld.wave = wave;
    ld.lane = lane;
    ld.next = 0;
    ld.pred = ld.read_pred(0);
    eng::mainloop<kKBN, false>(ld.nk, ld, (eng::lds_u16 *)sA0, (eng::lds_u16 *)sB0, (eng::lds_u16 *)sA1,
                               (eng::lds_u16 *)sB1, (eng::lds_u16 *)sA2, (eng::lds_u16 *)sB2, acc, wm, wn, lane);
  }

  // C = beta * C + acc; a lane holds row (lane % 16) of A fragment j and
  // features 4 (lane / 16) .. +3 of B fragment i.
#pragma unroll
  for (int j = 0; j < S::FM; ++j) {
    const int m = m0 + wm * S::TM + j * 16 + lane % 16;
    if (m >= a.M) continue;
    float *crow = a.C + (size_t)m * a.ldc + n0 + wn * S::TN + 4 * (lane / 16);
#pragma unroll
    for (int i = 0; i < S::FN; ++i) {
      f32x4 v = acc[i][j];
      if (a.beta) v += *reinterpret_cast<const f32x4 *>(crow + i * 16);
      *reinterpret_cast<f32x4 *>(crow + i * 16) = v;
    }
  }
}

__device__ __forceinline__ float wave_sum_k(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float dot8k(const u32x4 &w, const u32x4 &x, float acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc = fmaf(bf_lo(w[e]), bf_lo(x[e]), acc);
    acc = fmaf(bf_hi(w[e]), bf_hi(x[e]), acc);
  }
  return acc;
}

// Matrix-vector GEMM-K for M <= 4. The four waves first list the K-groups
// some token keeps (one ballot per 64 groups); then each wave owns one output
// feature and streams only the listed groups' segments of its weight row,
// 16 bytes per lane with consecutive lanes on consecutive chunks, a block of
// 8 chunks per lane issued before any is used.
__global__ __launch_bounds__(256) void gemv_k_kernel(KArgs a) {
  constexpr int U = 8;
  __shared__ uint16_t sGrp[kKMaxGroups];
  __shared__ uint8_t sOn[kKMaxGroups];
  __shared__ int sCnt[4];
  const int NG = a.K / a.G;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  int base = 0;
  for (int g0 = 0; g0 < NG; g0 += 4 * kWave) {
    const int g = g0 + wave * kWave + lane;
    int on = 0;
    if (g < NG)
      for (int m = 0; m < a.M; ++m) on |= (a.mask[(size_t)m * NG + g] != 0) << m;
    const uint64_t bal = __ballot(on != 0);
    if (lane == 0) sCnt[wave] = __popcll(bal);
    __syncthreads();
    int before = base;
    for (int w = 0; w < wave; ++w) before += sCnt[w];
    if (on) {
      const int pos = before + rank_below(bal);
      sGrp[pos] = (uint16_t)g;
      sOn[pos] = (uint8_t)on;
    }
    base += sCnt[0] + sCnt[1] + sCnt[2] + sCnt[3];
    __syncthreads();
  }
  const int cpg = a.G / 8;
  const int nchunks = base * cpg;
  const int n = blockIdx.x * 4 + wave;
  const rsrc_t wr = make_rsrc(a.B + (size_t)n * a.ldb, (uint64_t)a.K * 2);
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nchunks; c0 += kWave * U) {
    u32x4 w[U];
    int kk[U], on[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave + lane;
      const bool ok = c < nchunks;
      const int gi = ok ? c / cpg : 0;
      kk[u] = sGrp[gi] * a.G + (c % cpg) * 8;
      on[u] = ok ? sOn[gi] : 0;
      w[u] = buf_ld16(wr, ok ? (uint32_t)kk[u] * 2u : kOffNone);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (m >= a.M) break;
      const rsrc_t xr = make_rsrc(a.A + (size_t)m * a.lda, (uint64_t)a.K * 2);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool use = (on[u] >> m) & 1;
        const u32x4 x = buf_ld16(xr, use ? (uint32_t)kk[u] * 2u : kOffNone);
        s[m] = dot8k(w[u], x, s[m]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (m >= a.M) break;
    const float v = wave_sum_k(s[m]);
    if (lane == 0) {
      float *dst = a.C + (size_t)m * a.ldc + n;
      *dst = a.beta ? *dst + v : v;
    }
  }
}

int launch_gemm_k(const KArgs &a, hipStream_t s) {
  if (a.M <= 4) {
    hipLaunchKernelGGL(gemv_k_kernel, dim3(a.N / 4), dim3(256), 0, s, a);
  } else {
    const int tiles = ((a.M + eng::kBM - 1) / eng::kBM) * (a.N / kKBN);
    hipLaunchKernelGGL(gemm_k_kernel, dim3(tiles), dim3(eng::kThreads), 0, s, a);
  }
  return check_launch();
}

}  // namespace wide
