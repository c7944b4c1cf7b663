// GEMM-K on gfx950: the K-axis routed projection (W_o, W_down).
//
// WIDE (arXiv 2607.28418) Appendix B, Eq. 21 and Algorithm 3:
//   C[m][n] = sum_g mask[m][g] * sum_{k in group g} A[m][k] * B[n][k].
// The page runs one pipeline per (sorted row tile, K-group) and scatters each
// fp32 partial into C with global atomics. On MI355X the same work is done
// with an accumulator that never leaves the chip:
//   - a workgroup owns C[r0:r0+128, n0:n0+128] in ORIGINAL row order and keeps
//     it as an fp32 tile in LDS (64 KB of the 160 KB);
//   - from the mask bytes of its 128 rows it builds, per K-group, a 128-bit
//     row set (one ballot per 64 rows) and the list of groups with any active
//     row; an empty (tile, group) pair is skipped outright (level 0);
//   - for each active group it loads only the active rows of A, packed to the
//     front of the LDS tile in row order (level 1: the slot of a row is the
//     popcount of the active rows below it), issues MFMA fragments only up to
//     the active count (level 2), and adds the 16x16 fp32 results into the LDS
//     accumulator at the rows they came from. Within one group the rows are
//     distinct and each (row, column) belongs to one lane, so the adds need no
//     atomics; groups follow each other between barriers, so the summation
//     order is fixed and the result is reproducible bit for bit;
//   - the K loop runs over (active group, 64-wide K step) items with the LDS
//     double buffer flowing across group boundaries, so short groups do not
//     drain the pipeline;
//   - C is written once, coalesced, as beta*C + acc.
// For M <= 4 a matrix-vector kernel streams only the active K-groups of each
// weight row.
#include "common.hpp"
#include "launch.hpp"

namespace wide {

constexpr int kKBM = 128;
constexpr int kKBN = 128;
constexpr int kKBK = 64;
constexpr int kKLds = kKBK + 8;
constexpr int kKAccLd = kKBN + 4;
constexpr int kKMaxGroups = 512;
constexpr int kKThreads = 256;

__global__ __launch_bounds__(kKThreads, 1) void gemm_k_kernel(KArgs a) {
  __shared__ __attribute__((aligned(16))) float sAcc[kKBM * kKAccLd];
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kKBM * kKLds];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kKBN * kKLds];
  __shared__ uint64_t sBits[kKMaxGroups][2];
  __shared__ uint16_t sGrp[kKMaxGroups];
  __shared__ uint8_t sRowOf[2][kKBM];
  __shared__ int sNact;

  const int n_tiles = a.N / kKBN;
  const int m_tiles = (a.M + kKBM - 1) / kKBM;
  const int L = xcd_remap(blockIdx.x, n_tiles * m_tiles);
  const int n0 = (L / m_tiles) * kKBN;
  const int r0 = (L % m_tiles) * kKBM;
  const int NG = a.K / a.G;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;

  for (int i = tid * 4; i < kKBM * kKAccLd; i += kKThreads * 4)
    *reinterpret_cast<f32x4 *>(&sAcc[i]) = f32x4{0.f, 0.f, 0.f, 0.f};

  // Row sets per group: wave w covers rows (w & 1) * 64 + lane of every
  // second group starting at w >> 1.
  {
    const int half = wave & 1;
    const int r = r0 + half * 64 + lane;
    const uint8_t *mrow = a.mask + (size_t)r * NG;
    for (int g = wave >> 1; g < NG; g += 2) {
      const uint64_t b = __ballot(r < a.M && mrow[g] != 0);
      if (lane == 0) sBits[g][half] = b;
    }
  }
  __syncthreads();
  if (wave == 0) {
    int base = 0;
    for (int g0 = 0; g0 < NG; g0 += kWave) {
      const int g = g0 + lane;
      const bool nz = g < NG && (sBits[g][0] | sBits[g][1]) != 0ull;
      const uint64_t bal = __ballot(nz);
      if (nz) sGrp[base + rank_below(bal)] = (uint16_t)g;
      base += __popcll(bal);
    }
    if (lane == 0) sNact = base;
  }
  __syncthreads();

  const int kpg = a.G / kKBK;
  const int nitems = uniform(sNact) * kpg;
  const int chunk = tid % 8;
  const int rbase = tid / 8;
  const int wm = wave / 2, wn = wave % 2;

  u32x4 ra[4], rb[4];
  int rslot[4];
  auto gload = [&](int item) {
    const int gi = item / kpg, ks = item % kpg;
    const int g = sGrp[gi];
    const uint64_t b0 = sBits[g][0], b1 = sBits[g][1];
    const int kcol = g * a.G + ks * kKBK + chunk * 8;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = rbase + 32 * p;
      const uint64_t bits = r < 64 ? b0 : b1;
      const uint64_t below = bits & ((1ull << (r & 63)) - 1ull);
      const bool on = (bits >> (r & 63)) & 1ull;
      rslot[p] = on ? (r < 64 ? 0 : __popcll(b0)) + __popcll(below) : -1;
      if (on) ra[p] = ld16(a.A + (size_t)(r0 + r) * a.lda + kcol);  // level 1
      rb[p] = ld16(a.B + (size_t)(n0 + r) * a.ldb + kcol);
    }
  };
  auto lstore = [&](int buf, int par) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (rslot[p] >= 0) {
        st16(&sA[buf][rslot[p] * kKLds + chunk * 8], ra[p]);
        if (chunk == 0) sRowOf[par][rslot[p]] = (uint8_t)(rbase + 32 * p);
      }
      st16(&sB[buf][(rbase + 32 * p) * kKLds + chunk * 8], rb[p]);
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nitems > 0) {
    gload(0);
    lstore(0, 0);
  }
  __syncthreads();
  for (int it = 0; it < nitems; ++it) {
    const int cur = it & 1;
    const int gi = it / kpg, ks = it % kpg;
    const int g = sGrp[gi];
    const int cnt = uniform(__popcll(sBits[g][0]) + __popcll(sBits[g][1]));
    if (it + 1 < nitems) gload(it + 1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int koff = kk * 32 + (lane / 16) * 8;
      u32x4 bf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[j] = ld16(&sB[cur][(wn * 64 + 16 * j + lane % 16) * kKLds + koff]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = wm + 2 * i;
        if (16 * f < cnt) {  // level 2
          const u32x4 af = ld16(&sA[cur][(16 * f + lane % 16) * kKLds + koff]);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(af, bf[j], acc[i][j]);
        }
      }
    }
    if (ks == kpg - 1) {
      // Add this group's partial products into the LDS accumulator.
      const int par = gi & 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = wm + 2 * i;
        if (16 * f >= cnt) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int slot = 16 * f + 4 * (lane / 16) + v;
          if (slot < cnt) {
            float *dst = &sAcc[sRowOf[par][slot] * kKAccLd + wn * 64 + lane % 16];
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[16 * j] += acc[i][j][v];
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    if (it + 1 < nitems) lstore(cur ^ 1, ((it + 1) / kpg) & 1);
    __syncthreads();
  }

  // C = beta * C + acc, 16-byte stores.
  for (int i = tid; i < kKBM * (kKBN / 4); i += kKThreads) {
    const int r = i / (kKBN / 4), c = (i % (kKBN / 4)) * 4;
    if (r0 + r >= a.M) continue;
    f32x4 v = *reinterpret_cast<const f32x4 *>(&sAcc[r * kKAccLd + c]);
    f32x4 *dst = reinterpret_cast<f32x4 *>(a.C + (size_t)(r0 + r) * a.ldc + n0 + c);
    if (a.beta) v += *dst;
    *dst = v;
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

// Matrix-vector GEMM-K for M <= 4: a workgroup owns 16 output features and
// streams, for each, only the K-groups that some token keeps.
__global__ __launch_bounds__(256) void gemv_k_kernel(KArgs a) {
  __shared__ uint16_t sGrp[kKMaxGroups];
  __shared__ uint8_t sOn[kKMaxGroups];
  __shared__ int sNact;
  const int NG = a.K / a.G;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  if (wave == 0) {
    int base = 0;
    for (int g0 = 0; g0 < NG; g0 += kWave) {
      const int g = g0 + lane;
      int on = 0;
      if (g < NG)
        for (int m = 0; m < a.M; ++m) on |= (a.mask[(size_t)m * NG + g] != 0) << m;
      const uint64_t bal = __ballot(on != 0);
      if (on) {
        const int pos = base + rank_below(bal);
        sGrp[pos] = (uint16_t)g;
        sOn[pos] = (uint8_t)on;
      }
      base += __popcll(bal);
    }
    if (lane == 0) sNact = base;
  }
  __syncthreads();
  const int cpg = a.G / 8;
  const int nchunks = sNact * cpg;
  const int nb = blockIdx.x * 16 + wave * 4;
  float s[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) s[m][r] = 0.f;
  for (int c = lane; c < nchunks; c += kWave) {
    const int gi = c / cpg;
    const int k = sGrp[gi] * a.G + (c % cpg) * 8;
    const int on = sOn[gi];
    u32x4 x[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if ((on >> m) & 1) x[m] = ld16(a.A + (size_t)m * a.lda + k);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const u32x4 w = ld16(a.B + (size_t)(nb + r) * a.ldb + k);
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if ((on >> m) & 1) s[m][r] = dot8k(w, x[m], s[m][r]);
    }
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (m >= a.M) break;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = wave_sum_k(s[m][r]);
      if (lane == 0) {
        float *dst = a.C + (size_t)m * a.ldc + nb + r;
        *dst = a.beta ? *dst + v : v;
      }
    }
  }
}

int launch_gemm_k(const KArgs &a, hipStream_t s) {
  if (a.M <= 4) {
    hipLaunchKernelGGL(gemv_k_kernel, dim3(a.N / 16), dim3(256), 0, s, a);
  } else {
    const int tiles = (a.N / kKBN) * ((a.M + kKBM - 1) / kKBM);
    hipLaunchKernelGGL(gemm_k_kernel, dim3(tiles), dim3(kKThreads), 0, s, a);
  }
  return check_launch();
}

}  // namespace wide
