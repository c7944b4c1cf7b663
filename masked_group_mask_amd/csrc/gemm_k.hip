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
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace wide {

constexpr int kKBM = 128;          // original rows per workgroup tile
constexpr int kKBN = 128;          // output features per workgroup tile
constexpr int kKAccLd = kKBN + 4;  // LDS accumulator row stride (fp32)
constexpr int kKMaxGroups = 512;
constexpr int kKThreads = 512;  // 8 waves: two per SIMD

// LDS tiles hold rows of 64 bf16 (128 bytes, 8 chunks of 16 bytes) without
// padding. Chunk `c` of row `s` sits at position c ^ ((s / 2) % 8): the 16
// rows one MFMA operand read touches then cover all 64 banks once.
__device__ __forceinline__ int tile_pos(int s, int c) { return c ^ ((s >> 1) & 7); }

constexpr int kKBK = 64;                       // K depth of one pipeline item
constexpr int kKTile = 128 * kKBK;             // bf16 elements per 128-row tile

// Logical tile id -> (row tile, feature tile). raster 0: row tiles fastest
// (consecutive tiles share weights); 1: feature tiles fastest (they share the
// activation rows); 2: blocks of 4 row tiles x 8 feature tiles, so the 32
// workgroups an XCD runs at once share both operands in its L2.
__device__ __forceinline__ void tile_order(int L, int m_tiles, int n_tiles, int raster, int &mt,
                                           int &nt) {
  constexpr int SM = 4, SN = 8;
  if (raster == 2 && m_tiles % SM == 0 && n_tiles % SN == 0) {
    const int blk = L / (SM * SN), in = L % (SM * SN);
    const int nb = n_tiles / SN;
    mt = (blk / nb) * SM + in % SM;
    nt = (blk % nb) * SN + in / SM;
  } else if (raster == 1) {
    mt = L / n_tiles;
    nt = L % n_tiles;
  } else {
    mt = L % m_tiles;
    nt = L / m_tiles;
  }
}

// One workgroup = C[r0:r0+128, n0:n0+128]. The work is a sequence of items
// (active group, 64-wide slice of its K range). Per item:
//   - the group's active rows of A (their list is built from the mask two
//     items ahead) and the 128 weight rows are loaded with whole 128-byte
//     lines per row and staged in swizzled LDS tiles (double-buffered; the
//     loads of item i+1 are in flight while item i computes);
//   - each wave computes D^T[n][slot] = W[n][k] * A[slot][k] for its 32
//     features and every 16-slot fragment up to the active count, on
//     v_mfma_f32_16x16x32_bf16, so a lane ends with 4 consecutive features
//     of one compact row;
//   - after the group's last slice those 4 values are added into the fp32
//     LDS accumulator at the row the slot came from (16-byte read-add-write).
__global__ __launch_bounds__(kKThreads, 1) void gemm_k_kernel(KArgs a) {
  constexpr int kWaves = kKThreads / kWave;
  __shared__ __attribute__((aligned(16))) float sAcc[kKBM * kKAccLd];
  __shared__ __attribute__((aligned(16))) uint16_t sAct[2][kKTile];
  __shared__ __attribute__((aligned(16))) uint16_t sW[2][kKTile];
  __shared__ uint64_t sBits[kKMaxGroups][2];
  __shared__ uint16_t sGrp[kKMaxGroups];
  __shared__ uint8_t sRowOf[3][kKBM];
  __shared__ int sNact;
  static_assert(sizeof(sAct) >= 64 * kKMaxGroups, "mask staging needs 64 rows x max groups");

  const int n_tiles = a.N / kKBN;
  const int m_tiles = (a.M + kKBM - 1) / kKBM;
  const int L = xcd_remap(blockIdx.x, n_tiles * m_tiles);
  int mt, nt;
  tile_order(L, m_tiles, n_tiles, a.raster, mt, nt);
  const int n0 = nt * kKBN;
  const int r0 = mt * kKBM;
  const int NG = a.K / a.G;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;

  for (int i = tid * 4; i < kKBM * kKAccLd; i += kKThreads * 4)
    *reinterpret_cast<f32x4 *>(&sAcc[i]) = f32x4{0.f, 0.f, 0.f, 0.f};

  // Row sets per group. Each half of the mask tile ([64 rows][NG] bytes, at
  // most 32 KB) is copied to LDS (the activation buffers are free until the
  // main loop); then every wave ballots the 64 rows of a quarter of the groups.
  {
    uint8_t *sMask = reinterpret_cast<uint8_t *>(&sAct[0][0]);
    const bool vec = (NG % 16) == 0 && (reinterpret_cast<uintptr_t>(a.mask) % 16) == 0;
    for (int half = 0; half < 2; ++half) {
      const int rb = r0 + half * 64;
      const int rows = max(0, min(64, a.M - rb));
      const uint8_t *src = a.mask + (size_t)rb * NG;
      const int nbytes = rows * NG;
      if (vec) {
        for (int i = tid * 16; i < nbytes; i += kKThreads * 16) st16(sMask + i, ld16(src + i));
      } else {
        for (int i = tid; i < nbytes; i += kKThreads) sMask[i] = src[i];
      }
      __syncthreads();
      for (int g = wave; g < NG; g += kWaves) {
        const uint64_t bal = __ballot(lane < rows && sMask[lane * NG + g] != 0);
        if (lane == 0) sBits[g][half] = bal;
      }
      __syncthreads();
    }
  }
  // Active groups (level 0: a (tile, group) pair with no active row is skipped).
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

  const int ipg = a.G / kKBK;  // items per group
  const int nact = uniform(sNact);
  const int nitems = nact * ipg;

  // slot -> row list of active group ordinal gi, into ring slot gi % 3
  // (waves 0 and 1 each rank 64 rows with a ballot).
  auto build_list = [&](int gi) {
    if (gi >= nact || wave >= 2) return;
    const int g = sGrp[gi];
    const uint64_t b0 = sBits[g][0], b1 = sBits[g][1];
    const uint64_t bw = wave == 0 ? b0 : b1;
    if ((bw >> lane) & 1ull) {
      const int slot = (wave == 0 ? 0 : __popcll(b0)) + rank_below(bw);
      sRowOf[gi % 3][slot] = (uint8_t)(wave * 64 + lane);
    }
  };

  const int chunk = tid % 8;
  const int rsub = tid / 8;  // 0..63
  const int wm = wave / 4;   // slot fragments wm, wm + 2, ...
  const int wn = wave % 4;   // features wn * 32 .. + 32
  const rsrc_t arows = make_rsrc(a.A + (size_t)r0 * a.lda,
                                 (uint64_t)min(kKBM, a.M - r0) * a.lda * 2);
  const uint16_t *wbase = a.B + (size_t)n0 * a.ldb + chunk * 8;
  u32x4 ra[2], rw[2];

  auto issue = [&](int item) {
    const int gi = item / ipg, ks = item % ipg;
    const int g = sGrp[gi];
    const int cnt = __popcll(sBits[g][0]) + __popcll(sBits[g][1]);
    const int kcol = g * a.G + ks * kKBK + chunk * 8;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int sl = rsub + 64 * p;
      // level 1: only the active rows are fetched (packed by slot)
      const uint32_t off = sl < cnt ? (uint32_t)(sRowOf[gi % 3][sl] * a.lda + kcol) * 2u : kOffNone;
      ra[p] = buf_ld16(arows, off);
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) rw[p] = ld16(wbase + (size_t)(rsub + 64 * p) * a.ldb + (kcol - chunk * 8));
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = rsub + 64 * p;
      st16(&sAct[buf][r * kKBK + tile_pos(r, chunk) * 8], ra[p]);
      st16(&sW[buf][r * kKBK + tile_pos(r, chunk) * 8], rw[p]);
    }
  };

  f32x4 acc[2][4];  // [feature fragment][own slot fragment j: sf = wm + 2j]
#pragma unroll
  for (int nf = 0; nf < 2; ++nf)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[nf][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The slot -> row list of the group of item j is built in iteration j - 2
  // (before the barrier that precedes the loads of item j, issued in
  // iteration j - 1); ring slot g % 3 is then free, as group g - 3 has
  // finished. Items 0 and 1 are covered here.
  build_list(0);
  if (ipg == 1) build_list(1);
  __syncthreads();
  if (nitems > 0) {
    issue(0);
    stage(0);
  }
  __syncthreads();

  for (int it = 0; it < nitems; ++it) {
    const int cur = it & 1;
    const int gi = it / ipg, ks = it % ipg;
    const int g = sGrp[gi];
    const int cnt = uniform(__popcll(sBits[g][0]) + __popcll(sBits[g][1]));
    const int live = (cnt + 15) / 16;
    const bool more = it + 1 < nitems;
    const bool last = ks == ipg - 1;
    const int ring = gi % 3;
    if (more) issue(it + 1);  // the next item's global loads go out first

    u32x4 wfr[2][2];  // [feature fragment][k step]
#pragma unroll
    for (int nf = 0; nf < 2; ++nf)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int r = wn * 32 + nf * 16 + lane % 16;
        wfr[nf][q] = ld16(&sW[cur][r * kKBK + tile_pos(r, q * 4 + lane / 16) * 8]);
      }
    // level 2: only ceil(cnt/16) 16-slot fragments are issued; the body is
    // specialised on that count (rounded up to even) so all LDS reads of a K
    // step are issued before its MFMAs, with no branch in between.
    auto body = [&](auto nsf_c) {
      constexpr int NJ = decltype(nsf_c)::value / 2;  // own fragments: sf = wm + 2j
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        u32x4 act[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int s = (wm + 2 * j) * 16 + lane % 16;
          act[j] = ld16(&sAct[cur][s * kKBK + tile_pos(s, q * 4 + lane / 16) * 8]);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int nf = 0; nf < 2; ++nf) acc[nf][j] = mfma16x16x32(wfr[nf][q], act[j], acc[nf][j]);
      }
      if (last) {
        // Add the group's partial products into the LDS accumulator at the
        // rows the slots came from (16-byte read-add-write per lane; within a
        // group every (row, feature) belongs to one lane).
        int rrow[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int s = (wm + 2 * j) * 16 + lane % 16;
          rrow[j] = s < cnt ? (int)sRowOf[ring][s] : -1;
        }
        f32x4 old[NJ][2];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int nf = 0; nf < 2; ++nf)
            if (rrow[j] >= 0)
              old[j][nf] = *reinterpret_cast<const f32x4 *>(
                  &sAcc[rrow[j] * kKAccLd + wn * 32 + nf * 16 + (lane / 16) * 4]);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int nf = 0; nf < 2; ++nf) {
            if (rrow[j] >= 0)
              *reinterpret_cast<f32x4 *>(&sAcc[rrow[j] * kKAccLd + wn * 32 + nf * 16 + (lane / 16) * 4]) =
                  old[j][nf] + acc[nf][j];
            acc[nf][j] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
      }
    };
    switch ((live + 1) / 2) {
      case 0: break;
      case 1: body(std::integral_constant<int, 2>{}); break;
      case 2: body(std::integral_constant<int, 4>{}); break;
      case 3: body(std::integral_constant<int, 6>{}); break;
      default: body(std::integral_constant<int, 8>{}); break;
    }
    if ((it + 2) % ipg == 0) build_list((it + 2) / ipg);
    if (more) stage(cur ^ 1);
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
    const int tiles = (a.N / kKBN) * ((a.M + kKBM - 1) / kKBM);
    hipLaunchKernelGGL(gemm_k_kernel, dim3(tiles), dim3(kKThreads), 0, s, a);
  }
  return check_launch();
}

}  // namespace wide
