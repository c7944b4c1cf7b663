// Row order by routing pattern on gfx950 (a scheduling order for GEMM-K).
//
// WIDE (arXiv 2607.28418), Appendix B, Eq. 21: GEMM-K adds group g's partial
// product only for the rows that keep g. A 16-row MFMA fragment can skip
// group g's multiply-adds only when none of its 16 rows keeps g, which
// token-level masks in token order almost never give. Sorting the rows by
// their whole pattern over the groups puts rows that skip the same groups
// next to each other: in the reflected Gray code order of the patterns,
// neighbouring patterns differ in one group, so every group's active rows
// form few, long runs (with 8 groups: one run for the first group, 2^(k-1)
// runs for group k). The order is a permutation of the rows; the GEMM-K
// result of every row does not depend on where the row sits.
//
// key(m) = inverse Gray code of the pattern p(m) = sum over the first
// min(NG, 8) groups g of [mask[m][g] != 0] << (nb - 1 - g), so group 0 is the
// most significant bit. The order is the stable sort of the rows by key
// (rows with equal keys stay ascending), built by one workgroup: a histogram
// of the keys, its exclusive scan, then a stable scatter in chunks of 1024
// rows in which a row's rank among equal keys comes from wave ballots over
// the 8 key bits and per-wave key counts.
#include "common.hpp"
#include "launch.hpp"

namespace wide {

constexpr int kOrdThreads = 1024;
constexpr int kOrdWaves = kOrdThreads / kWave;
constexpr int kOrdBins = 256;

__device__ __forceinline__ int pattern_key(const uint8_t *mask, int m, int NG, int nb) {
  const uint8_t *row = mask + (size_t)m * NG;
  int p = 0;
  for (int g = 0; g < nb; ++g) p |= (row[g] != 0) << (nb - 1 - g);
  // inverse Gray code: prefix XOR from the top bit down
  int k = p;
  k ^= k >> 1;
  k ^= k >> 2;
  k ^= k >> 4;
  return k;
}

__global__ __launch_bounds__(kOrdThreads) void pattern_order_kernel(const uint8_t *mask, int M, int NG,
                                                                    int32_t *order) {
  __shared__ int sBase[kOrdBins];              // next free position of each key
  __shared__ int sCnt[kOrdWaves][kOrdBins];    // rows of each key per wave in the chunk
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int nb = NG < 8 ? NG : 8;
  for (int i = tid; i < kOrdBins; i += kOrdThreads) sBase[i] = 0;
  for (int i = tid; i < kOrdWaves * kOrdBins; i += kOrdThreads) (&sCnt[0][0])[i] = 0;
  __syncthreads();
  // histogram
  for (int m = tid; m < M; m += kOrdThreads) atomicAdd(&sBase[pattern_key(mask, m, NG, nb)], 1);
  __syncthreads();
  // exclusive scan of the 256 bins by the first wave (4 bins per lane)
  if (wave == 0) {
    int v[4], s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = sBase[4 * lane + j];
      s += v[j];
    }
    int x = s;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    int run = x - s;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sBase[4 * lane + j] = run;
      run += v[j];
    }
  }
  __syncthreads();
  // stable scatter, chunk by chunk
  for (int c0 = 0; c0 < M; c0 += kOrdThreads) {
    const int m = c0 + tid;
    const bool valid = m < M;
    const int key = valid ? pattern_key(mask, m, NG, nb) : -1;
    // lanes of this wave with the same key (8 ballots over the key bits)
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint64_t bal = __ballot(valid && ((key >> b) & 1));
      peers &= ((key >> b) & 1) ? bal : ~bal;
    }
    const int rank = rank_below(peers);
    const int n = __popcll(peers);
    if (valid && rank == n - 1) sCnt[wave][key] = n;  // one writer per key per wave
    __syncthreads();
    if (valid) {
      int before = sBase[key] + rank;
      for (int w = 0; w < wave; ++w) before += sCnt[w][key];
      order[before] = m;
    }
    __syncthreads();
    // advance the bases past this chunk and clear the counts
    for (int k = tid; k < kOrdBins; k += kOrdThreads) {
      int t = 0;
      for (int w = 0; w < kOrdWaves; ++w) {
        t += sCnt[w][k];
        sCnt[w][k] = 0;
      }
      sBase[k] += t;
    }
    __syncthreads();
  }
}

int launch_pattern_order(const uint8_t *mask, int M, int NG, int32_t *order, hipStream_t s) {
  hipLaunchKernelGGL(pattern_order_kernel, dim3(1), dim3(kOrdThreads), 0, s, mask, M, NG, order);
  return check_launch();
}

}  // namespace wide
