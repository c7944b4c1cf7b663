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
// (rows with equal keys stay ascending), built by one workgroup in which each
// wave counts, then places, a contiguous range of rows.
#include "common.hpp"
#include "launch.hpp"

namespace wide {

constexpr int kOrdThreads = 1024;
constexpr int kOrdWaves = kOrdThreads / kWave;
constexpr int kOrdBins = 256;
constexpr int kOrdKeyRegs = 16;  // 64-row rounds per wave whose keys stay in registers

// Key of row m from the first min(NG, 8) bytes of its mask row: one 8-byte
// load (WIDE = 8), two 4-byte loads (WIDE = 4) or byte loads (WIDE = 1), all
// unconditional so a thread's loads are in flight together (the caller
// clamps m to a valid row).
template <int WIDE>
__device__ __forceinline__ int pattern_key(const uint8_t *mask, int m, int NG, int nb) {
  const uint8_t *row = mask + (size_t)m * NG;
  uint8_t v[8];
  if (WIDE == 8) {
    const uint64_t w = *reinterpret_cast<const uint64_t *>(row);
#pragma unroll
    for (int g = 0; g < 8; ++g) v[g] = (uint8_t)(w >> (8 * g));
  } else if (WIDE == 4) {
    const uint32_t w0 = *reinterpret_cast<const uint32_t *>(row);
    const uint32_t w1 = *reinterpret_cast<const uint32_t *>(row + (nb > 4 ? 4 : 0));
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      v[g] = (uint8_t)(w0 >> (8 * g));
      v[g + 4] = (uint8_t)(w1 >> (8 * g));
    }
  } else {
#pragma unroll
    for (int g = 0; g < 8; ++g) v[g] = row[g < nb ? g : 0];
  }
  int p = 0;
#pragma unroll
  for (int g = 0; g < 8; ++g) p |= (g < nb && v[g] != 0) ? 1 << (nb - 1 - g) : 0;
  // inverse Gray code: prefix XOR from the top bit down
  int k = p;
  k ^= k >> 1;
  k ^= k >> 2;
  k ^= k >> 4;
  return k;
}

// Lanes of the wave holding the same key as this lane (8 ballots over the
// key bits); invalid lanes carry key -1 and match nobody valid.
__device__ __forceinline__ uint64_t key_peers(int key, bool valid) {
  uint64_t peers = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const uint64_t bal = __ballot(valid && ((key >> b) & 1));
    peers &= ((key >> b) & 1) ? bal : ~bal;
  }
  return peers;
}

// Wave w owns the contiguous rows [w R, (w + 1) R), R = ceil(M / 16) rounded
// up to 64, and walks them 64 at a time. Pass 1 counts its keys in its own
// row of sH (only that wave touches it, in order: no barrier inside a pass);
// between the passes the counts become, per key, the base of the key's bin
// plus the rows of that key owned by earlier waves; pass 2 places every row
// at its wave's running offset for its key plus its rank among the equal
// keys of its round, which keeps equal keys in ascending row order.
template <int WIDE>
__global__ __launch_bounds__(kOrdThreads) void pattern_order_kernel(const uint8_t *mask, int M, int NG,
                                                                    int32_t *order) {
  __shared__ int sH[kOrdWaves][kOrdBins];
  __shared__ int sTmp[kOrdWaves];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int nb = NG < 8 ? NG : 8;
  const int R = ((M + kOrdWaves - 1) / kOrdWaves + kWave - 1) / kWave * kWave;
  const int r0 = wave * R, rounds = R / kWave;
  for (int i = tid; i < kOrdWaves * kOrdBins; i += kOrdThreads) (&sH[0][0])[i] = 0;
  __syncthreads();
  int keep[kOrdKeyRegs];
  // pass 1: count (keys of the first kOrdKeyRegs rounds kept for pass 2)
  for (int c = 0; c < rounds; c += kOrdKeyRegs) {
    int key[kOrdKeyRegs];
#pragma unroll
    for (int u = 0; u < kOrdKeyRegs; ++u) {
      const int m = r0 + (c + u) * kWave + lane;
      const bool ok = c + u < rounds && m < M;
      const int kk = pattern_key<WIDE>(mask, ok ? m : M - 1, NG, nb);
      key[u] = ok ? kk : -1;
    }
#pragma unroll
    for (int u = 0; u < kOrdKeyRegs; ++u) {
      const uint64_t peers = key_peers(key[u], key[u] >= 0);
      if (key[u] >= 0 && rank_below(peers) == 0) sH[wave][key[u]] += __popcll(peers);
      if (c == 0) keep[u] = key[u];
    }
  }
  __syncthreads();
  // bin bases: thread k < 256 owns key k
  int tot = 0;
  if (tid < kOrdBins) {
#pragma unroll
    for (int w = 0; w < kOrdWaves; ++w) tot += sH[w][tid];
  }
  // exclusive scan of the 256 totals over waves 0..3 (64 keys each)
  int x = tot;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1 && wave < 4) sTmp[wave] = x;
  __syncthreads();
  if (tid < kOrdBins) {
    int base = x - tot;
    for (int w = 0; w < wave; ++w) base += sTmp[w];
#pragma unroll
    for (int w = 0; w < kOrdWaves; ++w) {
      const int c = sH[w][tid];
      sH[w][tid] = base;
      base += c;
    }
  }
  __syncthreads();
  // pass 2: place
  for (int c = 0; c < rounds; ++c) {
    const int m = r0 + c * kWave + lane;
    const bool valid = m < M;
    int key = -1;
    if (valid) {
      if (c < kOrdKeyRegs) {
#pragma unroll
        for (int u = 0; u < kOrdKeyRegs; ++u)
          if (u == c) key = keep[u];
      } else {
        key = pattern_key<WIDE>(mask, m, NG, nb);
      }
    }
    const uint64_t peers = key_peers(key, valid);
    if (valid) {
      const int at = sH[wave][key];
      order[at + rank_below(peers)] = m;
      // the first lane of each key advances the wave's offset for the next round
      if (rank_below(peers) == 0) sH[wave][key] = at + __popcll(peers);
    }
  }
}

int launch_pattern_order(const uint8_t *mask, int M, int NG, int32_t *order, hipStream_t s) {
  // widest load every row start allows (only bytes of the row itself are read)
  const uintptr_t base = reinterpret_cast<uintptr_t>(mask);
  if (NG >= 8 && NG % 8 == 0 && base % 8 == 0)
    hipLaunchKernelGGL(pattern_order_kernel<8>, dim3(1), dim3(kOrdThreads), 0, s, mask, M, NG, order);
  else if (NG >= 4 && NG % 4 == 0 && base % 4 == 0)
    hipLaunchKernelGGL(pattern_order_kernel<4>, dim3(1), dim3(kOrdThreads), 0, s, mask, M, NG, order);
  else
    hipLaunchKernelGGL(pattern_order_kernel<1>, dim3(1), dim3(kOrdThreads), 0, s, mask, M, NG, order);
  return check_launch();
}

}  // namespace wide
