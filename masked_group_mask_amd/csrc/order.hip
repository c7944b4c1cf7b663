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
// 64-row rounds per wave whose keys stay in registers (fewer with byte loads,
// whose eight loads per row would otherwise spill at 128 registers a thread)
template <int WIDE>
constexpr int ord_key_regs() { return WIDE == 1 ? 4 : 16; }

// Key of row m from the first min(NG, 8) bytes of its mask row: one 8-byte
// load (WIDE = 8), two 4-byte loads (WIDE = 4) or byte loads (WIDE = 1), all
// unconditional so a thread's loads are in flight together (the caller
// clamps m to a valid row).
// The first min(NG, 8) mask bytes of row m, as loaded (split from the key so
// that a thread can issue all its loads before it uses any).
struct RowBytes {
  uint32_t lo, hi;
};

template <int WIDE>
__device__ __forceinline__ RowBytes load_row_bytes(const uint8_t *mask, int m, int NG, int nb) {
  const uint8_t *row = mask + (size_t)m * NG;
  RowBytes r;
  if (WIDE == 8) {
    const uint64_t w = *reinterpret_cast<const uint64_t *>(row);
    r.lo = (uint32_t)w;
    r.hi = (uint32_t)(w >> 32);
  } else if (WIDE == 4) {
    r.lo = *reinterpret_cast<const uint32_t *>(row);
    r.hi = *reinterpret_cast<const uint32_t *>(row + (nb > 4 ? 4 : 0));
  } else {
    r.lo = r.hi = 0u;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const uint32_t b = row[g < nb ? g : 0];
      if (g < 4)
        r.lo |= b << (8 * g);
      else
        r.hi |= b << (8 * (g - 4));
    }
  }
  return r;
}

__device__ __forceinline__ int row_key(RowBytes r, int nb) {
  uint8_t v[8];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    v[g] = (uint8_t)(r.lo >> (8 * g));
    v[g + 4] = (uint8_t)(r.hi >> (8 * g));
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

template <int WIDE>
__device__ __forceinline__ int pattern_key(const uint8_t *mask, int m, int NG, int nb) {
  return row_key(load_row_bytes<WIDE>(mask, m, NG, nb), nb);
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
// One compute unit does it all, so the kernel is bound by latency (~17 us
// at 8192 rows on MI355X, most of it the first pass's mask loads and its
// dependent LDS updates).
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
  constexpr int KR = ord_key_regs<WIDE>();
  int keep[KR];
  // pass 1: count (keys of the first KR rounds kept for pass 2)
  for (int c = 0; c < rounds; c += KR) {
    // every load of the chunk in flight before the first is used
    RowBytes raw[KR];
#pragma unroll
    for (int u = 0; u < KR; ++u) {
      const int m = r0 + (c + u) * kWave + lane;
      const bool ok = c + u < rounds && m < M;
      raw[u] = load_row_bytes<WIDE>(mask, ok ? m : M - 1, NG, nb);
    }
    __builtin_amdgcn_sched_barrier(0);
    int key[KR];
#pragma unroll
    for (int u = 0; u < KR; ++u) {
      const int m = r0 + (c + u) * kWave + lane;
      const bool ok = c + u < rounds && m < M;
      key[u] = ok ? row_key(raw[u], nb) : -1;
    }
#pragma unroll
    for (int u = 0; u < KR; ++u) {
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
      if (c < KR) {
#pragma unroll
        for (int u = 0; u < KR; ++u)
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
  const int wide = NG >= 8 && NG % 8 == 0 && base % 8 == 0 ? 8 : NG >= 4 && NG % 4 == 0 && base % 4 == 0 ? 4 : 1;
  const dim3 g(1), b(kOrdThreads);
  if (wide == 8)
    hipLaunchKernelGGL(pattern_order_kernel<8>, g, b, 0, s, mask, M, NG, order);
  else if (wide == 4)
    hipLaunchKernelGGL(pattern_order_kernel<4>, g, b, 0, s, mask, M, NG, order);
  else
    hipLaunchKernelGGL(pattern_order_kernel<1>, g, b, 0, s, mask, M, NG, order);
  return check_launch();
}

}  // namespace wide
