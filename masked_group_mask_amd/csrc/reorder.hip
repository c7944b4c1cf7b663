// Mask reordering on gfx950.
//
// WIDE (arXiv 2607.28418) section 3.3, Eq. 7 and Appendix B, Algorithm 1:
// every routing column is sorted so that its active rows form a prefix and an
// index maps each logical row back to its physical row. Here the sort is the
// stable two-way partition (active rows ascending, then inactive rows
// ascending), computed with wavefront ballots:
//   - pass 1 counts the active rows of each column (ballot + popcount);
//   - pass 2 walks the rows again; a row's number of active predecessors is
//     the running count of earlier chunks + the counts of lower waves in this
//     chunk + the active lanes below it in its wave (mbcnt). An active row
//     goes to that position; an inactive row r goes to
//     count + (r - active predecessors).
// One workgroup of 8 waves owns GPW columns for all rows, so no global
// scratch or second launch is needed. Up to 16384 rows a workgroup owns one
// column and keeps its rows in registers between the passes
// (reorder_reg_kernel); longer columns re-read the mask from L2 per chunk.
#include "common.hpp"
#include "launch.hpp"

namespace wide {

constexpr int kReorderThreads = 512;
constexpr int kReorderWaves = kReorderThreads / kWave;

template <int GPW>
__device__ __forceinline__ void load_mask_bytes(const uint8_t *row, int ng, bool aligned8,
                                                bool valid, uint8_t (&v)[GPW]) {
  if (GPW == 8 && aligned8) {
    uint64_t w = valid ? *reinterpret_cast<const uint64_t *>(row) : 0ull;
#pragma unroll
    for (int j = 0; j < GPW; ++j) v[j] = (uint8_t)(w >> (8 * j));
  } else {
#pragma unroll
    for (int j = 0; j < GPW; ++j) v[j] = (valid && j < ng) ? row[j] : (uint8_t)0;
  }
}

template <int GPW>
__global__ __launch_bounds__(kReorderThreads) void reorder_kernel(const uint8_t *__restrict__ mask,
                                                                  int rows, int groups,
                                                                  int32_t *__restrict__ perm,
                                                                  int32_t *__restrict__ counts) {
  const int b = blockIdx.y;
  const int g0 = blockIdx.x * GPW;
  const int ng = min(GPW, groups - g0);
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const uint8_t *mb = mask + (size_t)b * rows * groups + g0;
  const bool aligned8 = ((groups % 8) == 0) && ((g0 % 8) == 0) &&
                        ((reinterpret_cast<uintptr_t>(mask) % 8) == 0);

  __shared__ int s_cnt[2][GPW][kReorderWaves];
  __shared__ int s_total[GPW];

  // Pass 1: active rows per column.
  int wcount[GPW];
#pragma unroll
  for (int j = 0; j < GPW; ++j) wcount[j] = 0;
  for (int r0 = 0; r0 < rows; r0 += kReorderThreads) {
    const int r = r0 + tid;
    uint8_t v[GPW];
    load_mask_bytes<GPW>(mb + (size_t)r * groups, ng, aligned8, r < rows, v);
#pragma unroll
    for (int j = 0; j < GPW; ++j) wcount[j] += __popcll(__ballot(v[j] != 0));
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < GPW; ++j) s_cnt[0][j][wave] = wcount[j];
  }
  __syncthreads();
  if (tid < GPW) {
    int t = 0;
    for (int w = 0; w < kReorderWaves; ++w) t += s_cnt[0][tid][w];
    s_total[tid] = t;
    if (tid < ng) counts[(size_t)b * groups + g0 + tid] = t;
  }
  __syncthreads();

  int total[GPW];
#pragma unroll
  for (int j = 0; j < GPW; ++j) total[j] = s_total[j];

  // Pass 2: scatter each row to its partitioned position.
  int base[GPW];  // active rows in earlier chunks
#pragma unroll
  for (int j = 0; j < GPW; ++j) base[j] = 0;
  int par = 0;
  for (int r0 = 0; r0 < rows; r0 += kReorderThreads, par ^= 1) {
    const int r = r0 + tid;
    uint8_t v[GPW];
    load_mask_bytes<GPW>(mb + (size_t)r * groups, ng, aligned8, r < rows, v);
    uint64_t bal[GPW];
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
      bal[j] = __ballot(v[j] != 0);
      if (lane == 0) s_cnt[par][j][wave] = __popcll(bal[j]);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
      int below = 0, chunk = 0;
      for (int w = 0; w < kReorderWaves; ++w) {
        const int c = s_cnt[par][j][w];
        below += (w < wave) ? c : 0;
        chunk += c;
      }
      if (r < rows && j < ng) {
        const int before = base[j] + below + rank_below(bal[j]);
        const int pos = v[j] ? before : total[j] + (r - before);
        perm[((size_t)b * groups + g0 + j) * rows + pos] = r;
      }
      base[j] += chunk;
    }
    // s_cnt[par] is rewritten two chunks later, after the next barrier.
  }
}

// The same partition for one column per workgroup with its rows held in
// registers (CH chunks of 512 rows, rows <= 512 CH): one round of mask loads
// instead of one per chunk and pass. Pass 1 stores the active count of every
// (chunk, wave); the counts become exclusive prefixes in LDS (chunk totals
// scanned over the chunks, then over the waves of a chunk), three barriers
// in all; pass 2 ranks each row within its wave from the ballot it recomputes
// from registers.
template <int CH>
__global__ __launch_bounds__(kReorderThreads) void reorder_reg_kernel(const uint8_t *__restrict__ mask,
                                                                      int rows, int groups,
                                                                      int32_t *__restrict__ perm,
                                                                      int32_t *__restrict__ counts) {
  const int b = blockIdx.y;
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const uint8_t *mb = mask + (size_t)b * rows * groups + g;

  __shared__ int s_c[CH][kReorderWaves];  // counts, then exclusive prefixes
  __shared__ int s_pre[CH + 1];           // active rows before chunk i; the total last

  bool v[CH];  // row i * 512 + tid is active
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int r = i * kReorderThreads + tid;
    v[i] = r < rows && mb[(size_t)r * groups] != 0;
  }
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = __popcll(__ballot(v[i]));
    if (lane == 0) s_c[i][wave] = c;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < CH; ++i) {
      s_pre[i] = run;
      for (int w = 0; w < kReorderWaves; ++w) run += s_c[i][w];
    }
    s_pre[CH] = run;
    counts[(size_t)b * groups + g] = run;
  }
  __syncthreads();
  for (int i = tid; i < CH; i += kReorderThreads) {
    int acc = s_pre[i];
    for (int w = 0; w < kReorderWaves; ++w) {
      const int c = s_c[i][w];
      s_c[i][w] = acc;
      acc += c;
    }
  }
  __syncthreads();
  int32_t *pg = perm + ((size_t)b * groups + g) * rows;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int r = i * kReorderThreads + tid;
    const uint64_t bal = __ballot(v[i]);
    if (r < rows) {
      const int before = s_c[i][wave] + rank_below(bal);
      pg[v[i] ? before : s_pre[CH] + (r - before)] = r;
    }
  }
}

int launch_reorder(const uint8_t *mask, int batch, int rows, int groups, int32_t *perm,
                   int32_t *counts, hipStream_t stream) {
  const dim3 block(kReorderThreads);
  if (rows <= 32 * kReorderThreads) {
    // One column per workgroup, rows in registers: the most workgroups (one
    // per column), and the per-row work of a workgroup stays small. Measured
    // against 2, 4 and 8 columns per workgroup: fastest at every size tried.
    const dim3 grid(groups, batch);
    if (rows <= 8 * kReorderThreads)
      hipLaunchKernelGGL(reorder_reg_kernel<8>, grid, block, 0, stream, mask, rows, groups, perm, counts);
    else if (rows <= 16 * kReorderThreads)
      hipLaunchKernelGGL(reorder_reg_kernel<16>, grid, block, 0, stream, mask, rows, groups, perm, counts);
    else
      hipLaunchKernelGGL(reorder_reg_kernel<32>, grid, block, 0, stream, mask, rows, groups, perm, counts);
  } else if (groups >= 16) {
    const dim3 grid((groups + 7) / 8, batch);
    hipLaunchKernelGGL(reorder_kernel<8>, grid, block, 0, stream, mask, rows, groups, perm, counts);
  } else {
    const dim3 grid(groups, batch);
    hipLaunchKernelGGL(reorder_kernel<1>, grid, block, 0, stream, mask, rows, groups, perm, counts);
  }
  return check_launch();
}

}  // namespace wide
