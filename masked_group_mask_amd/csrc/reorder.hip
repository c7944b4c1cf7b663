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

// The same partition with every row of the workgroup's columns held in
// registers (CH chunks of 512 rows, rows <= 512 CH): one round of mask loads
// instead of one per chunk and pass. Pass 1 stores the active count of every
// (chunk, column, wave); the counts become exclusive prefixes in LDS (chunk
// totals scanned over chunks, then over the waves of a chunk), three
// barriers in all; pass 2 ranks each row within its wave from the ballot it
// recomputes from registers.
template <int GPW, int CH>
__global__ __launch_bounds__(kReorderThreads) void reorder_reg_kernel(const uint8_t *__restrict__ mask,
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

  __shared__ int s_c[CH][GPW][kReorderWaves];  // counts, then exclusive prefixes
  __shared__ int s_pre[CH + 1][GPW];           // active rows before chunk i

  uint64_t v[CH];  // byte j = column g0 + j of row i * 512 + tid
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    uint8_t by[GPW];
    const int r = i * kReorderThreads + tid;
    load_mask_bytes<GPW>(mb + (size_t)r * groups, ng, aligned8, r < rows, by);
    uint64_t w = 0;
#pragma unroll
    for (int j = 0; j < GPW; ++j) w |= (uint64_t)(by[j] != 0) << (8 * j);
    v[i] = w;
  }
#pragma unroll
  for (int i = 0; i < CH; ++i)
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
      const int c = __popcll(__ballot((v[i] >> (8 * j)) & 1));
      if (lane == 0) s_c[i][j][wave] = c;
    }
  __syncthreads();
  if (tid < GPW) {
    int run = 0;
    for (int i = 0; i < CH; ++i) {
      s_pre[i][tid] = run;
      for (int w = 0; w < kReorderWaves; ++w) run += s_c[i][tid][w];
    }
    s_pre[CH][tid] = run;
    if (tid < ng) counts[(size_t)b * groups + g0 + tid] = run;
  }
  __syncthreads();
  for (int k = tid; k < CH * GPW; k += kReorderThreads) {
    const int i = k / GPW, j = k % GPW;
    int acc = s_pre[i][j];
    for (int w = 0; w < kReorderWaves; ++w) {
      const int c = s_c[i][j][w];
      s_c[i][j][w] = acc;
      acc += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int r = i * kReorderThreads + tid;
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
      const bool act = (v[i] >> (8 * j)) & 1;
      const uint64_t bal = __ballot(act);
      if (r < rows && j < ng) {
        const int before = s_c[i][j][wave] + rank_below(bal);
        const int pos = act ? before : s_pre[CH][j] + (r - before);
        perm[((size_t)b * groups + g0 + j) * rows + pos] = r;
      }
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
      hipLaunchKernelGGL((reorder_reg_kernel<1, 8>), grid, block, 0, stream, mask, rows, groups, perm, counts);
    else if (rows <= 16 * kReorderThreads)
      hipLaunchKernelGGL((reorder_reg_kernel<1, 16>), grid, block, 0, stream, mask, rows, groups, perm, counts);
    else
      hipLaunchKernelGGL((reorder_reg_kernel<1, 32>), grid, block, 0, stream, mask, rows, groups, perm, counts);
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
