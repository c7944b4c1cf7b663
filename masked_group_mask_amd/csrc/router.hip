// Token-level group router on the GPU ("WIDE: Boosting Adaptive LLM Inference
// via Token-level Dynamic Width Pruning", section 3.1 "Routing Components",
// Eq. 4 and 5): the bottleneck logits R = X W1 W2, paired per group, and the
// inference decision "class 0 is the argmax" (a tie keeps class 0). The mask
// it writes feeds the reorder directly, so the routing decision never leaves
// the device.
#include "common.hpp"
#include "launch.hpp"

namespace wide {

constexpr int kRtTok = 32;    // tokens per workgroup
constexpr int kRtWaves = 4;   // waves per workgroup; they split the reduction over D
constexpr int kRtU = 4;       // 32-deep chunks per wave per batch of loads

// Workgroup = 32 consecutive tokens. Stage 1, H = X W1^T (32 x r, fp32): wave
// w takes the 32-deep chunks w, w + 4, ... of D; per chunk its lanes load the
// X fragments of the two 16-token blocks and the W1 fragments of the r/16
// output blocks straight into registers (16 bytes per lane: 64 contiguous
// bytes of 16 rows per load) and run 16x16x32 bf16 MFMAs. The four partial H
// are summed in LDS. Stage 2, R = H W2^T: thread p takes (token, group)
// pairs; W2 sits in LDS transposed ([r][2 N_G]) so a lane reads the two
// classes of its group as one 32-bit word, consecutive lanes on consecutive
// words. Each logit is an fp32 chain over j = 0 .. r-1 in order.
template <int R16>
__global__ __launch_bounds__(kRtWaves * kWave) void router_kernel(RouterArgs a) {
  constexpr int R = 16 * R16;
  extern __shared__ __attribute__((aligned(16))) uint16_t sW2T[];  // [R][2 NG]
  __shared__ float sH[kRtWaves][kRtTok][R + 1];
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int t0 = blockIdx.x * kRtTok;
  const int NG2 = 2 * a.groups;

  // W2 [2 NG][R] -> LDS [R][2 NG].
  for (int i = tid; i < NG2 * R16 * 2; i += kRtWaves * kWave) {
    const int n = i / (R / 8), j0 = (i % (R / 8)) * 8;
    const u32x4 w = ld16(a.W2 + (size_t)n * R + j0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sW2T[(j0 + 2 * e) * NG2 + n] = (uint16_t)(w[e] & 0xffffu);
      sW2T[(j0 + 2 * e + 1) * NG2 + n] = (uint16_t)(w[e] >> 16);
    }
  }

  const rsrc_t xr = make_rsrc(a.X, (uint64_t)a.M * a.ldx * 2);
  const rsrc_t wr = make_rsrc(a.W1, (uint64_t)R * a.D * 2);
  const int nch = (a.D + 31) / 32;
  const int kq = 8 * (lane / 16);
  f32x4 acc[2][R16];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int nb = 0; nb < R16; ++nb) acc[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  bool rowok[2];
  uint32_t rowoff[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int t = t0 + rb * 16 + lane % 16;
    rowok[rb] = t < a.M;
    rowoff[rb] = (uint32_t)((size_t)t * a.ldx * 2);
  }
  for (int c0 = wave; c0 < nch; c0 += kRtWaves * kRtU) {
    u32x4 xa[kRtU][2], wb[kRtU][R16];
#pragma unroll
    for (int u = 0; u < kRtU; ++u) {
      const int k = 32 * (c0 + kRtWaves * u) + kq;
      const bool kok = k < a.D;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        xa[u][rb] = buf_ld16(xr, kok && rowok[rb] ? rowoff[rb] + (uint32_t)k * 2u : kOffNone);
#pragma unroll
      for (int nb = 0; nb < R16; ++nb)
        wb[u][nb] = buf_ld16(wr, kok ? (uint32_t)(((nb * 16 + lane % 16) * a.D + k) * 2) : kOffNone);
    }
#pragma unroll
    for (int u = 0; u < kRtU; ++u)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int nb = 0; nb < R16; ++nb) acc[rb][nb] = mfma16x16x32(xa[u][rb], wb[u][nb], acc[rb][nb]);
  }
  // Lane l holds H[token 16 rb + 4 (l / 16) + v][j = 16 nb + l % 16].
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int nb = 0; nb < R16; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) sH[wave][rb * 16 + 4 * (lane / 16) + v][nb * 16 + lane % 16] = acc[rb][nb][v];
  __syncthreads();
  for (int i = tid; i < kRtTok * R; i += kRtWaves * kWave) {
    const int t = i / R, j = i % R;
    sH[0][t][j] = (sH[0][t][j] + sH[1][t][j]) + (sH[2][t][j] + sH[3][t][j]);
  }
  __syncthreads();

  const int ntok = min(kRtTok, a.M - t0);
  const uint32_t *w2p = reinterpret_cast<const uint32_t *>(sW2T);  // (class 0, class 1) of a group
  for (int p = tid; p < ntok * a.groups; p += kRtWaves * kWave) {
    const int t = p / a.groups, g = p % a.groups;
    float r0 = 0.f, r1 = 0.f;
#pragma unroll 8
    for (int j = 0; j < R; ++j) {
      const float h = sH[0][t][j];
      const uint32_t w = w2p[j * a.groups + g];
      r0 = fmaf(h, bf_lo(w), r0);
      r1 = fmaf(h, bf_hi(w), r1);
    }
    const size_t row = (size_t)(t0 + t);
    a.mask[row * a.groups + g] = r0 >= r1 ? 1 : 0;  // argmax is class 0 (ties included): run the group
    if (a.logits) *reinterpret_cast<f32x2 *>(a.logits + row * NG2 + 2 * g) = f32x2{r0, r1};
  }
}

int launch_router(const RouterArgs &a, hipStream_t s) {
  const dim3 grid((a.M + kRtTok - 1) / kRtTok), block(kRtWaves * kWave);
  const size_t lds = (size_t)2 * a.groups * a.r * sizeof(uint16_t);
  switch (a.r / 16) {
    case 1: hipLaunchKernelGGL(router_kernel<1>, grid, block, lds, s, a); break;
    case 2: hipLaunchKernelGGL(router_kernel<2>, grid, block, lds, s, a); break;
    case 3: hipLaunchKernelGGL(router_kernel<3>, grid, block, lds, s, a); break;
    default: hipLaunchKernelGGL(router_kernel<4>, grid, block, lds, s, a); break;
  }
  const int st = check_launch();
  if (st != WIDE_OK || a.perm == nullptr) return st;
  return launch_reorder(a.mask, a.batch, a.rows, a.groups, a.perm, a.counts, s);
}

}  // namespace wide
