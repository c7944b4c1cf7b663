// Head-group-masked causal GQA attention on gfx950.
//
// WIDE (arXiv 2607.28418) section 3.1, Eq. 2 (the attention output is gated
// per GQA head group, K and V are never pruned) and Appendix B, Algorithm 4
// (sorted query tiles, gathered Q, dense K/V pipeline, online softmax on the
// active rows, causal key range cut at the largest active query position,
// scatter of the normalised rows).
//
// Prefill: a workgroup owns (batch b, query head h, sorted query tile) of 128
// rows taken from perm[b][g] with g = h / (Hq/Hk). Because perm lists active
// rows in ascending position, the tile's last active row bounds the causal
// key range and each wave's own last row bounds the tiles it must compute.
// Level 0: a tile past counts[b][g] exits. Level 1: only active Q rows are
// gathered. Level 2: a wave with no active row, or whose rows all precede a
// key tile, skips that tile's MFMAs.
// The score tile is computed transposed, S^T = K Q^T, with
// v_mfma_f32_16x16x32_bf16, so every lane holds one query's scores; the
// running max, the rescale of the output and the row sums are then lane-local
// except for two cross-lane max steps. P^T feeds the PV product straight from
// registers; V is staged transposed in LDS. Softmax runs in fp32 with exp2 and
// the scale folded with log2(e).
//
// Decode (Tq = 1): the reorder is bypassed and the routing byte (or count) is
// read per (b, g). A split-KV kernel lets the Hq/Hk heads of an active group
// share each K/V chunk and writes (max, sum, unnormalised output) partials; a
// second kernel merges the splits with log-sum-exp weights.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace wide {

constexpr int kAq = 128;            // sorted query rows per workgroup
constexpr int kAk = 64;             // keys per K/V tile
constexpr int kAd = 128;            // head size
constexpr int kAKLds = kAd + 8;     // sK row stride (bf16)
constexpr int kAVLds = kAk + 8;     // sVt row stride (bf16)
constexpr float kLog2e = 1.4426950408889634f;

template <bool OUT_F32>
__device__ __forceinline__ void store4(void *O, size_t idx, float a, float b, float c, float d) {
  if (OUT_F32) {
    *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(O) + idx) = f32x4{a, b, c, d};
  } else {
    u32x2 w = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
    *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(O) + idx) = w;
  }
}

template <bool OUT_F32>
__global__ __launch_bounds__(256, 2) void attn_prefill_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kAk * kAKLds];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[2][kAd * kAVLds];
  __shared__ int sPos[kAq];

  const int ntile = (a.Tq + kAq - 1) / kAq;
  const int tile = ntile - 1 - (int)blockIdx.x;  // later tiles see more keys: start them first
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int rep = a.Hq / a.Hk;
  const int g = h / rep;
  const int cnt = a.counts[(size_t)b * a.Hk + g];
  const int m0 = tile * kAq;
  if (m0 >= cnt) return;  // level 0
  const int rows = min(kAq, cnt - m0);
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;

  const int32_t *pg = a.perm + ((size_t)b * a.Hk + g) * a.Tq;
  if (tid < kAq) sPos[tid] = tid < rows ? pg[m0 + tid] : -1;
  __syncthreads();

  const int delta = a.Tk - a.Tq;
  const int jmin = a.leftpad ? a.leftpad[b] : 0;
  const int jmax = a.causal ? min(a.Tk, sPos[rows - 1] + delta + 1) : a.Tk;
  const int t_begin = jmin / kAk;
  const int t_end = jmax > jmin ? (jmax + kAk - 1) / kAk : t_begin;

  // This wave's 32 query rows.
  const int wrows = uniform(max(0, min(32, rows - wave * 32)));
  const int wjmax = wrows > 0 ? (a.causal ? min(a.Tk, sPos[wave * 32 + wrows - 1] + delta + 1) : a.Tk) : 0;
  int qpos[2];
#pragma unroll
  for (int qf = 0; qf < 2; ++qf) qpos[qf] = sPos[wave * 32 + qf * 16 + lane % 16];

  const size_t q_row = (size_t)a.Hq * kAd;       // elements between tokens of Q/O
  const size_t kv_row = (size_t)a.Hk * kAd;      // elements between tokens of K/V
  // Q, K and V of this batch as buffer resources: inactive query rows and keys
  // past Tk get out-of-range offsets (zeros, no traffic), so every load is
  // issued unconditionally.
  const rsrc_t q_rsrc = make_rsrc(a.Q + (size_t)b * a.Tq * q_row, (uint64_t)a.Tq * q_row * 2);
  const rsrc_t k_rsrc = make_rsrc(a.K + (size_t)b * a.Tk * kv_row, (uint64_t)a.Tk * kv_row * 2);
  const rsrc_t v_rsrc = make_rsrc(a.V + (size_t)b * a.Tk * kv_row, (uint64_t)a.Tk * kv_row * 2);
  u32x4 qreg[2][4];
#pragma unroll
  for (int qf = 0; qf < 2; ++qf)
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
      qreg[qf][ds] = buf_ld16(q_rsrc, qpos[qf] >= 0
          ? (uint32_t)(qpos[qf] * q_row + h * kAd + ds * 32 + (lane / 16) * 8) * 2u : kOffNone);

  // K/V tile loaders: K rows (tid/16 + 16p), V key pairs (2*(tid/16) + 32p, +1).
  const int kc = tid % 16;
  const int kr = tid / 16;
  const uint32_t kv_col = (uint32_t)(g * kAd + kc * 8) * 2u;
  u32x4 rk[4], rv[4];
  auto gload = [&](int t) {
    const int j0 = t * kAk;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int j = j0 + kr + 16 * p;
      rk[p] = buf_ld16(k_rsrc, j < a.Tk ? (uint32_t)j * (uint32_t)kv_row * 2u + kv_col : kOffNone);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int j = j0 + 32 * (p / 2) + 2 * kr + (p % 2);
      rv[p] = buf_ld16(v_rsrc, j < a.Tk ? (uint32_t)j * (uint32_t)kv_row * 2u + kv_col : kOffNone);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < 4; ++p) st16(&sK[buf][(kr + 16 * p) * kAKLds + kc * 8], rk[p]);
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const u32x4 e0 = rv[2 * pp], e1 = rv[2 * pp + 1];
      uint32_t *dst = reinterpret_cast<uint32_t *>(&sVt[buf][(kc * 8) * kAVLds + 32 * pp + 2 * kr]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = (e % 2) ? (e0[e / 2] >> 16) : (e0[e / 2] & 0xffffu);
        const uint32_t hi = (e % 2) ? (e1[e / 2] & 0xffff0000u) : (e1[e / 2] << 16);
        dst[e * (kAVLds / 2)] = lo | hi;
      }
    }
  };

  const float sl2 = a.scale * kLog2e;
  float mrun[2] = {-INFINITY, -INFINITY};
  float zpart[2] = {0.f, 0.f};
  f32x4 oacc[8][2];
#pragma unroll
  for (int df = 0; df < 8; ++df)
#pragma unroll
    for (int qf = 0; qf < 2; ++qf) oacc[df][qf] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (t_begin < t_end) {
    gload(t_begin);
    lstore(0);
  }
  __syncthreads();
  for (int t = t_begin; t < t_end; ++t) {
    const int cur = (t - t_begin) & 1;
    if (t + 1 < t_end) gload(t + 1);
    const int j0 = t * kAk;
    if (j0 < wjmax) {  // level 2: the wave's rows see some key of this tile
      f32x4 s[4][2];
#pragma unroll
      for (int kf = 0; kf < 4; ++kf)
#pragma unroll
        for (int qf = 0; qf < 2; ++qf) s[kf][qf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
#pragma unroll
        for (int kf = 0; kf < 4; ++kf) {
          const u32x4 kfrag = ld16(&sK[cur][(kf * 16 + lane % 16) * kAKLds + ds * 32 + (lane / 16) * 8]);
#pragma unroll
          for (int qf = 0; qf < 2; ++qf) s[kf][qf] = mfma16x16x32(kfrag, qreg[qf][ds], s[kf][qf]);
        }
      }
      // Mask, scale, online softmax (log2 domain).
#pragma unroll
      for (int qf = 0; qf < 2; ++qf) {
        const int lim = a.causal ? qpos[qf] + delta : a.Tk - 1;
        float rmax = -INFINITY;
#pragma unroll
        for (int kf = 0; kf < 4; ++kf)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int j = j0 + kf * 16 + 4 * (lane / 16) + v;
            const bool ok = qpos[qf] >= 0 && j >= jmin && j <= lim && j < a.Tk;
            const float x = ok ? s[kf][qf][v] * sl2 : -INFINITY;
            s[kf][qf][v] = x;
            rmax = fmaxf(rmax, x);
          }
        rmax = fmaxf(rmax, __shfl_xor(rmax, 16, kWave));
        rmax = fmaxf(rmax, __shfl_xor(rmax, 32, kWave));
        const float mnew = fmaxf(mrun[qf], rmax);
        const float muse = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = exp2f(mrun[qf] - muse);
        mrun[qf] = mnew;
        float psum = 0.f;
#pragma unroll
        for (int kf = 0; kf < 4; ++kf)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float p = exp2f(s[kf][qf][v] - muse);
            s[kf][qf][v] = p;
            psum += p;
          }
        zpart[qf] = zpart[qf] * alpha + psum;
#pragma unroll
        for (int df = 0; df < 8; ++df) oacc[df][qf] *= alpha;
      }
      // O^T += V^T P^T over two 32-key steps.
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 pb[2];
#pragma unroll
        for (int qf = 0; qf < 2; ++qf) {
          const f32x4 lo = s[2 * ks][qf], hi = s[2 * ks + 1][qf];
          pb[qf] = u32x4{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                         pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])};
        }
#pragma unroll
        for (int df = 0; df < 8; ++df) {
          const uint16_t *vrow = &sVt[cur][(df * 16 + lane % 16) * kAVLds + ks * 32 + 4 * (lane / 16)];
          const u32x2 lo = *reinterpret_cast<const u32x2 *>(vrow);
          const u32x2 hi = *reinterpret_cast<const u32x2 *>(vrow + 16);
          const u32x4 vfrag = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
          for (int qf = 0; qf < 2; ++qf) oacc[df][qf] = mfma16x16x32(vfrag, pb[qf], oacc[df][qf]);
        }
      }
    }
    if (t + 1 < t_end) lstore(cur ^ 1);
    __syncthreads();
  }

  // Normalise and scatter the active rows to O[b][t][h][:].
  uint16_t *Ob16 = nullptr;
  (void)Ob16;
#pragma unroll
  for (int qf = 0; qf < 2; ++qf) {
    float z = zpart[qf];
    z += __shfl_xor(z, 16, kWave);
    z += __shfl_xor(z, 32, kWave);
    if (qpos[qf] < 0) continue;
    const float inv = z > 0.f ? 1.f / z : 0.f;
    const size_t obase = ((size_t)b * a.Tq + qpos[qf]) * q_row + (size_t)h * kAd;
#pragma unroll
    for (int df = 0; df < 8; ++df) {
      const f32x4 o = oacc[df][qf] * inv;
      store4<OUT_F32>(a.O, obase + df * 16 + 4 * (lane / 16), o[0], o[1], o[2], o[3]);
    }
  }
}

// ---------------------------------------------------------------------------
// Decode: split-KV partials + merge.
// ---------------------------------------------------------------------------

constexpr int kDecKeys = 256;      // keys per split
constexpr int kDecMaxRep = 8;      // query heads per KV head supported
constexpr int kDecPart = kAd + 4;  // floats per partial: o[128], m, z (+pad)

__device__ __forceinline__ bool group_active(const AttnArgs &a, int b, int g) {
  if (a.mask) return a.mask[(size_t)b * a.Hk + g] != 0;
  return a.counts[(size_t)b * a.Hk + g] > 0;
}

__global__ __launch_bounds__(256) void attn_decode_split_kernel(AttnArgs a, int nsplit) {
  __shared__ float sQ[kDecMaxRep][kAd];
  __shared__ float sP[kDecMaxRep][kDecKeys];
  __shared__ float sRed[kDecMaxRep][4];
  __shared__ float sO[4][kDecMaxRep][kAd];

  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  if (!group_active(a, b, g)) return;  // the group is off for this token: nothing is read
  const int rep = a.Hq / a.Hk;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int jmin = a.leftpad ? a.leftpad[b] : 0;
  const int j0 = split * kDecKeys;
  const int jlo = max(j0, jmin);
  const int jhi = min(j0 + kDecKeys, a.Tk);  // Tq = 1: every key precedes the query
  float *ws = reinterpret_cast<float *>(a.workspace);
  const size_t q_row = (size_t)a.Hq * kAd, kv_row = (size_t)a.Hk * kAd;

  if (jlo >= jhi) {
    if (tid < rep) {
      float *part = ws + (((size_t)b * a.Hq + g * rep + tid) * nsplit + split) * kDecPart;
      part[kAd] = -INFINITY;
      part[kAd + 1] = 0.f;
    }
    return;
  }

  const uint16_t *Qb = a.Q + (size_t)b * q_row + (size_t)g * rep * kAd;
  for (int i = tid; i < rep * kAd; i += 256) sQ[i / kAd][i % kAd] = bf2f(Qb[i]);
  __syncthreads();

  // Scores: one key per thread.
  const float sl2 = a.scale * kLog2e;
  const int j = j0 + tid;
  const bool ok = j >= jlo && j < jhi;
  float sc[kDecMaxRep];
#pragma unroll
  for (int r = 0; r < kDecMaxRep; ++r) sc[r] = 0.f;
  if (ok) {
    const uint16_t *krow = a.K + ((size_t)b * a.Tk + j) * kv_row + (size_t)g * kAd;
#pragma unroll 4
    for (int c = 0; c < kAd / 8; ++c) {
      const u32x4 w = ld16(krow + c * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float kv = (e % 2) ? bf_hi(w[e / 2]) : bf_lo(w[e / 2]);
#pragma unroll
        for (int r = 0; r < kDecMaxRep; ++r)
          if (r < rep) sc[r] = fmaf(kv, sQ[r][c * 8 + e], sc[r]);
      }
    }
  }
  // Block max and sum per head.
  float mx[kDecMaxRep];
#pragma unroll
  for (int r = 0; r < kDecMaxRep; ++r) {
    sc[r] = ok ? sc[r] * sl2 : -INFINITY;
    float v = sc[r];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    if (lane == 0) sRed[r][wave] = v;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kDecMaxRep; ++r) {
    mx[r] = fmaxf(fmaxf(sRed[r][0], sRed[r][1]), fmaxf(sRed[r][2], sRed[r][3]));
    const float p = ok ? exp2f(sc[r] - mx[r]) : 0.f;
    if (r < rep) sP[r][tid] = p;
  }
  __syncthreads();
  float zs[kDecMaxRep];
#pragma unroll
  for (int r = 0; r < kDecMaxRep; ++r) {
    float v = (r < rep) ? sP[r][tid] : 0.f;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    zs[r] = v;
  }
  __syncthreads();
  if (lane == 0)
#pragma unroll
    for (int r = 0; r < kDecMaxRep; ++r) sRed[r][wave] = zs[r];

  // Unnormalised output: thread = (dim pair, quarter of the keys).
  const int dp = tid % 64, kq = tid / 64;
  float o0[kDecMaxRep], o1[kDecMaxRep];
#pragma unroll
  for (int r = 0; r < kDecMaxRep; ++r) o0[r] = o1[r] = 0.f;
  const int kb = j0 + kq * 64;
  for (int jj = 0; jj < 64; ++jj) {
    const int jk = kb + jj;
    if (jk < jlo || jk >= jhi) continue;
    const uint32_t w = *reinterpret_cast<const uint32_t *>(a.V + ((size_t)b * a.Tk + jk) * kv_row +
                                                          (size_t)g * kAd + 2 * dp);
    const float v0 = bf_lo(w), v1 = bf_hi(w);
#pragma unroll
    for (int r = 0; r < kDecMaxRep; ++r) {
      if (r >= rep) break;
      const float p = sP[r][kq * 64 + jj];
      o0[r] = fmaf(p, v0, o0[r]);
      o1[r] = fmaf(p, v1, o1[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < kDecMaxRep; ++r) {
    if (r >= rep) break;
    sO[kq][r][2 * dp] = o0[r];
    sO[kq][r][2 * dp + 1] = o1[r];
  }
  __syncthreads();
  for (int i = tid; i < rep * kAd; i += 256) {
    const int r = i / kAd, d = i % kAd;
    float *part = ws + (((size_t)b * a.Hq + g * rep + r) * nsplit + split) * kDecPart;
    part[d] = sO[0][r][d] + sO[1][r][d] + sO[2][r][d] + sO[3][r][d];
    if (d == 0) {
      part[kAd] = mx[r];
      part[kAd + 1] = sRed[r][0] + sRed[r][1] + sRed[r][2] + sRed[r][3];
    }
  }
}

template <bool OUT_F32>
__global__ __launch_bounds__(kAd) void attn_decode_merge_kernel(AttnArgs a, int nsplit) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int rep = a.Hq / a.Hk;
  if (!group_active(a, b, h / rep)) return;
  const int d = threadIdx.x;
  const float *ws = reinterpret_cast<const float *>(a.workspace) + ((size_t)b * a.Hq + h) * nsplit * kDecPart;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ws[s * kDecPart + kAd]);
  float Z = 0.f, o = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < nsplit; ++s) {
      const float m = ws[s * kDecPart + kAd];
      if (m == -INFINITY) continue;
      const float w = exp2f(m - M);
      Z += w * ws[s * kDecPart + kAd + 1];
      o += w * ws[s * kDecPart + d];
    }
  }
  const float out = Z > 0.f ? o / Z : 0.f;
  const size_t idx = (size_t)b * a.Hq * kAd + (size_t)h * kAd + d;
  if (OUT_F32)
    reinterpret_cast<float *>(a.O)[idx] = out;
  else
    reinterpret_cast<uint16_t *>(a.O)[idx] = f2bf(out);
}

size_t attn_workspace_bytes(int64_t B, int64_t Tq, int64_t Tk, int64_t Hq, int64_t Hk, int64_t d) {
  (void)Hk;
  (void)d;
  if (Tq != 1) return 0;
  const int64_t nsplit = (Tk + kDecKeys - 1) / kDecKeys;
  return (size_t)B * Hq * nsplit * kDecPart * sizeof(float);
}

int launch_attn(const AttnArgs &a, hipStream_t s) {
  if (a.Tq == 1) {
    const int nsplit = (a.Tk + kDecKeys - 1) / kDecKeys;
    hipLaunchKernelGGL(attn_decode_split_kernel, dim3(nsplit, a.Hk, a.B), dim3(256), 0, s, a, nsplit);
    if (a.o_f32)
      hipLaunchKernelGGL(attn_decode_merge_kernel<true>, dim3(a.Hq, a.B), dim3(kAd), 0, s, a, nsplit);
    else
      hipLaunchKernelGGL(attn_decode_merge_kernel<false>, dim3(a.Hq, a.B), dim3(kAd), 0, s, a, nsplit);
    return check_launch();
  }
  dim3 grid((a.Tq + kAq - 1) / kAq, a.Hq, a.B);
  if (a.o_f32)
    hipLaunchKernelGGL(attn_prefill_kernel<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attn_prefill_kernel<false>, grid, dim3(256), 0, s, a);
  return check_launch();
}

}  // namespace wide
