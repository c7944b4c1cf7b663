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
constexpr int kDecPart = kAd + 4;  // floats per partial: o[128], m, z (+pad)

__device__ __forceinline__ bool group_active(const AttnArgs &a, int b, int g) {
  if (a.mask) return a.mask[(size_t)b * a.Hk + g] != 0;
  return a.counts[(size_t)b * a.Hk + g] > 0;
}

// One split = 256 keys of one active (b, g), for all Hq/Hk heads of the
// group. Lane l of a wave handles key quad slot l / 16 and head-dim chunk
// l % 16 (8 values), so every 16-byte load of K and V covers whole lines of
// four key rows; the 16 K loads and 16 V loads of a lane are issued before
// any is used. Scores are reduced over the 16 lanes of a key, then the
// split's max and sum per head come from an LDS reduction; the unnormalised
// output is reduced over the key slots of a wave and then over the waves.
template <int RMAX>
__global__ __launch_bounds__(256) void attn_decode_split_kernel(AttnArgs a, int nsplit) {
  constexpr int IT = kDecKeys / 16;  // key quads per wave (16 x 4 = 64 keys)
  __shared__ float sP[RMAX][kDecKeys];
  __shared__ float sRed[RMAX][4];
  __shared__ float sO[4][RMAX][kAd];

  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  if (!group_active(a, b, g)) return;  // the group is off for this token: nothing is read
  const int rep = a.Hq / a.Hk;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int kq = lane / 16, dc = lane % 16;
  const int jmin = a.leftpad ? a.leftpad[b] : 0;
  const int j0 = split * kDecKeys;
  const int jlo = max(j0, jmin);
  const int jhi = min(j0 + kDecKeys, a.Tk);  // Tq = 1: every key precedes the query
  float *ws = reinterpret_cast<float *>(a.workspace);
  const size_t q_row = (size_t)a.Hq * kAd, kv_row = (size_t)a.Hk * kAd;

  if (jlo >= jhi) {  // every key of the split is before the sequence's left padding
    for (int i = tid; i < rep * kDecPart; i += 256) {
      const int r = i / kDecPart, c = i % kDecPart;
      float *part = ws + (((size_t)b * a.Hq + g * rep + r) * nsplit + split) * kDecPart;
      part[c] = c == kAd ? -INFINITY : 0.f;
    }
    return;
  }

  const rsrc_t kr = make_rsrc(a.K + (size_t)b * a.Tk * kv_row, (uint64_t)a.Tk * kv_row * 2);
  const rsrc_t vr = make_rsrc(a.V + (size_t)b * a.Tk * kv_row, (uint64_t)a.Tk * kv_row * 2);
  u32x4 kreg[IT], vreg[IT];
  bool kok[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int j = j0 + wave * (kDecKeys / 4) + i * 4 + kq;
    kok[i] = j >= jlo && j < jhi;
    const uint32_t off = kok[i] ? (uint32_t)((size_t)j * kv_row + g * kAd + dc * 8) * 2u : kOffNone;
    kreg[i] = buf_ld16(kr, off);
  }
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int j = j0 + wave * (kDecKeys / 4) + i * 4 + kq;
    const uint32_t off = kok[i] ? (uint32_t)((size_t)j * kv_row + g * kAd + dc * 8) * 2u : kOffNone;
    vreg[i] = buf_ld16(vr, off);
  }
  // This lane's 8 query values for every head of the group.
  const uint16_t *Qb = a.Q + (size_t)b * q_row + (size_t)g * rep * kAd + dc * 8;
  float qv[RMAX][8];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    const u32x4 w = r < rep ? ld16(Qb + r * kAd) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[r][e] = (e % 2) ? bf_hi(w[e / 2]) : bf_lo(w[e / 2]);
  }

  // Scores (log2 domain): dot over this lane's chunk, then over the 16 lanes of the key.
  const float sl2 = a.scale * kLog2e;
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    float sc[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((e % 2) ? bf_hi(kreg[i][e / 2]) : bf_lo(kreg[i][e / 2]), qv[r][e], acc);
      sc[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      if (r >= rep) break;
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) sc[r] += __shfl_xor(sc[r], o, kWave);
    }
    if (dc == 0) {
      const int jl = wave * (kDecKeys / 4) + i * 4 + kq;
#pragma unroll
      for (int r = 0; r < RMAX; ++r)
        if (r < rep) sP[r][jl] = kok[i] ? sc[r] * sl2 : -INFINITY;
    }
  }
  __syncthreads();
  // Split max and sum per head: thread t owns key t.
  float mx[RMAX], zs[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    float v = r < rep ? sP[r][tid] : -INFINITY;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    if (lane == 0) sRed[r][wave] = v;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    mx[r] = fmaxf(fmaxf(sRed[r][0], sRed[r][1]), fmaxf(sRed[r][2], sRed[r][3]));
    if (r < rep) {
      const float p = exp2f(sP[r][tid] - mx[r]);  // -inf -> 0; the split has a valid key
      sP[r][tid] = p;
      zs[r] = p;
    } else {
      zs[r] = 0.f;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) zs[r] += __shfl_xor(zs[r], o, kWave);
  }
  if (lane == 0)
#pragma unroll
    for (int r = 0; r < RMAX; ++r) sRed[r][wave] = zs[r];

  // Unnormalised output for this lane's chunk, over this wave's keys.
  float o[RMAX][8];
#pragma unroll
  for (int r = 0; r < RMAX; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[r][e] = 0.f;
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int jl = wave * (kDecKeys / 4) + i * 4 + kq;
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      if (r >= rep) break;
      const float p = sP[r][jl];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[r][e] = fmaf(p, (e % 2) ? bf_hi(vreg[i][e / 2]) : bf_lo(vreg[i][e / 2]), o[r][e]);
    }
  }
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    if (r >= rep) break;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[r][e] += __shfl_xor(o[r][e], 16, kWave);
      o[r][e] += __shfl_xor(o[r][e], 32, kWave);
    }
    if (kq == 0)
#pragma unroll
      for (int e = 0; e < 8; ++e) sO[wave][r][dc * 8 + e] = o[r][e];
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

// Merge of the splits of one (b, h): weights 2^(m_s - max) from the split
// maxima (staged in LDS), then the weighted sum of the partial outputs with
// the reads unrolled.
template <bool OUT_F32>
__global__ __launch_bounds__(kAd) void attn_decode_merge_kernel(AttnArgs a, int nsplit) {
  __shared__ float sW[1024];
  __shared__ float sZ;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int rep = a.Hq / a.Hk;
  if (!group_active(a, b, h / rep)) return;
  const int d = threadIdx.x;
  const float *ws = reinterpret_cast<const float *>(a.workspace) + ((size_t)b * a.Hq + h) * nsplit * kDecPart;
  // split maxima -> LDS, global max, weights
  for (int s = d; s < nsplit; s += kAd) sW[s] = ws[s * kDecPart + kAd];
  __syncthreads();
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, sW[s]);
  __syncthreads();
  for (int s = d; s < nsplit; s += kAd) {
    const float m = sW[s];
    sW[s] = (M == -INFINITY || m == -INFINITY) ? 0.f : exp2f(m - M);
  }
  __syncthreads();
  if (d == 0) {
    float Z = 0.f;
    for (int s = 0; s < nsplit; ++s) Z += sW[s] * ws[s * kDecPart + kAd + 1];
    sZ = Z;
  }
  float o = 0.f;
  int s = 0;
  for (; s + 8 <= nsplit; s += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = ws[(s + u) * kDecPart + d];
#pragma unroll
    for (int u = 0; u < 8; ++u) o = fmaf(sW[s + u], v[u], o);
  }
  for (; s < nsplit; ++s) o = fmaf(sW[s], ws[s * kDecPart + d], o);
  __syncthreads();
  const float Z = sZ;
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
    const dim3 grid(nsplit, a.Hk, a.B);
    const int rep = a.Hq / a.Hk;
    if (rep == 1)
      hipLaunchKernelGGL(attn_decode_split_kernel<1>, grid, dim3(256), 0, s, a, nsplit);
    else if (rep == 2)
      hipLaunchKernelGGL(attn_decode_split_kernel<2>, grid, dim3(256), 0, s, a, nsplit);
    else if (rep <= 4)
      hipLaunchKernelGGL(attn_decode_split_kernel<4>, grid, dim3(256), 0, s, a, nsplit);
    else
      hipLaunchKernelGGL(attn_decode_split_kernel<8>, grid, dim3(256), 0, s, a, nsplit);
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
