// Head-group-masked causal GQA attention on gfx950.
//
// WIDE (arXiv 2607.28418) section 3.1, Eq. 2 (the attention output is gated
// per GQA head group, K and V are never pruned) and Appendix B, Algorithm 4
// (sorted query tiles, gathered Q, dense K/V pipeline, online softmax on the
// active rows, causal key range cut at the largest active query position,
// scatter of the normalised rows).
//
// Prefill: a workgroup owns (batch b, query head h, sorted query tile) of 256
// rows taken from perm[b][grp] of the head's routing group grp = h / (Hq/NG)
// (NG = Hk by default: one group per KV head; finer sub-GQA groups down to one
// head each); the head reads KV head h / (Hq/Hk). Because perm lists active
// rows in ascending position, the tile's last active row bounds the causal
// key range and each wave's own last row bounds the tiles it must compute.
// Level 0: a tile past counts[b][grp] exits. Level 1: only active Q rows are
// gathered. Level 2: a wave with no active row, or whose rows all precede a
// key tile, skips that tile's MFMAs.
// The score tile is computed transposed, S^T = K Q^T, with
// v_mfma_f32_16x16x32_bf16, so every lane holds one query's scores; the
// running max, the rescale of the output and the row sums are then lane-local
// except for two cross-lane max steps. P^T feeds the PV product straight from
// registers; V is staged in LDS as loaded and its transposed fragments come
// from the gfx950 transposing LDS read. Softmax runs in fp32 with exp2 and
// the scale folded with log2(e).
//
// Decode (Tq = 1): the reorder is bypassed and the routing byte (or count) is
// read per (b, group). A split-KV kernel (one wave per 64 keys of a KV head)
// serves all query heads of the KV head at once on the matrix cores and
// writes (max, sum, unnormalised output) partials; a second kernel merges the
// splits of each active head with log-sum-exp weights.
#include <math.h>

#include <mutex>

#include "common.hpp"
#include "launch.hpp"
#include "mma_engine.hpp"

namespace wide {

constexpr int kAWaves = 8;             // two waves per SIMD
constexpr int kAQB = 2;                // 16-query blocks per wave
constexpr int kAqw = 16 * kAQB;        // queries per wave
constexpr int kAq = kAWaves * kAqw;    // sorted query rows per workgroup
constexpr int kAThreads = 64 * kAWaves;
constexpr int kAk = 64;    // keys per K/V stage
constexpr int kAd = 128;   // head size
constexpr int kAStage = kAk * kAd;  // bf16 elements of one K (or V) stage
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.f;  // log2 of the largest p the prefill softmax lets through unrescaled

template <bool OUT_F32>
__device__ __forceinline__ void store4(void *O, size_t idx, float a, float b, float c, float d) {
  if (OUT_F32) {
    *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(O) + idx) = f32x4{a, b, c, d};
  } else {
    u32x2 w = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
    *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(O) + idx) = w;
  }
}

// Stage layouts (row = key, 256 bytes = 16 chunks of 16 bytes):
//   K: chunk c of row r at position c ^ (r % 16): the 16 rows one K fragment
//      read touches (same chunk) hit 16 distinct positions;
//   V: chunk c of row r at position c ^ 2 (r % 8): a transposing read takes
//      a 32-byte chunk pair from 8 rows per half wave, on distinct positions.
__device__ __forceinline__ int k_swz(int r) { return r & 15; }
__device__ __forceinline__ int v_swz(int r) { return (r & 7) << 1; }

// Max and sum over the lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four lanes
// that hold keys of one query) with gfx950's lane-swap instructions instead of
// LDS permutes: swapping a register with itself across lane halves (16 within
// each 32, or 32) leaves, in the two results, lane l's own value and its
// partner's, in some order, so one max or add finishes each step.
__device__ __forceinline__ void swap16(float x, float &u, float &v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  u = __uint_as_float(r[0]);
  v = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float x, float &u, float &v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  u = __uint_as_float(r[0]);
  v = __uint_as_float(r[1]);
}
// max(a, b, c) as one instruction. Written out because the compiler's own
// fmaxf first quiets each operand that does not come from an arithmetic op
// (here the MFMA results), one extra instruction per operand; the scores are
// never signalling NaNs.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float quad_max(float x) {
  float u, v;
  swap16(x, u, v);
  swap32(max3(u, v, v), u, v);
  return max3(u, v, v);
}
__device__ __forceinline__ float quad_sum(float x) {
  float u, v;
  swap16(x, u, v);
  swap32(u + v, u, v);
  return u + v;
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// gfx950 transposing LDS read: within each 16-lane group, lane i receives
// element i % 4 of the 8 bytes addressed by lane 4j + i / 4, for j = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const WIDE_LDS uint16_t *p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((WIDE_LDS i16x4 *)p);
  return __builtin_bit_cast(u32x2, v);
}

// Prefill: workgroup = (query head h, sorted query tile, batch b); the tile is
// 256 consecutive entries of perm[b][g], wave w owning entries 64w .. 64w+63.
template <bool OUT_F32>
__global__ __launch_bounds__(kAThreads) void attn_prefill_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) uint16_t sK0[kAStage];
  __shared__ __attribute__((aligned(1024))) uint16_t sV0[kAStage];
  __shared__ __attribute__((aligned(1024))) uint16_t sK1[kAStage];
  __shared__ __attribute__((aligned(1024))) uint16_t sV1[kAStage];
  __shared__ __attribute__((aligned(1024))) uint16_t sK2[kAStage];
  __shared__ __attribute__((aligned(1024))) uint16_t sV2[kAStage];
  __shared__ __attribute__((aligned(1024))) uint16_t sK3[kAStage];
  __shared__ __attribute__((aligned(1024))) uint16_t sV3[kAStage];
  __shared__ int sPos[kAq];

  // Heads of one KV group run on one XCD (they stream the same K/V); the
  // heaviest causal tiles (latest positions) start first. Tiles are cut from
  // the end of the group's active rows: tile y holds sorted rows
  // [cnt - 256 (y + 1), cnt - 256 y), so only the earliest tile, whose causal
  // key range is the shortest, can be partial. A partial latest tile costs
  // nearly a full one (its few rows see every key); measured on MI355X at the
  // Qwen3-14B prefill shape with half the groups on, the kernel's span went
  // from 441 to 419 us with this cut.
  const int x = blockIdx.x;
  const int h = a.Hq % 8 == 0 ? (x % 8) * (a.Hq / 8) + x / 8 : x;
  const int b = blockIdx.z;
  const int rep = a.Hq / a.Hk;
  const int g = h / rep;                  // KV head
  const int grp = h / (a.Hq / a.NG);      // routing group of the head
  const int cnt = a.counts[(size_t)b * a.NG + grp];
  const int s1 = cnt - (int)blockIdx.y * kAq;
  if (s1 <= 0) return;  // level 0
  const int s0 = max(0, s1 - kAq);
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int c = lane % 16, q = lane / 16;
  if (tid < kAq) sPos[tid] = s0 + tid < s1 ? a.perm[((size_t)b * a.NG + grp) * a.Tq + s0 + tid] : -1;
  __syncthreads();

  const int delta = a.Tk - a.Tq;
  const int jmin = a.leftpad ? a.leftpad[b] : 0;
  const int nvalid = s1 - s0;
  const int wg_maxpos = sPos[nvalid - 1];
  const int wlo = wave * kAqw, wvalid = max(0, min(kAqw, nvalid - wlo));
  const int w_maxpos = wvalid > 0 ? sPos[wlo + wvalid - 1] : -1;
  // first row of the wave (or -1 when the wave has an empty row: forces masks)
  const int w_minpos = wvalid == kAqw ? sPos[wlo] : -1;

  // Key tiles [t0, t1).
  const int t0 = jmin / kAk;
  const int kend = a.causal ? min(a.Tk, wg_maxpos + delta + 1) : a.Tk;
  const int t1 = (kend + kAk - 1) / kAk;
  const int nk = max(0, t1 - t0);

  // Q fragments (B operand of S^T = K Q^T): query 16 qb + c of the wave,
  // head dims 32 ds + 8 q .. +7.
  const size_t q_row = (size_t)a.Hq * kAd, kv_row = (size_t)a.Hk * kAd;
  const rsrc_t qr = make_rsrc(a.Q + (size_t)b * a.Tq * q_row, (uint64_t)a.Tq * q_row * 2);
  u32x4 qf[kAQB][4];
  int qpos[kAQB];
#pragma unroll
  for (int qb = 0; qb < kAQB; ++qb) {
    qpos[qb] = sPos[wlo + qb * 16 + c];
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      const uint32_t off = qpos[qb] >= 0 ? (uint32_t)(((size_t)qpos[qb] * q_row + (size_t)h * kAd + ds * 32 + 8 * q) * 2)
                                         : kOffNone;
      qf[qb][ds] = buf_ld16(qr, off);
    }
  }
  int jend[kAQB];
#pragma unroll
  for (int qb = 0; qb < kAQB; ++qb) jend[qb] = a.causal ? qpos[qb] + delta + 1 : a.Tk;

  // K/V stage loads: 16 instructions of 1 KB (4 rows) per operand per stage,
  // wave w issuing j = w + W i; lane l takes row 4j + l/16, position l % 16.
  const rsrc_t kr = make_rsrc(a.K + (size_t)b * a.Tk * kv_row, (uint64_t)a.Tk * kv_row * 2);
  const rsrc_t vr = make_rsrc(a.V + (size_t)b * a.Tk * kv_row, (uint64_t)a.Tk * kv_row * 2);
  auto issue = [&](int t, WIDE_LDS uint16_t *sk, WIDE_LDS uint16_t *sv) {
    const int k0 = (t0 + t) * kAk;
    const bool live = t < nk;
#pragma unroll
    for (int i = 0; i < 16 / kAWaves; ++i) {
      const int j = wave + kAWaves * i;
      const int r = 4 * j + lane / 16, p = lane % 16;
      const bool ok = live && k0 + r < a.Tk;
      const uint32_t base = (uint32_t)(((size_t)(k0 + r) * kv_row + (size_t)g * kAd) * 2);
      eng::load_lds(kr, (eng::lds_u16 *)(sk + j * 512), ok ? base + (uint32_t)((p ^ k_swz(r)) * 16) : kOffNone, 0u);
      eng::load_lds(vr, (eng::lds_u16 *)(sv + j * 512), ok ? base + (uint32_t)((p ^ v_swz(r)) * 16) : kOffNone, 0u);
    }
  };

  f32x4 o[8][kAQB];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int qb = 0; qb < kAQB; ++qb) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[kAQB], l[kAQB];
#pragma unroll
  for (int qb = 0; qb < kAQB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
  }
  const float sl2 = a.scale * kLog2e;

  auto compute = [&](int t, const WIDE_LDS uint16_t *sk, const WIDE_LDS uint16_t *sv) {
    const int k0 = (t0 + t) * kAk;
    if (k0 > w_maxpos + delta && a.causal) return;  // level 2: every row of the wave precedes the tile
    if (w_maxpos < 0) return;                        // the wave has no active row
    f32x4 sc[4][kAQB];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int qb = 0; qb < kAQB; ++qb) sc[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int r = kb * 16 + c;
        const u32x4 kf = *(const WIDE_LDS u32x4 *)(sk + r * kAd + (((ds * 4 + q) ^ k_swz(r)) * 8));
#pragma unroll
        for (int qb = 0; qb < kAQB; ++qb) sc[kb][qb] = mfma16x16x32(kf, qf[qb][ds], sc[kb][qb]);
      }
    // Element-wise masks only where some row of the wave may see a key
    // outside [jmin, jend): tiles that cross a causal diagonal, the left
    // padding or the end of the keys (a uniform branch; the masked path uses
    // selects only).
    const bool need_mask = k0 < jmin || k0 + kAk > a.Tk || (a.causal && k0 + kAk - 1 > w_minpos + delta);
    if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < kAQB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int key = k0 + kb * 16 + 4 * q + v;
            const bool ok = key >= jmin && key < jend[qb];
            sc[kb][qb][v] = ok ? sc[kb][qb][v] : -INFINITY;
          }
    }
    // Online softmax in the log2 domain. m is a row's reference: the running
    // max of scale*log2e*s, moved only when a tile's max exceeds it by more
    // than kLazy. Until then the tile's p = 2^(t - m) stay below 2^kLazy (no
    // overflow in fp32 sums or bf16 P) and the output needs no rescale; p, the
    // row sum l and the output share the reference, so the normalised result
    // is the same up to rounding. The rescale of the output, 64 multiplies per
    // lane, then runs only when some row of the wave moved its reference,
    // which after the first tiles is rare.
    float alpha[kAQB];
    u32x4 pf[2][kAQB];
#pragma unroll
    for (int qb = 0; qb < kAQB; ++qb) {
      // max of the lane's 16 scores: a chain of 8 three-way maxima
      float mx = max3(sc[0][qb][0], sc[0][qb][1], sc[0][qb][2]);
#pragma unroll
      for (int e = 3; e < 15; e += 2) mx = max3(mx, sc[e / 4][qb][e % 4], sc[(e + 1) / 4][qb][(e + 1) % 4]);
      mx = quad_max(max3(mx, sc[3][qb][3], sc[3][qb][3]));
      const float cand = mx * sl2;
      const bool up = cand > m[qb] + kLazy;  // m = -inf: any finite max moves it
      const float mref = up ? cand : m[qb];
      const float muse = mref == -INFINITY ? 0.f : mref;  // a row with no valid key yet: p = 0
      alpha[qb] = up ? exp2_fast(m[qb] - muse) : 1.f;
      m[qb] = mref;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float p = exp2_fast(fmaf(sc[kb][qb][v], sl2, -muse));
          sc[kb][qb][v] = p;
          ls += p;
        }
      l[qb] = l[qb] * alpha[qb] + ls;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        pf[ks][qb] = u32x4{pack_bf16x2(sc[2 * ks][qb][0], sc[2 * ks][qb][1]),
                           pack_bf16x2(sc[2 * ks][qb][2], sc[2 * ks][qb][3]),
                           pack_bf16x2(sc[2 * ks + 1][qb][0], sc[2 * ks + 1][qb][1]),
                           pack_bf16x2(sc[2 * ks + 1][qb][2], sc[2 * ks + 1][qb][3])};
    }
    // Rescale the output only when some row's max moved (a wave-wide vote).
    bool moved = false;
#pragma unroll
    for (int qb = 0; qb < kAQB; ++qb) moved |= alpha[qb] != 1.f;
    if (__ballot(moved)) {
#pragma unroll
      for (int qb = 0; qb < kAQB; ++qb)
#pragma unroll
        for (int db = 0; db < 8; ++db) o[db][qb] *= alpha[qb];
    }
    // O^T += V^T P^T. V^T fragment (16 head dims x 32 keys) from two
    // transposing reads: keys 32 ks + 4 q + j, then 32 ks + 16 + 4 q + j,
    // matching the key order of the P^T registers.
    const int sidx = lane % 16;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int chunk = 2 * db + (sidx % 4) / 2;
        const int r0 = ks * 32 + 4 * q + sidx / 4, r1 = r0 + 16;
        const u32x2 lo = lds_read_tr16(sv + r0 * kAd + ((chunk ^ v_swz(r0)) * 8) + 4 * (sidx % 2));
        const u32x2 hi = lds_read_tr16(sv + r1 * kAd + ((chunk ^ v_swz(r1)) * 8) + 4 * (sidx % 2));
        const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int qb = 0; qb < kAQB; ++qb) o[db][qb] = mfma16x16x32(vf, pf[ks][qb], o[db][qb]);
      }
  };

  WIDE_LDS uint16_t *k0s = (WIDE_LDS uint16_t *)sK0, *v0s = (WIDE_LDS uint16_t *)sV0;
  WIDE_LDS uint16_t *k1s = (WIDE_LDS uint16_t *)sK1, *v1s = (WIDE_LDS uint16_t *)sV1;
  WIDE_LDS uint16_t *k2s = (WIDE_LDS uint16_t *)sK2, *v2s = (WIDE_LDS uint16_t *)sV2;
  WIDE_LDS uint16_t *k3s = (WIDE_LDS uint16_t *)sK3, *v3s = (WIDE_LDS uint16_t *)sV3;
  // A ring of 4 stages with one barrier per pair of key tiles: at the barrier
  // of pair (t, t+1) both stages have landed for every wave and every wave is
  // done with the previous pair, whose two buffers then receive stages t+2 and
  // t+3. Half as many barriers as one per tile, with the same two tiles of
  // latency cover, and the waves drift apart within a pair (fewer coinciding
  // stalls on the two waves that share a SIMD).
  issue(0, k0s, v0s);
  issue(1, k1s, v1s);
  int t = 0;
#define WIDE_ATTN_PAIR(CK0, CV0, CK1, CV1, NK0, NV0, NK1, NV1) \
  {                                                            \
    WIDE_WAIT_VM_LGKM0(0);                                     \
    WIDE_BARRIER();                                            \
    issue(t + 2, NK0, NV0);                                    \
    issue(t + 3, NK1, NV1);                                    \
    compute(t, CK0, CV0);                                      \
    if (t + 1 < nk) compute(t + 1, CK1, CV1);                  \
    t += 2;                                                    \
  }
  while (t < nk) {
    WIDE_ATTN_PAIR(k0s, v0s, k1s, v1s, k2s, v2s, k3s, v3s)
    if (t >= nk) break;
    WIDE_ATTN_PAIR(k2s, v2s, k3s, v3s, k0s, v0s, k1s, v1s)
  }
#undef WIDE_ATTN_PAIR
  WIDE_WAIT_VM_LGKM0(0);

  // Normalise and scatter: lane holds head dims 16 db + 4 q .. +3 of query
  // 16 qb + c of the wave.
#pragma unroll
  for (int qb = 0; qb < kAQB; ++qb) {
    float z = l[qb];
    z = quad_sum(z);
    if (qpos[qb] < 0) continue;
    const float inv = z > 0.f ? 1.f / z : 0.f;
    const size_t obase = ((size_t)b * a.Tq + qpos[qb]) * q_row + (size_t)h * kAd + 4 * q;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const f32x4 v = o[db][qb] * inv;
      store4<OUT_F32>(a.O, obase + db * 16, v[0], v[1], v[2], v[3]);
    }
  }
}

// ---------------------------------------------------------------------------
// Decode: split-KV partials + merge.
// ---------------------------------------------------------------------------

constexpr int kDecKeys = 64;       // keys per split (one wave)
constexpr int kDecPart = kAd + 4;  // floats per partial: o[128], m, z (+pad)

// Routing group g of sequence b is on for its (single) decoding token.
__device__ __forceinline__ bool group_active(const AttnArgs &a, int b, int g) {
  if (a.mask) return a.mask[(size_t)b * a.NG + g] != 0;
  return a.counts[(size_t)b * a.NG + g] > 0;
}

// Some routing group of KV head g (its NG / Hk groups) is on.
__device__ __forceinline__ bool kv_head_active(const AttnArgs &a, int b, int g) {
  const int per = a.NG / a.Hk;
  bool on = false;
  for (int j = 0; j < per; ++j) on |= group_active(a, b, g * per + j);
  return on;
}

// One split = 64 keys of one active (b, g) on one wave, for all Hq/Hk heads of
// the group at once (they share the keys), on the matrix cores with the heads
// as the 16 columns (unused columns hold zero queries and are never written):
//   S^T = K Q^T: the K fragments (16 keys x 32 head dims) are loaded straight
//     into registers, lane l taking key 16 t + l % 16 and the 16-byte chunk
//     4 ds + l / 16 of its row, so every load covers 64 contiguous bytes of 16
//     keys; Q^T uses the same chunk order;
//   O^T = V^T P^T: V goes to LDS with direct loads (prefill stage layout) and
//     its transposed fragments come from transposing reads; P^T is the score
//     registers themselves, packed to bf16.
// A lane holds the scores of one head for 16 keys, so the split's max and sum
// take two cross-lane steps. All loads are issued before any is used.
__global__ __launch_bounds__(kWave) void attn_decode_split_kernel(AttnArgs a, int nsplit) {
  __shared__ __attribute__((aligned(1024))) uint16_t sV[kDecKeys * kAd];
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  if (!kv_head_active(a, b, g)) return;  // every head of the KV head is off: nothing is read
  const int rep = a.Hq / a.Hk;
  const int lane = threadIdx.x;
  const int q = lane / 16, c16 = lane % 16;
  const int jmin = a.leftpad ? a.leftpad[b] : 0;
  const int j0 = split * kDecKeys;
  const int jlo = max(j0, jmin);
  const int jhi = min(j0 + kDecKeys, a.Tk);  // Tq = 1: every key precedes the query
  float *ws = reinterpret_cast<float *>(a.workspace);
  const size_t q_row = (size_t)a.Hq * kAd, kv_row = (size_t)a.Hk * kAd;

  if (jlo >= jhi) {  // every key of the split is before the sequence's left padding
    for (int i = lane; i < rep * kDecPart; i += kWave) {
      const int r = i / kDecPart, c = i % kDecPart;
      float *part = ws + (((size_t)b * a.Hq + g * rep + r) * nsplit + split) * kDecPart;
      part[c] = c == kAd ? -INFINITY : 0.f;
    }
    return;
  }

  const rsrc_t kr = make_rsrc(a.K + (size_t)b * a.Tk * kv_row, (uint64_t)a.Tk * kv_row * 2);
  const rsrc_t vr = make_rsrc(a.V + (size_t)b * a.Tk * kv_row, (uint64_t)a.Tk * kv_row * 2);
  WIDE_LDS uint16_t *sv = (WIDE_LDS uint16_t *)sV;
  // V: 16 instructions of 1 KB, instruction j covering keys 4 j .. 4 j + 3.
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = 4 * j + lane / 16, p = lane % 16;
    const bool ok = j0 + r >= jlo && j0 + r < jhi;
    const uint32_t base = (uint32_t)(((size_t)(j0 + r) * kv_row + (size_t)g * kAd) * 2);
    eng::load_lds(vr, (eng::lds_u16 *)(sv + j * 512), ok ? base + (uint32_t)((p ^ v_swz(r)) * 16) : kOffNone, 0u);
  }
  // K fragments of the four 16-key tiles.
  u32x4 kf[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int j = j0 + 16 * t + c16;
    const bool ok = j >= jlo && j < jhi;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      const uint32_t off = (uint32_t)(((size_t)j * kv_row + (size_t)g * kAd + 8 * (4 * ds + q)) * 2);
      kf[t][ds] = buf_ld16(kr, ok ? off : kOffNone);
    }
  }
  // Q^T fragments: column c16 is head g * rep + c16.
  u32x4 qf[4];
  const uint16_t *Qh = a.Q + (size_t)b * q_row + ((size_t)g * rep + c16) * kAd;
#pragma unroll
  for (int ds = 0; ds < 4; ++ds)
    qf[ds] = c16 < rep ? ld16(Qh + 8 * (4 * ds + q)) : u32x4{0u, 0u, 0u, 0u};

  // Scores (log2 domain) of keys 16 t + 4 q + i for head c16.
  const float sl2 = a.scale * kLog2e;
  f32x4 sc[4];
  float m = -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) acc = mfma16x16x32(kf[t][ds], qf[ds], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + 16 * t + 4 * q + i;
      acc[i] = (j >= jlo && j < jhi) ? acc[i] * sl2 : -INFINITY;
      m = fmaxf(m, acc[i]);
    }
    sc[t] = acc;
  }
  m = quad_max(m);  // finite: the split has a valid key
  float z = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pv = exp2_fast(sc[t][i] - m);  // -inf -> 0
      sc[t][i] = pv;
      z += pv;
    }
  z = quad_sum(z);
  // P^T fragments: keys 32 ks + 4 q + i, then 32 ks + 16 + 4 q + i.
  u32x4 pf[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    pf[ks] = u32x4{pack_bf16x2(sc[2 * ks][0], sc[2 * ks][1]), pack_bf16x2(sc[2 * ks][2], sc[2 * ks][3]),
                   pack_bf16x2(sc[2 * ks + 1][0], sc[2 * ks + 1][1]),
                   pack_bf16x2(sc[2 * ks + 1][2], sc[2 * ks + 1][3])};

  WIDE_WAIT_VM_LGKM0(0);  // V has landed in LDS
  WIDE_BARRIER();
  // O^T: rows = head dims 16 db + 4 q + i, column = head c16.
  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int chunk = 2 * db + (c16 % 4) / 2;
      const int r0 = ks * 32 + 4 * q + c16 / 4, r1 = r0 + 16;
      const u32x2 lo = lds_read_tr16(sv + r0 * kAd + ((chunk ^ v_swz(r0)) * 8) + 4 * (c16 % 2));
      const u32x2 hi = lds_read_tr16(sv + r1 * kAd + ((chunk ^ v_swz(r1)) * 8) + 4 * (c16 % 2));
      const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
      o[db] = mfma16x16x32(vf, pf[ks], o[db]);
    }
  }
  if (c16 < rep) {
    float *part = ws + (((size_t)b * a.Hq + g * rep + c16) * nsplit + split) * kDecPart;
#pragma unroll
    for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4 *>(part + 16 * db + 4 * q) = o[db];
    if (q == 0) {
      part[kAd] = m;
      part[kAd + 1] = z;
    }
  }
}

// Merge of the splits of one (b, h) and 16 of its head dims (8 workgroups
// per head): the split maxima are staged in LDS, the weights 2^(m_s - max)
// and the total sum come from block reductions, and the weighted sum of the
// partial outputs is split over 16 groups of splits, then reduced in LDS.
constexpr int kMergeThreads = 256;
constexpr int kMergeDims = 16;

__device__ __forceinline__ float block_max(float v, float *red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return v;
}

__device__ __forceinline__ float block_sum(float v, float *red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  v = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return v;
}

template <bool OUT_F32>
__global__ __launch_bounds__(kMergeThreads) void attn_decode_merge_kernel(AttnArgs a, int nsplit) {
  __shared__ float sW[4096];  // split weights (at most 4096 splits)
  __shared__ float sRed[4];
  __shared__ float sPart[kMergeThreads / kMergeDims][kMergeDims + 1];
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int d0 = blockIdx.z * kMergeDims;
  if (!group_active(a, b, h / (a.Hq / a.NG))) return;
  const int tid = threadIdx.x;
  const float *ws = reinterpret_cast<const float *>(a.workspace) + ((size_t)b * a.Hq + h) * nsplit * kDecPart;
  float mloc = -INFINITY;
  for (int s = tid; s < nsplit; s += kMergeThreads) {
    const float m = ws[(size_t)s * kDecPart + kAd];
    sW[s] = m;
    mloc = fmaxf(mloc, m);
  }
  const float M = block_max(mloc, sRed);
  float zloc = 0.f;
  for (int s = tid; s < nsplit; s += kMergeThreads) {
    const float m = sW[s];
    const float w = (M == -INFINITY || m == -INFINITY) ? 0.f : exp2f(m - M);
    sW[s] = w;
    zloc = fmaf(w, ws[(size_t)s * kDecPart + kAd + 1], zloc);
  }
  const float Z = block_sum(zloc, sRed);  // also orders the sW writes before the reads below
  const int dl = tid % kMergeDims, sg = tid / kMergeDims;
  constexpr int NG = kMergeThreads / kMergeDims;
  float o = 0.f;
  int s = sg;
  for (; s + 7 * NG < nsplit; s += 8 * NG) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = ws[(size_t)(s + u * NG) * kDecPart + d0 + dl];
#pragma unroll
    for (int u = 0; u < 8; ++u) o = fmaf(sW[s + u * NG], v[u], o);
  }
  for (; s < nsplit; s += NG) o = fmaf(sW[s], ws[(size_t)s * kDecPart + d0 + dl], o);
  sPart[sg][dl] = o;
  __syncthreads();
  if (tid < kMergeDims) {
    float t = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) t += sPart[g][tid];
    const float out = Z > 0.f ? t / Z : 0.f;
    const size_t idx = (size_t)b * a.Hq * kAd + (size_t)h * kAd + d0 + tid;
    if (OUT_F32)
      reinterpret_cast<float *>(a.O)[idx] = out;
    else
      reinterpret_cast<uint16_t *>(a.O)[idx] = f2bf(out);
  }
}

// ---------------------------------------------------------------------------
// Built-in scratch for callers that cannot allocate (wide_attn_noalloc).
// ---------------------------------------------------------------------------

// One array per device, alive until the process ends. In host code its name
// only stands for the symbol: the device address comes from
// hipGetSymbolAddress, queried once per device with that device current.
static __device__ __align__(256) unsigned char scratch[kAttnScratchBytes];

void *attn_scratch(int *status) {
  static std::mutex mu;
  static void *ptr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    *status = WIDE_ERR_NO_DEVICE;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      *status = WIDE_ERR_LAUNCH;
      return nullptr;
    }
    ptr[dev] = p;
  }
  *status = WIDE_OK;
  return ptr[dev];
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
    hipLaunchKernelGGL(attn_decode_split_kernel, grid, dim3(kWave), 0, s, a, nsplit);
    const dim3 mgrid(a.Hq, a.B, kAd / kMergeDims);
    if (a.o_f32)
      hipLaunchKernelGGL(attn_decode_merge_kernel<true>, mgrid, dim3(kMergeThreads), 0, s, a, nsplit);
    else
      hipLaunchKernelGGL(attn_decode_merge_kernel<false>, mgrid, dim3(kMergeThreads), 0, s, a, nsplit);
    return check_launch();
  }
  dim3 grid(a.Hq, (a.Tq + kAq - 1) / kAq, a.B);
  if (a.o_f32)
    hipLaunchKernelGGL(attn_prefill_kernel<true>, grid, dim3(kAThreads), 0, s, a);
  else
    hipLaunchKernelGGL(attn_prefill_kernel<false>, grid, dim3(kAThreads), 0, s, a);
  return check_launch();
}

}  // namespace wide
