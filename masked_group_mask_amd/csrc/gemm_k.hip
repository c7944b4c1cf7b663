// GEMM-K on gfx950: the K-axis routed projections (W_o, W_down).
//
// WIDE (arXiv 2607.28418), Appendix B, Eq. 21 and Algorithm 3:
//   C[m][n] = sum_g mask[m][g] * sum_{k in group g} A[m][k] * B[n][k].
// The page gives every (sorted row tile, K-group) pair its own pipeline and
// scatters each fp32 partial into C with atomics. Under token-level masks the
// rows a group keeps differ from group to group, so on MI355X that scatter
// (one fp32 read-add-write per active row and feature per group, through LDS
// or L2 atomics) costs more than the multiply-adds it saves while the group
// is short (G = 128 needs 2G = 256 MFMA flops per scattered value; the LDS
// moves a value in and out more slowly than that). Here C stays in registers:
//   - a workgroup owns C[m0:m0+256, n0:n0+BN] in original row order and
//     runs the shared MFMA main loop over the whole K range; BN = 320 or 192
//     where those tiles fill whole rounds of the compute units, else 256 (or
//     128 when N is not a multiple of 256);
//   - the A slice of a row whose group is off for that token is never read
//     (level 1): its load offset is set out of range, the buffer load moves
//     no data and the stage holds zeros there, so the product adds exactly 0;
//   - a tile none of whose rows keeps any group writes beta*C and exits
//     (level 0);
//   - the per-row predicates come from a bit table built once per tile from
//     the mask bytes: bit r of word i of group g = row 32i + r keeps group g;
//   - the summation order is fixed, so results are reproducible bit for bit.
// For M <= 4 a matrix-vector kernel streams only the K-groups some token
// keeps.
#include <atomic>

#include "common.hpp"
#include "launch.hpp"
#include "mma_engine.hpp"

namespace wide {

constexpr int kKMaxGroups = 512;
constexpr int kKRasterM = 32;  // m-tiles per raster group (eng::tile_of)
// the 320-wide tiles' raster group: 16 m-tiles, so that an XCD's concurrent
// tiles share two column blocks of B and each row block of A is read by two
// of them (measured on MI355X, Qwen3-14B down_proj at 50%: 1.08 against 1.09
// ms at 32, and 1.11 against 1.20 ms on all-ones masks)
constexpr int kKRasterM320 = 16;
// likewise 8 for the other widths when the column tiles split evenly over the
// XCDs (each XCD then owns its own column blocks; measured on MI355X at the
// Llama3.1-8B prefill shapes, N = 4096: down_proj 1.50 against 1.61 ms
// masked and 1.67 against 1.86 on all-ones masks; the 32 above was measured
// at N = 5120, whose 20 column tiles do not split over the XCDs)
constexpr int kKRasterMXcd = 8;

// The raster of the token-order tiles of width BN over NT column tiles. The
// K-split fixup and the half-width tail tiles use it with BN = 256, so every
// kernel of a launch finds a tile at the same place.
__device__ __forceinline__ void k_tile_of(int BN, int L, int MT, int NT, int &mt, int &tn) {
  if (BN == 320)
    eng::tile_of<kKRasterM320>(L, MT, NT, mt, tn);
  else if (NT % 8 == 0)
    eng::tile_of<kKRasterMXcd>(L, MT, NT, mt, tn);
  else
    eng::tile_of<kKRasterM>(L, MT, NT, mt, tn);
}

// Tile order of the kernel over pattern-sorted rows. Sorted row tiles differ
// in cost (the number of groups their rows keep), and the plain raster gives
// each XCD the same few m-tiles for every n-tile, so the XCDs ended far apart
// (measured: compute units busy 70% of the span). Here logical tile j is
// (m-tile j % MT, n-tile j / MT), and the whole tiles are dealt so that each
// XCD owns a contiguous range of j (xcd_remap): it walks one or two n-tiles
// over every m-tile, the same mix of costs on every XCD, with its weight
// columns shared in its L2. Tiles of the K-split tail keep j = L.
__device__ __forceinline__ void ord_tile_of(int L, int whole, int MT, int &mt, int &tn) {
  const int j = L < whole ? xcd_remap(L, whole) : L;
  mt = j % MT;
  tn = j / MT;
}

// Builds the tile's bit table: bit r of word i of group g says whether tile
// row 32 i + r keeps group g. Thread t reads the mask row of tile row t % 256
// (for the groups g = t / 256 mod THREADS / 256) and each wave turns one
// group column of its 64 rows into two words by ballot. Returns whether any
// row of the tile keeps any group. `flag` is one word of a stage buffer (the
// 4-wave tile has no LDS left for a word of its own); the barrier after every
// wave has read it keeps the first stage loads, issued right after, from
// overwriting it early.
// `m` is the token row of this thread's tile row (tid % 256), or -1 for a
// tile row past the end.
template <int THREADS>
__device__ __forceinline__ bool build_bits(const KArgs &a, int m, WIDE_LDS uint32_t *bits, WIDE_LDS int *flag) {
  constexpr int PARTS = THREADS / 256;
  const int NG = a.K / a.G;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int part = tid / 256, wrow = wave % 4;
  const bool valid = m >= 0;
  const uint8_t *row = a.mask + (size_t)(valid ? m : 0) * NG;
  if (tid == 0) *flag = 0;
  __syncthreads();
  int any = 0;
  auto put = [&](int g, bool on) {
    const uint64_t bal = __ballot(on);
    any |= bal != 0;
    if (lane == 0) {
      bits[g * 8 + wrow * 2] = (uint32_t)bal;
      bits[g * 8 + wrow * 2 + 1] = (uint32_t)(bal >> 32);
    }
  };
  if (NG % 4 == 0 && reinterpret_cast<uintptr_t>(a.mask) % 4 == 0) {
    // 4 groups per 32-bit load; part p takes the words w with w % PARTS == p
    const uint32_t *row4 = reinterpret_cast<const uint32_t *>(row);
    const int nw = NG / 4;
    for (int w0 = part; w0 < nw; w0 += 8 * PARTS) {
      uint32_t w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int wi = w0 + u * PARTS;
        w[u] = (valid && wi < nw) ? row4[wi] : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int wi = w0 + u * PARTS;
        if (wi < nw)
#pragma unroll
          for (int e = 0; e < 4; ++e) put(4 * wi + e, ((w[u] >> (8 * e)) & 0xffu) != 0);
      }
    }
  } else {
    for (int g0 = part; g0 < NG; g0 += 8 * PARTS) {
      uint8_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int g = g0 + u * PARTS;
        v[u] = (valid && g < NG) ? row[g] : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (g0 + u * PARTS < NG) put(g0 + u * PARTS, v[u] != 0);
    }
  }
  if (any && lane == 0) *flag = 1;
  __syncthreads();
  const bool r = *flag != 0;
  __syncthreads();
  return r;
}

// Stage loader of the tile: A rows predicated by the bit table, B rows
// dense. The bit words of a stage's group are read from LDS a step before the
// stage is issued, among the fragment reads, and unpacked only when it is, so
// the LDS latency never sits in front of the loads.
// SMALLG: groups narrower than a 64-deep stage (G = 16 or 32): a stage then
// spans 64 / G groups and each lane's 16-byte chunk of a row (8 reduction
// elements) lies in one of them, so the predicate is taken per lane from the
// bit of (row, group of its chunk), read from the table when the stage is
// issued.
// Every load instruction of a wave moves rows 8 W apart from the previous
// one's at the same swizzle, so one per-lane byte offset (that of instruction
// 0) serves them all and instruction i adds i times the row stride to the
// wave-uniform offset. A rows past M or skipping the group take the out-of-
// range offset instead, so only rows below M are ever addressed.
template <class S, bool SMALLG>
struct KLoader {
  static constexpr int kDsReads = SMALLG ? 0 : 2;
  static constexpr int kLoadGap = 0;
  // the bit words kept across the step leave room for fewer fragments (no
  // spills at BN = 320 with 4 A-fragment groups; measured faster than 2)
  static constexpr int kWideAGroups = 4;
  static constexpr int AHEAD = S::STAGES - 1;  // stages in flight ahead of the one multiplied
  rsrc_t ar, br, none;
  uint32_t aoff, boff;        // lane's byte offset in load instruction 0 (A, B)
  uint32_t astride, bstride;  // bytes from one load instruction's rows to the next's
  const WIDE_LDS uint32_t *bits;
  int nk, kb, steps_per_group, NG, G, wave, lane;  // steps kb .. kb + nk - 1 of K
  u32x4 wlo, whi;  // bit words (rows 0..127, 128..255) of the group of the next stage

  __device__ __forceinline__ void fetch(int t) {
    if (SMALLG) return;
    const int g = min((t + kb) / steps_per_group, NG - 1);
    wlo = *(const WIDE_LDS u32x4 *)(bits + g * 8);
    whi = *(const WIDE_LDS u32x4 *)(bits + g * 8 + 4);
  }

  __device__ __forceinline__ void operator()(int t, eng::lds_u16 *sa, eng::lds_u16 *sb) {
    uint32_t p = 0;
    if (SMALLG) {
#pragma unroll
      for (int i = 0; i < S::AI; ++i) {
        const int r = eng::load_row<S::WAVES>(wave, i, lane);
        const int c = (lane % 8) ^ eng::swz(r);  // chunk of the row this lane loads
        const int g = min(((t + kb) * eng::kBK + 8 * c) / G, NG - 1);
        p |= ((bits[g * 8 + (r >> 5)] >> (r & 31)) & 1u) << i;
      }
    } else {
      // Load instruction i covers tile row 8 (wave + W i) + lane / 8: word
      // (W / 4) i + wave / 4 of the table, bit (8 wave + lane / 8) % 32.
      const int sh = (wave * 8 + lane / 8) % 32;
      const bool hiw = S::WAVES == 8 && wave >= 4;
#pragma unroll
      for (int i = 0; i < S::AI; ++i) {
        const int w = (S::WAVES / 4) * i;  // word index for waves 0..3
        const uint32_t x = w < 4 ? (hiw ? wlo[(w + 1) % 4] : wlo[w % 4]) : (hiw ? whi[(w + 1) % 4] : whi[w % 4]);
        p |= ((x >> sh) & 1u) << i;
      }
    }
    const bool live = t < nk;
    const rsrc_t ra = live ? ar : none, rb = live ? br : none;
    const uint32_t k0 = (uint32_t)(t + kb) * eng::kBK * 2u;
#pragma unroll
    for (int i = 0; i < S::AI; ++i)
      eng::load_lds(ra, eng::load_dst<S::WAVES>(sa, wave, i), ((p >> i) & 1u) ? aoff : kOffNone, k0 + i * astride);
#pragma unroll
    for (int i = 0; i < S::BI; ++i)
      eng::load_lds(rb, eng::load_dst<S::WAVES>(sb, wave, i), boff, k0 + i * bstride);
    if (t < AHEAD) fetch(t + 1);  // prologue: these stages are issued before any is multiplied
  }
  // while stage t is multiplied, stage t + AHEAD has just been issued
  __device__ __forceinline__ void prefetch(int t) { fetch(t + AHEAD + 1); }
};

template <int BN, int W, bool SMALLG>
__global__ __launch_bounds__(64 * W) void gemm_k_kernel(KArgs a) {
  using S = eng::Shape<BN, W>;
  // third-stage buffers only for 3 stages (unused placeholders, which the
  // compiler drops, else: the 320-wide tile's two stages and its 16 KB bit
  // table fill the 160 KB of LDS exactly)
  constexpr int A3 = S::STAGES == 3 ? S::A_ELEMS : 8, B3 = S::STAGES == 3 ? S::B_ELEMS : 8;
  constexpr int AL3 = S::STAGES == 3 ? 1024 : 16;
  __shared__ __attribute__((aligned(1024))) uint16_t sA0[S::A_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sB0[S::B_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sA1[S::A_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sB1[S::B_ELEMS];
  __shared__ __attribute__((aligned(AL3))) uint16_t sA2[A3];
  __shared__ __attribute__((aligned(AL3))) uint16_t sB2[B3];
  __shared__ __attribute__((aligned(16))) uint32_t sBits[kKMaxGroups][8];

  const int MT = (a.M + eng::kBM - 1) / eng::kBM;
  int mt, tn, n0;
  int part = 0, nparts = 1, slot = 0;  // K slice of this workgroup; slot: split tile index
  if (a.split_tail) {  // half of a 256 x 256 tile of the raster
    k_tile_of(256, a.tile_base + (int)blockIdx.x / 2, MT, a.N / 256, mt, tn);
    n0 = tn * 256 + ((int)blockIdx.x % 2) * BN;
  } else {
    int L = (int)blockIdx.x;
    if (a.ksplit > 1 && L >= a.head) {
      slot = (L - a.head) / a.ksplit;
      part = (L - a.head) % a.ksplit;
      nparts = a.ksplit;
      L = a.head + slot;
    }
    k_tile_of(BN, a.tile_base + L, MT, a.N / BN, mt, tn);
    n0 = tn * BN;
  }
  const int m0 = mt * eng::kBM;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int wm = wave / S::WNW, wn = wave % S::WNW;

  const int mrow = m0 + (int)threadIdx.x % eng::kBM;
  const bool any = build_bits<S::THREADS>(a, mrow < a.M ? mrow : -1, (WIDE_LDS uint32_t *)&sBits[0][0],
                                          (WIDE_LDS int *)sA1);
  eng::Acc<S> acc;
#pragma unroll
  for (int i = 0; i < S::FN; ++i)
#pragma unroll
    for (int j = 0; j < S::FM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (any) {  // level 0: otherwise the tile's product is exactly zero
    KLoader<S, SMALLG> ld;
    const int rows = min(eng::kBM, a.M - m0);
    ld.ar = make_rsrc(a.A + (size_t)m0 * a.lda, (uint64_t)rows * a.lda * 2);  // rows past M: out of range
    ld.br = make_rsrc(a.B + (size_t)n0 * a.ldb, (uint64_t)BN * a.ldb * 2);
    ld.none = make_rsrc(a.A, 0);
    const int r0 = eng::load_row<W>(wave, 0, lane);
    ld.aoff = (uint32_t)r0 * (uint32_t)a.lda * 2u + eng::load_chunk_bytes(r0, lane);
    ld.boff = (uint32_t)r0 * (uint32_t)a.ldb * 2u + eng::load_chunk_bytes(r0, lane);
    ld.astride = 8u * W * (uint32_t)a.lda * 2u;
    ld.bstride = 8u * W * (uint32_t)a.ldb * 2u;
    ld.bits = (const WIDE_LDS uint32_t *)&sBits[0][0];
    const int nk_all = a.K / eng::kBK;
    ld.kb = part * nk_all / nparts;
    ld.nk = (part + 1) * nk_all / nparts - ld.kb;
    ld.steps_per_group = max(1, a.G / eng::kBK);
    ld.NG = a.K / a.G;
    ld.G = a.G;
    ld.wave = wave;
    ld.lane = lane;
    ld.fetch(0);
    eng::mainloop<S, BN, false>(ld.nk, ld, (eng::lds_u16 *)sA0, (eng::lds_u16 *)sB0, (eng::lds_u16 *)sA1,
                                (eng::lds_u16 *)sB1, (eng::lds_u16 *)sA2, (eng::lds_u16 *)sB2, acc, wm, wn, lane);
  }

  // A lane holds row (lane % 16) of A fragment j and features
  // 4 (lane / 16) .. +3 of B fragment i.
  if (part < nparts - 1) {
    // K slices other than the last: the partial tile goes to the workspace
    // (256 x BN fp32, row-major, one per slice), for the fixup kernel.
    float *wt = a.ws + ((size_t)slot * (nparts - 1) + part) * (size_t)(eng::kBM * BN);
#pragma unroll
    for (int j = 0; j < S::FM; ++j) {
      float *wrow = wt + (size_t)(wm * S::TM + j * 16 + lane % 16) * BN + wn * S::TN + 4 * (lane / 16);
#pragma unroll
      for (int i = 0; i < S::FN; ++i) *reinterpret_cast<f32x4 *>(wrow + i * 16) = acc[i][j];
    }
    return;
  }
  // C = beta * C + acc (for a K-split tile, the last slice's part; the
  // fixup kernel adds the others).
#pragma unroll
  for (int j = 0; j < S::FM; ++j) {
    const int m = m0 + wm * S::TM + j * 16 + lane % 16;
    if (m >= a.M) continue;
    float *crow = a.C + (size_t)m * a.ldc + n0 + wn * S::TN + 4 * (lane / 16);
#pragma unroll
    for (int i = 0; i < S::FN; ++i) {
      f32x4 v = acc[i][j];
      if (a.beta) v += *reinterpret_cast<const f32x4 *>(crow + i * 16);
      *reinterpret_cast<f32x4 *>(crow + i * 16) = v;
    }
  }
}

// ---- Ordered GEMM-K: rows sorted by routing pattern, inactive work skipped --
//
// With `order` (a permutation of the token rows that puts rows with the same
// routing pattern next to each other, e.g. wide_order_by_pattern), a
// workgroup owns the tile of sorted positions m0 .. m0+256 and features
// n0 .. n0+256. Its A rows are gathered through the order and its C rows
// scattered back through it; the accumulators stay in registers in tile
// order, so no partial result is ever moved between rows. Then:
//   - the k-loop runs only over the K-groups some row of the tile keeps
//     (the tile's live groups, listed once from the bit table);
//   - a load instruction whose 8 rows all skip the step's group is not issued;
//   - a wave's 16-row A fragment none of whose rows keeps the step's group
//     skips its multiply-adds (a wave-uniform branch around its 4 MFMAs).
// An output row's sum runs over the same products in the same order as in
// the unordered kernel: the work skipped adds exact zeros there.
//
// One step: the A and B fragments of the stage are read, then for every A
// fragment jj its MFMAs (when live), followed in the first half by one of
// the next stage's 8 load instructions, so the loads stay spread over the
// step whatever is skipped. The bit words of the group two steps ahead are
// read from LDS during a step, so no load waits on them.
struct OrdStep {
  uint32_t fl;   // bit jj: this wave's A fragment jj has a row that keeps the step's group
  uint32_t lb;   // byte i: the rows of this wave's A load instruction i that keep it
  uint32_t li;   // bit i: A load instruction i is issued (its 16-row fragment is live)
  uint32_t k0;   // byte offset of the step's 64-deep slice of K
};

// What a step needs from LDS: the 8 bit words of its group (the bit table
// compacted to live-group order) and the group itself. Read right after a
// barrier, decoded a step later, so no wait is ever spent on them.
struct OrdRaw {
  u32x4 lo, hi;
  int g;
  int kk;
  bool on;
};

__device__ __forceinline__ OrdRaw ord_fetch(const WIDE_LDS uint32_t *bits, const WIDE_LDS uint16_t *live, int gi,
                                            int kk, bool on) {
  OrdRaw r;
  r.on = on;
  r.kk = kk;
  if (on) {
    r.lo = *(const WIDE_LDS u32x4 *)(bits + gi * 8);
    r.hi = *(const WIDE_LDS u32x4 *)(bits + gi * 8 + 4);
    r.g = live[gi];
  } else {
    r.lo = r.hi = u32x4{0u, 0u, 0u, 0u};
    r.g = 0;
  }
  return r;
}

// Decoding for wave (wm, wave): A fragment jj covers tile rows 128 wm + 16 jj
// .. +15 (half jj % 2 of bit word 4 wm + jj / 2); A load instruction i covers
// tile rows 8 (wave + 8 i) .. +7 (byte wave % 4 of bit word 2 i + wave / 4),
// one half of the 16-row fragment in half (wave % 4) / 2 of that word. A load
// is left out only when that whole fragment is dead: a live fragment is
// multiplied in full, so its inactive rows must hold the zeros an
// out-of-range load writes, not an older stage.
__device__ __forceinline__ OrdStep ord_decode(const OrdRaw &raw, int G, int wm, int wave) {
  OrdStep r{0u, 0u, 0u, 0u};
  if (!raw.on) return r;
  const uint32_t w[8] = {raw.lo[0], raw.lo[1], raw.lo[2], raw.lo[3], raw.hi[0], raw.hi[1], raw.hi[2], raw.hi[3]};
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const uint32_t word = wm == 0 ? w[jj / 2] : w[4 + jj / 2];
    r.fl |= (((word >> (16 * (jj % 2))) & 0xffffu) != 0u ? 1u : 0u) << jj;
  }
  const int bsh = 8 * (wave % 4), fsh = 16 * ((wave % 4) / 2);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t word = wave < 4 ? w[2 * i] : w[2 * i + 1];
    r.lb |= ((word >> bsh) & 0xffu) << (8 * i);
    r.li |= (((word >> fsh) & 0xffffu) != 0u ? 1u : 0u) << i;
  }
  r.fl = (uint32_t)__builtin_amdgcn_readfirstlane(r.fl);
  r.lb = (uint32_t)__builtin_amdgcn_readfirstlane(r.lb);
  r.li = (uint32_t)__builtin_amdgcn_readfirstlane(r.li);
  const int g = __builtin_amdgcn_readfirstlane(raw.g);  // wave-uniform: buffer offsets need SGPRs
  r.k0 = (uint32_t)(g * G + raw.kk * eng::kBK) * 2u;
  return r;
}

__global__ __launch_bounds__(512) void gemm_k_ordered_kernel(KArgs a) {
  using S = eng::Shape<256, 8>;
  constexpr int BN = 256;
  __shared__ __attribute__((aligned(1024))) uint16_t sA0[S::A_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sB0[S::B_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sA1[S::A_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sB1[S::B_ELEMS];
  __shared__ __attribute__((aligned(16))) uint32_t sBits[kKMaxGroups][8];
  __shared__ int sRows[eng::kBM];
  __shared__ uint16_t sLive[kKMaxGroups];
  __shared__ int sScan[S::WAVES + 1];

  const int MT = (a.M + eng::kBM - 1) / eng::kBM;
  int mt, tn;
  int part = 0, nparts = 1, slot = 0;
  {
    int L = (int)blockIdx.x;
    if (a.ksplit > 1 && L >= a.head) {
      slot = (L - a.head) / a.ksplit;
      part = (L - a.head) % a.ksplit;
      nparts = a.ksplit;
      L = a.head + slot;
    }
    ord_tile_of(L, a.ksplit > 1 ? a.head : (int)gridDim.x, MT, mt, tn);
  }
  const int m0 = mt * eng::kBM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / S::WNW, wn = wave % S::WNW;
  const int NG = a.K / a.G;
  if (tid < eng::kBM) {
    // an entry outside [0, M) (not a permutation) is dropped, never dereferenced
    const int m = m0 + tid < a.M ? a.order[m0 + tid] : -1;
    sRows[tid] = (unsigned)m < (unsigned)a.M ? m : -1;
  }
  __syncthreads();
  WIDE_LDS uint32_t *bits = (WIDE_LDS uint32_t *)&sBits[0][0];
  const bool any = build_bits<S::THREADS>(a, sRows[tid % eng::kBM], bits, (WIDE_LDS int *)sA1);

  eng::Acc<S> acc;
#pragma unroll
  for (int i = 0; i < S::FN; ++i)
#pragma unroll
    for (int j = 0; j < S::FM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (any) {
    // List the live groups in ascending order (one thread per group).
    int nlive = 0;
    for (int g0 = 0; g0 < NG; g0 += S::THREADS) {
      const int g = g0 + tid;
      bool on = false;
      if (g < NG) {
        const u32x4 lo = *(const WIDE_LDS u32x4 *)(bits + g * 8), hi = *(const WIDE_LDS u32x4 *)(bits + g * 8 + 4);
        on = ((lo[0] | lo[1] | lo[2] | lo[3]) | (hi[0] | hi[1] | hi[2] | hi[3])) != 0u;
      }
      const uint64_t bal = __ballot(on);
      if (lane == 0) sScan[wave] = __popcll(bal);
      __syncthreads();
      int before = nlive, tot = 0;
#pragma unroll
      for (int w = 0; w < S::WAVES; ++w) {
        const int c = sScan[w];
        before += w < wave ? c : 0;
        tot += c;
      }
      if (on) sLive[before + rank_below(bal)] = (uint16_t)g;
      nlive += tot;
      __syncthreads();
    }
    // Compact the bit table to live-group order (row gi = group sLive[gi]):
    // all reads, a barrier, then the writes (a slot may be another's source).
    {
      u32x4 lo = u32x4{0u, 0u, 0u, 0u}, hi = lo;
      const bool mine = tid < nlive;
      if (mine) {
        const int g = sLive[tid];
        lo = *(const WIDE_LDS u32x4 *)(bits + g * 8);
        hi = *(const WIDE_LDS u32x4 *)(bits + g * 8 + 4);
      }
      __syncthreads();
      if (mine) {
        *(WIDE_LDS u32x4 *)(bits + tid * 8) = lo;
        *(WIDE_LDS u32x4 *)(bits + tid * 8 + 4) = hi;
      }
      __syncthreads();
    }
    const int spg = a.G / eng::kBK;
    const int nk_all = nlive * spg;
    const int kb = part * nk_all / nparts;
    const int nk = (part + 1) * nk_all / nparts - kb;

    const rsrc_t ar = make_rsrc(a.A, (uint64_t)a.M * a.lda * 2);
    const rsrc_t br = make_rsrc(a.B + (size_t)n0 * a.ldb, (uint64_t)BN * a.ldb * 2);
    uint32_t aoff[S::AI], boff[S::BI];
#pragma unroll
    for (int i = 0; i < S::AI; ++i) {
      const int r = eng::load_row<8>(wave, i, lane);
      const int phys = sRows[r];
      aoff[i] = phys >= 0 ? (uint32_t)phys * (uint32_t)a.lda * 2u + eng::load_chunk_bytes(r, lane) : kOffNone;
    }
#pragma unroll
    for (int i = 0; i < S::BI; ++i) {
      const int r = eng::load_row<8>(wave, i, lane);
      boff[i] = (uint32_t)r * (uint32_t)a.ldb * 2u + eng::load_chunk_bytes(r, lane);
    }
    const WIDE_LDS uint16_t *live = (const WIDE_LDS uint16_t *)sLive;
    const int wv = __builtin_amdgcn_readfirstlane(wave), wmu = __builtin_amdgcn_readfirstlane(wm);
    // One load slot: slots 2i are A instruction i (not issued when its whole
    // 16-row fragment skips the group), slots 2i + 1 B instruction i.
    auto load_slot = [&](int q, const OrdStep &st, eng::lds_u16 *sa, eng::lds_u16 *sb, bool on) {
      const int i = q / 2;
      if (q % 2 == 0) {
        const uint32_t byte = (st.lb >> (8 * i)) & 0xffu;
        if (on && ((st.li >> i) & 1u))
          eng::load_lds(ar, eng::load_dst<8>(sa, wave, i), ((byte >> (lane / 8)) & 1u) ? aoff[i] : kOffNone, st.k0);
      } else if (on) {
        eng::load_lds(br, eng::load_dst<8>(sb, wave, i), boff[i], st.k0);
      }
    };
    auto compute = [&](const eng::lds_u16 *sa, const eng::lds_u16 *sb, uint32_t fl, const OrdStep &nx,
                       eng::lds_u16 *na, eng::lds_u16 *nb, bool nx_on) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4 fb[S::FN], fa[S::FM];
#pragma unroll
        for (int i = 0; i < S::FN; ++i) {
          const int row = wn * S::TN + i * 16 + lane % 16;
          fb[i] = *(const WIDE_LDS u32x4 *)(sb + row * eng::kBK + (((s * 4 + lane / 16) ^ eng::swz(row)) * 8));
        }
#pragma unroll
        for (int jj = 0; jj < S::FM; ++jj) {
          const int row = wm * S::TM + jj * 16 + lane % 16;
          fa[jj] = *(const WIDE_LDS u32x4 *)(sa + row * eng::kBK + (((s * 4 + lane / 16) ^ eng::swz(row)) * 8));
        }
        // keep the fragment reads here, ahead of the branches
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int jj = 0; jj < S::FM; ++jj) {
          if (fl & (1u << jj)) {
#pragma unroll
            for (int i = 0; i < S::FN; ++i) acc[i][jj] = mfma16x16x32(fb[i], fa[jj], acc[i][jj]);
          }
          if (s == 0) {
            __builtin_amdgcn_sched_barrier(0);
            load_slot(jj, nx, na, nb, nx_on);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    };

    eng::lds_u16 *a0 = (eng::lds_u16 *)sA0, *b0 = (eng::lds_u16 *)sB0;
    eng::lds_u16 *a1 = (eng::lds_u16 *)sA1, *b1 = (eng::lds_u16 *)sB1;
    // step counters of the step after next: group index and step within it
    int gi2 = (kb + 2) / spg, kk2 = (kb + 2) % spg;
    OrdStep cur = ord_decode(ord_fetch(bits, live, kb / spg, kb % spg, nk > 0), a.G, wmu, wv);
    OrdStep nxt = ord_decode(ord_fetch(bits, live, (kb + 1) / spg, (kb + 1) % spg, nk > 1), a.G, wmu, wv);
#pragma unroll
    for (int q = 0; q < S::NLOAD; ++q) load_slot(q, cur, a0, b0, nk > 0);
    for (int t = 0; t < nk; ++t) {
      WIDE_WAIT_VM_LGKM0(0);
      WIDE_BARRIER();
      // the step after next: read now, decoded at the end of this step
      const OrdRaw raw = ord_fetch(bits, live, gi2, kk2, t + 2 < nk);
      if (++kk2 == spg) {
        kk2 = 0;
        ++gi2;
      }
      const bool odd = t & 1;
      compute(odd ? a1 : a0, odd ? b1 : b0, cur.fl, nxt, odd ? a0 : a1, odd ? b0 : b1, t + 1 < nk);
      cur = nxt;
      // Pin the raw words here: without this the compiler moves them to
      // scalar registers right after the reads, waiting on them there.
      OrdRaw late = raw;
      asm volatile("" : "+v"(late.lo), "+v"(late.hi), "+v"(late.g));
      nxt = ord_decode(late, a.G, wmu, wv);
    }
    WIDE_WAIT_VM_LGKM0(0);
  }

  if (part < nparts - 1) {
    float *wt = a.ws + ((size_t)slot * (nparts - 1) + part) * (size_t)(eng::kBM * BN);
#pragma unroll
    for (int j = 0; j < S::FM; ++j) {
      float *wrow = wt + (size_t)(wm * S::TM + j * 16 + lane % 16) * BN + wn * S::TN + 4 * (lane / 16);
#pragma unroll
      for (int i = 0; i < S::FN; ++i) *reinterpret_cast<f32x4 *>(wrow + i * 16) = acc[i][j];
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < S::FM; ++j) {
    const int m = sRows[wm * S::TM + j * 16 + lane % 16];
    if (m < 0) continue;
    float *crow = a.C + (size_t)m * a.ldc + n0 + wn * S::TN + 4 * (lane / 16);
#pragma unroll
    for (int i = 0; i < S::FN; ++i) {
      f32x4 v = acc[i][j];
      if (a.beta) v += *reinterpret_cast<const f32x4 *>(crow + i * 16);
      *reinterpret_cast<f32x4 *>(crow + i * 16) = v;
    }
  }
}

// Matrix-vector GEMM-K for M = MT <= 4 tokens. The four waves first list the
// K-groups some token keeps (one ballot per 64 groups); then each wave owns
// one output feature and streams only the listed groups' segments of its
// weight row, 16 bytes per lane with consecutive lanes on consecutive chunks,
// a block of 8 chunks per lane issued before any is used. Every wave walks
// the same chunk list, so a block's x chunks of every token go to LDS once
// per workgroup (direct loads, zeros where the token does not keep the
// group) and the products read them there.
template <int MT>
__global__ __launch_bounds__(256) void gemv_k_kernel(KArgs a) {
  constexpr int U = 8;
  __shared__ __attribute__((aligned(16))) uint16_t sx[MT][U * kWave * 8];  // a block of x per token
  __shared__ uint16_t sGrp[kKMaxGroups];
  __shared__ uint8_t sOn[kKMaxGroups];
  __shared__ int sCnt[4];
  const int NG = a.K / a.G;
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  int base = 0;
  for (int g0 = 0; g0 < NG; g0 += 4 * kWave) {
    const int g = g0 + wave * kWave + lane;
    int on = 0;
    if (g < NG)
      for (int m = 0; m < MT; ++m) on |= (a.mask[(size_t)m * NG + g] != 0) << m;
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
  float s[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) s[m] = 0.f;
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
    }
    if (c0 > 0) __syncthreads();  // every wave is done with the previous block of x
    // x -> LDS: instruction (m, u), u = wave, wave + 4, moves list chunks c0 + 64 u + lane
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const rsrc_t xr = make_rsrc(a.A + (size_t)m * a.lda, (uint64_t)a.K * 2);
#pragma unroll
      for (int i = 0; i < U / 4; ++i) {
        const int u = wave + 4 * i;
        int kku = kk[0], onu = on[0];
#pragma unroll
        for (int v = 1; v < U; ++v)
          if (v == u) kku = kk[v], onu = on[v];
        eng::load_lds(xr, (eng::lds_u16 *)&sx[m][u * kWave * 8], (onu >> m) & 1 ? (uint32_t)kku * 2u : kOffNone, 0u);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = buf_ld16(wr, on[u] ? (uint32_t)kk[u] * 2u : kOffNone);
    __builtin_amdgcn_sched_barrier(0);
    WIDE_WAIT_VM_LGKM0(U);  // this wave's x loads have landed; its weights may still be in flight
    __syncthreads();        // and every other wave's
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const u32x4 x = *(const WIDE_LDS u32x4 *)((const WIDE_LDS uint16_t *)&sx[m][0] + (u * kWave + lane) * 8);
        s[m] = dot8(w[u], x, s[m]);
      }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const float v = wave_sum(s[m]);
    if (lane == 0) {
      float *dst = a.C + (size_t)m * a.ldc + n;
      *dst = a.beta ? *dst + v : v;
    }
  }
}

int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load();
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n);
  }
  return n;
}

// Second pass of the K-split tiles: adds the workspace partials of the
// other slices to C, in slice order, so C = (beta C + last slice) + slice 0 +
// slice 1 + ... for every run. One thread per 4 consecutive features of a
// tile row (64 workgroups per tile).
__global__ __launch_bounds__(256) void gemm_k_fixup_kernel(KArgs a) {
  constexpr int Q = 256 / 4;                  // 4-feature quads per tile row
  constexpr int PER_TILE = eng::kBM * Q / 256;  // workgroups per tile
  constexpr size_t TILE = (size_t)eng::kBM * 256;
  const int slot = blockIdx.x / PER_TILE;
  const int e = (blockIdx.x % PER_TILE) * 256 + threadIdx.x;
  const int r = e / Q, q = e % Q;
  const int MT = (a.M + eng::kBM - 1) / eng::kBM;
  int mt, tn;
  if (a.order)
    ord_tile_of(a.head + slot, a.head, MT, mt, tn);
  else
    k_tile_of(256, a.head + slot, MT, a.N / 256, mt, tn);
  const int pos = mt * eng::kBM + r;
  if (pos >= a.M) return;
  const int m = a.order ? a.order[pos] : pos;
  if ((unsigned)m >= (unsigned)a.M) return;
  float *c = a.C + (size_t)m * a.ldc + tn * 256 + 4 * q;
  f32x4 v = *reinterpret_cast<const f32x4 *>(c);
  const float *w = a.ws + (size_t)slot * (a.ksplit - 1) * TILE + (size_t)r * 256 + 4 * q;
  for (int p = 0; p < a.ksplit - 1; ++p) v += *reinterpret_cast<const f32x4 *>(w + p * TILE);
  *reinterpret_cast<f32x4 *>(c) = v;
}

namespace {

// Tiles of the 8-wave 256 x 256 kernel and how its last, partly filled round
// is spread: with T tiles on C compute units, the T mod C tiles of that round
// (all T when T < C) are each split into S slices of K when they fill at most
// half of it, S = min(C / leftover, 8, K-steps / 8) (at least 2).
struct KSplitPlan {
  int tiles, head, ksplit;
};

KSplitPlan ksplit_plan(int M, int N, int K) {
  KSplitPlan p{0, 0, 1};
  if (M <= 4 || N % 256 != 0) return p;
  const int cus = cu_count();
  p.tiles = ((M + eng::kBM - 1) / eng::kBM) * (N / 256);
  p.head = p.tiles;
  const int tail = p.tiles % cus;
  if (tail == 0 || 2 * tail > cus) return p;
  const int s = min(min(cus / tail, 8), (K / eng::kBK) / 8);
  if (s < 2) return p;
  p.head = p.tiles - tail;
  p.ksplit = s;
  return p;
}

size_t plan_bytes(const KSplitPlan &p) {
  return p.ksplit > 1 ? (size_t)(p.tiles - p.head) * (size_t)(p.ksplit - 1) * eng::kBM * 256 * sizeof(float) : 0;
}

}  // namespace

size_t gemm_k_workspace_bytes(int M, int N, int K) { return plan_bytes(ksplit_plan(M, N, K)); }

template <int BN, int W>
static void launch_k_tiles(const KArgs &a, dim3 grid, hipStream_t s) {
  if (a.G % eng::kBK == 0)
    hipLaunchKernelGGL((gemm_k_kernel<BN, W, false>), grid, dim3(64 * W), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_k_kernel<BN, W, true>), grid, dim3(64 * W), 0, s, a);
}

// Tiled launches. When 256 x 320 tiles fill whole rounds of the compute
// units (N = 5120 at M = 8192: 512 tiles, where 256 x 256 tiles make 640)
// and G is a multiple of 64, the 8-wave 320-wide kernel runs alone
// (measured on MI355X at 50% activity: o_proj, K = 5120, 0.39 ms against
// 0.41, down_proj, K = 17408, 1.07 against 1.16). Likewise 256 x 192 tiles
// when they fill whole rounds and 256 x 256 ones do not (N = 3072 at
// M = 4096: 256 tiles where 256 x 256 ones leave 64 of 256 CUs idle).
// Otherwise, with N a multiple of 256, the 8-wave 256 x 256 kernel runs.
// When its tiles leave a last round at most half full (640 tiles on 256 CUs
// run as 3 rounds, 2.5 of work) and the caller gave the workspace, each
// leftover tile is split along K over S workgroups of the same launch, which
// run after the full rounds (one round of 1/S the length), and a fixup
// kernel adds the slices. Without a workspace the leftover tiles are covered
// by twice as many 256 x 128 workgroups of the 4-wave kernel in a second
// launch (measured on MI355X: barely faster than a third full round). Each
// output element's summation order is fixed by the shape, so results are
// reproducible bit for bit.
int launch_gemm_k(const KArgs &a0, hipStream_t s) {
  KArgs a = a0;
  a.tile_base = 0;
  a.split_tail = 0;
  a.head = 0;
  a.ksplit = 1;
  const int mt = (a.M + eng::kBM - 1) / eng::kBM;
  if (a.M <= 4) {
    const dim3 grid(a.N / 4), block(256);
    switch (a.M) {
      case 1: hipLaunchKernelGGL(gemv_k_kernel<1>, grid, block, 0, s, a); break;
      case 2: hipLaunchKernelGGL(gemv_k_kernel<2>, grid, block, 0, s, a); break;
      case 3: hipLaunchKernelGGL(gemv_k_kernel<3>, grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL(gemv_k_kernel<4>, grid, block, 0, s, a); break;
    }
  } else if (a.N % 256 == 0 && a.order != nullptr && a.G % eng::kBK == 0) {
    // rows through the order; the leftover round split along K with a workspace
    const KSplitPlan p = ksplit_plan(a.M, a.N, a.K);
    if (p.ksplit > 1 && a.ws != nullptr && a.ws_bytes >= plan_bytes(p)) {
      const int tail = p.tiles - p.head;
      a.head = p.head;
      a.ksplit = p.ksplit;
      hipLaunchKernelGGL(gemm_k_ordered_kernel, dim3(p.head + tail * p.ksplit), dim3(512), 0, s, a);
      hipLaunchKernelGGL(gemm_k_fixup_kernel, dim3(tail * (eng::kBM * 64 / 256)), dim3(256), 0, s, a);
    } else {
      hipLaunchKernelGGL(gemm_k_ordered_kernel, dim3(mt * (a.N / 256)), dim3(512), 0, s, a);
    }
  } else if (a.N % 320 == 0 && a.G % eng::kBK == 0 && (mt * (a.N / 320)) % cu_count() == 0) {
    a.order = nullptr;
    hipLaunchKernelGGL((gemm_k_kernel<320, 8, false>), dim3(mt * (a.N / 320)), dim3(512), 0, s, a);
  } else if (a.N % 192 == 0 && a.G % eng::kBK == 0 && (mt * (a.N / 192)) % cu_count() == 0 &&
             (a.N % 256 != 0 || (mt * (a.N / 256)) % cu_count() != 0)) {
    a.order = nullptr;
    hipLaunchKernelGGL((gemm_k_kernel<192, 8, false>), dim3(mt * (a.N / 192)), dim3(512), 0, s, a);
  } else if (a.N % 256 == 0) {
    a.order = nullptr;
    const KSplitPlan p = ksplit_plan(a.M, a.N, a.K);
    if (p.ksplit > 1 && a.ws != nullptr && a.ws_bytes >= plan_bytes(p)) {
      const int tail = p.tiles - p.head;
      a.head = p.head;
      a.ksplit = p.ksplit;
      launch_k_tiles<256, 8>(a, dim3(p.head + tail * p.ksplit), s);
      hipLaunchKernelGGL(gemm_k_fixup_kernel, dim3(tail * (eng::kBM * 64 / 256)), dim3(256), 0, s, a);
    } else {
      const int tiles = mt * (a.N / 256), cus = cu_count();
      const int tail = tiles % cus;
      const int head = tiles > cus && tail > 0 && 2 * tail <= cus ? tiles - tail : tiles;
      launch_k_tiles<256, 8>(a, dim3(head), s);
      if (head < tiles) {
        a.tile_base = head;
        a.split_tail = 1;
        launch_k_tiles<128, 4>(a, dim3(2 * (tiles - head)), s);
      }
    }
  } else {
    a.order = nullptr;
    launch_k_tiles<128, 4>(a, dim3(mt * (a.N / 128)), s);
  }
  return check_launch();
}

}  // namespace wide
