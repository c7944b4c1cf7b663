// Shared MFMA main loop of the tiled GEMM kernels (gfx950). Internal to
// libwide.so.
//
// A workgroup of 4 waves computes a 256 x BN tile of D = A * B^T (A rows are
// tokens, B rows are output features). Every k-step moves a 64-deep slice of
// both operands (128-byte row segments) from global memory straight into LDS
// with buffer loads that write LDS directly, through a ring of 3 stages, so
// two slices are in flight while the third is multiplied and one barrier per
// step suffices. Each wave owns a 128 x BN/2 block of the tile and multiplies
// it with 16x16x32 bf16 MFMAs, fp32 accumulators held in registers.
//
// Loads past a buffer resource's range return zeros and move no data, which
// is how rows that are not active (or past the end) are skipped: the caller
// sets their per-lane offset out of range.
#pragma once

#include "common.hpp"

namespace wide {
namespace eng {

#define WIDE_LDS __attribute__((address_space(3)))
typedef WIDE_LDS uint16_t lds_u16;

constexpr int kBM = 256;      // A rows per tile
constexpr int kBK = 64;       // reduction depth per stage
constexpr int kThreads = 256;  // 4 waves, one per SIMD
constexpr int kGroupM = 4;    // m-tiles per raster group

template <int BN>
struct Shape {
  static constexpr int TM = 128;       // wave block rows (2 x 2 waves)
  static constexpr int TN = BN / 2;    // wave block columns
  static constexpr int FM = TM / 16;   // 16-row fragments of A per wave
  static constexpr int FN = TN / 16;   // 16-row fragments of B per wave
  static constexpr int AI = kBM / 32;  // A load instructions per wave per stage
  static constexpr int BI = BN / 32;   // B load instructions per wave per stage
  static constexpr int NLOAD = AI + BI;
  static constexpr int A_ELEMS = kBM * kBK;
  static constexpr int B_ELEMS = BN * kBK;
};

// A stage row is 8 chunks of 16 bytes; chunk c of row r is stored at position
// c ^ swz(r), so the 16 lanes that read one chunk of 16 consecutive rows hit
// 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// Load instruction i of a wave moves 1 KB: rows 8j .. 8j+7 (j = wave + 4i),
// lane l taking row 8j + l/8 and storing LDS position l % 8.
__device__ __forceinline__ int load_row(int wave, int i, int lane) { return (wave + 4 * i) * 8 + lane / 8; }
__device__ __forceinline__ uint32_t load_chunk_bytes(int row, int lane) {
  return (uint32_t)(((lane % 8) ^ swz(row)) * 16);
}

__device__ __forceinline__ void load_lds(rsrc_t r, lds_u16 *dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (WIDE_LDS void *)dst, 16, (int)voff, (int)soff, 0, 0);
}

// s_waitcnt vmcnt(n) lgkmcnt(0), expcnt not waited (gfx9 field layout).
#define WIDE_WAIT_VM_LGKM0(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | (0x7 << 4))
#define WIDE_BARRIER()                  \
  do {                                  \
    __builtin_amdgcn_sched_barrier(0);  \
    __builtin_amdgcn_s_barrier();       \
    __builtin_amdgcn_sched_barrier(0);  \
  } while (0)

template <int BN>
struct Frag {
  u32x4 a[Shape<BN>::FM], b[Shape<BN>::FN];
};

// B fragment i of wave column wn: rows wn*TN + 16i, or, for a split tile
// (SwiGLU: stage rows [0, BN/2) gate, [BN/2, BN) up), gate rows for the first
// half of the fragments and the matching up rows for the second half.
template <int BN, bool SPLIT>
__device__ __forceinline__ int b_frag_row(int wn, int i) {
  using S = Shape<BN>;
  if (!SPLIT) return wn * S::TN + i * 16;
  return i < S::FN / 2 ? wn * (S::TN / 2) + i * 16 : BN / 2 + wn * (S::TN / 2) + (i - S::FN / 2) * 16;
}

template <int BN, bool SPLIT>
__device__ __forceinline__ void compute_stage(const lds_u16 *sa, const lds_u16 *sb, f32x4 (&acc)[Shape<BN>::FN][Shape<BN>::FM],
                                              int wm, int wn, int lane) {
  using S = Shape<BN>;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    Frag<BN> f;
#pragma unroll
    for (int i = 0; i < S::FM; ++i) {
      const int row = wm * S::TM + i * 16 + lane % 16;
      f.a[i] = *(const WIDE_LDS u32x4 *)(sa + row * kBK + (((s * 4 + lane / 16) ^ swz(row)) * 8));
    }
#pragma unroll
    for (int i = 0; i < S::FN; ++i) {
      const int row = b_frag_row<BN, SPLIT>(wn, i) + lane % 16;
      f.b[i] = *(const WIDE_LDS u32x4 *)(sb + row * kBK + (((s * 4 + lane / 16) ^ swz(row)) * 8));
    }
    // D^T blocks: lane holds tile row (A) lane % 16 of fragment j and
    // columns (B) 4 * (lane / 16) + v of fragment i.
#pragma unroll
    for (int i = 0; i < S::FN; ++i)
#pragma unroll
      for (int j = 0; j < S::FM; ++j) acc[i][j] = mfma16x16x32(f.b[i], f.a[j], acc[i][j]);
  }
}

// The k-loop. `issue(t, sa, sb)` must issue exactly Shape<BN>::NLOAD buffer
// loads per wave for stage t into (sa, sb), out of range when t >= nk, and no
// other vector-memory loads. The three stage buffers are distinct LDS objects
// so the compiler can tell the stages apart when it places its own waits.
template <int BN, bool SPLIT, class Issue>
__device__ __forceinline__ void mainloop(int nk, Issue &issue, lds_u16 *a0, lds_u16 *b0, lds_u16 *a1, lds_u16 *b1,
                                         lds_u16 *a2, lds_u16 *b2, f32x4 (&acc)[Shape<BN>::FN][Shape<BN>::FM], int wm,
                                         int wn, int lane) {
  constexpr int NL = Shape<BN>::NLOAD;
  issue(0, a0, b0);
  issue(1, a1, b1);
  int t = 0;
  // Stage t sits in buffer t % 3; after the barrier every wave is done with
  // buffer (t + 2) % 3, which then receives stage t + 2.
#define WIDE_STEP(CA, CB, NA, NB)                                         \
  {                                                                       \
    WIDE_WAIT_VM_LGKM0(NL);                                               \
    WIDE_BARRIER();                                                       \
    issue(t + 2, NA, NB);                                                 \
    compute_stage<BN, SPLIT>(CA, CB, acc, wm, wn, lane);                  \
    ++t;                                                                  \
  }
  for (; t + 3 <= nk;) {
    WIDE_STEP(a0, b0, a2, b2)
    WIDE_STEP(a1, b1, a0, b0)
    WIDE_STEP(a2, b2, a1, b1)
  }
  if (t < nk) WIDE_STEP(a0, b0, a2, b2)
  if (t < nk) WIDE_STEP(a1, b1, a0, b0)
#undef WIDE_STEP
  WIDE_WAIT_VM_LGKM0(0);
}

// Workgroup id -> (m-tile, n-tile). The dispatcher deals workgroups to the 8
// XCDs round-robin; when the n-tiles split evenly, XCD x owns n-tiles
// [x NT/8, (x+1) NT/8) for every m-tile (so tiles that exit early are spread
// over all XCDs), visited in groups of kGroupM m-tiles, column by column, so
// concurrently running tiles share A rows and B rows in that XCD's L2.
__device__ __forceinline__ void tile_of(int L, int MT, int NT, int &mt, int &tn) {
  int x = 0, i = L, NX = NT;
  if (NT % 8 == 0) {
    x = L % 8;
    i = L / 8;
    NX = NT / 8;
  }
  const int per_group = kGroupM * NX;
  const int grp = i / per_group, in = i % per_group;
  const int first = grp * kGroupM;
  const int gm = min(kGroupM, MT - first);
  mt = first + in % gm;
  tn = x * NX + in / gm;
}

}  // namespace eng
}  // namespace wide
