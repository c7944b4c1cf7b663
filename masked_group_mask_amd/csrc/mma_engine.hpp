// Shared MFMA main loop of the tiled GEMM kernels (gfx950). Internal to
// libwide.so.
//
// A workgroup computes a 256 x BN tile of D = A * B^T (A rows are tokens, B
// rows are output features) with W waves: W = 4 (one per SIMD, 2 x 2 waves,
// BN = 64 or 128) or W = 8 (two per SIMD, 2 x 4 waves, BN = 256 or 320). Every wave
// owns a 128 x BN/(W/2) block and multiplies it with 16x16x32 bf16 MFMAs into
// fp32 accumulators held in registers.
//
// Every k-step moves a 64-deep slice of both operands (128-byte row segments)
// from global memory straight into LDS with buffer loads that write LDS
// directly: through a ring of 3 stages for W = 4 (LDS 48 KB per stage), of 2
// stages for W = 8 (64 KB per stage), one barrier per step.
//
// Measured on MI355X, the limits of this loop are the MFMA rate, the LDS read
// rate and the address unit that takes the stage loads: a CU accepts about
// one 1 KB load instruction per 15 cycles and a wave that issues a load the
// unit cannot take yet stalls, MFMAs included. The stage loads are therefore
// spread between MFMAs (scheduling groups impose the order), and the 8-wave
// tile halves both the load instructions and the LDS reads per flop.
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

constexpr int kBM = 256;    // A rows per tile (320 for the 320 x 256 tile)
constexpr int kBK = 64;     // reduction depth per stage

template <int BN, int W, int BM = kBM>
struct Shape {
  static_assert((W == 4 && BM == 256 && (BN == 64 || BN == 128)) ||
                    (W == 8 && ((BM == 256 && (BN == 192 || BN == 256 || BN == 320)) || (BM == 320 && BN == 256))),
                "unsupported tile");
  static constexpr int WAVES = W;
  static constexpr int THREADS = 64 * W;
  static constexpr int ROWS = BM;           // A rows of the tile
  static constexpr int WNW = W / 2;         // waves along n (2 along m)
  static constexpr int STAGES = W == 4 ? 3 : 2;
  static constexpr int TM = BM / 2;         // wave block rows
  static constexpr int TN = BN / WNW;       // wave block columns
  static constexpr int FM = TM / 16;        // 16-row fragments of A per wave
  static constexpr int FN = TN / 16;        // 16-row fragments of B per wave
  static constexpr int AI = BM / 8 / W;     // A load instructions per wave per stage
  static constexpr int BI = BN / 8 / W;     // B load instructions per wave per stage
  static constexpr int NLOAD = AI + BI;
  static constexpr int A_ELEMS = BM * kBK;
  static constexpr int B_ELEMS = BN * kBK;
};

// A stage row is 8 chunks of 16 bytes; chunk c of row r is stored at position
// c ^ swz(r), so the 16 lanes that read one chunk of 16 consecutive rows hit
// 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// Load instruction i of a wave moves 1 KB: rows 8j .. 8j+7 (j = wave + W i),
// lane l taking row 8j + l/8 and storing LDS position l % 8.
template <int W>
__device__ __forceinline__ int load_row(int wave, int i, int lane) { return (wave + W * i) * 8 + lane / 8; }
__device__ __forceinline__ uint32_t load_chunk_bytes(int row, int lane) {
  return (uint32_t)(((lane % 8) ^ swz(row)) * 16);
}
template <int W>
__device__ __forceinline__ lds_u16 *load_dst(lds_u16 *stage, int wave, int i) { return stage + (wave + W * i) * 512; }

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

template <class S>
struct Frag {
  u32x4 a[S::FM], b[S::FN];
};

template <class S>
using Acc = f32x4[S::FN][S::FM];

// B fragment i of wave column wn: rows wn*TN + 16i, or, for a split tile
// (SwiGLU: stage rows [0, BN/2) gate, [BN/2, BN) up), gate rows for the first
// half of the fragments and the matching up rows for the second half.
template <class S, int BN, bool SPLIT>
__device__ __forceinline__ int b_frag_row(int wn, int i) {
  if (!SPLIT) return wn * S::TN + i * 16;
  return i < S::FN / 2 ? wn * (S::TN / 2) + i * 16 : BN / 2 + wn * (S::TN / 2) + (i - S::FN / 2) * 16;
}

// One stage: two 32-deep halves, each reading its fragments then issuing the
// MFMAs. With more than 4 B fragments per wave (BN = 320) the A fragments are
// read and used in AG groups (Issue::kWideAGroups: 2 or 4), so fewer fragment
// registers are live at once; a loader that keeps more registers of its own
// across the step takes 4. With 10 A fragments (320 rows) they go in two
// groups of 5. `issue.prefetch(t)` runs after the first half's first reads
// (the loader's own LDS reads, consumed at the next step).
template <class S, class Issue>
constexpr int a_groups() { return S::FM > 8 ? 2 : S::FN > 4 ? Issue::kWideAGroups : 1; }

template <class S, int BN, bool SPLIT, class Issue>
__device__ __forceinline__ void compute_stage(const lds_u16 *sa, const lds_u16 *sb, Acc<S> &acc, int wm, int wn,
                                              int lane, Issue &issue, int t) {
  constexpr int AG = a_groups<S, Issue>(), FMG = S::FM / AG;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    u32x4 fb[S::FN];
#pragma unroll
    for (int i = 0; i < S::FN; ++i) {
      const int row = b_frag_row<S, BN, SPLIT>(wn, i) + lane % 16;
      fb[i] = *(const WIDE_LDS u32x4 *)(sb + row * kBK + (((s * 4 + lane / 16) ^ swz(row)) * 8));
    }
#pragma unroll
    for (int jg = 0; jg < AG; ++jg) {
      u32x4 fa[FMG];
#pragma unroll
      for (int jj = 0; jj < FMG; ++jj) {
        const int row = wm * S::TM + (jg * FMG + jj) * 16 + lane % 16;
        fa[jj] = *(const WIDE_LDS u32x4 *)(sa + row * kBK + (((s * 4 + lane / 16) ^ swz(row)) * 8));
      }
      if (s == 0 && jg == 0) issue.prefetch(t);
      // D^T blocks: lane holds tile row (A) lane % 16 of fragment j and
      // columns (B) 4 * (lane / 16) + v of fragment i.
#pragma unroll
      for (int i = 0; i < S::FN; ++i)
#pragma unroll
        for (int jj = 0; jj < FMG; ++jj) acc[i][jg * FMG + jj] = mfma16x16x32(fb[i], fa[jj], acc[i][jg * FMG + jj]);
    }
  }
}

// Scheduling groups of one A-fragment group: NR LDS reads, then NV x (Q
// MFMAs, 1 stage load), then the remaining MFMAs. Q is NM / NV (loads spread
// evenly), capped at QMAX when QMAX > 0 (loads packed towards the start).
template <int NR, int NM, int NV, int QMAX = 0>
__device__ __forceinline__ void interleave_half() {
  __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);  // DS reads
  if constexpr (NV > 0) {
    constexpr int Q = (QMAX > 0 && QMAX < NM / NV) ? QMAX : NM / NV;
    static_assert(Q >= 1, "more stage loads than MFMAs in a half");
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, Q, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // VMEM
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM - Q * NV, 0);
  } else {
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
  }
}

// Order of one step. 3 stages: the stage loads are spread over both halves.
// 2 stages: the next stage is needed at the next step, so its loads all go in
// the first half, at most QMAX MFMAs apart when QMAX > 0. The loader's own LDS
// reads come first in program order. With A-fragment groups, the loads are
// spread over the first half's groups (the first group takes the remainder).
template <class S, int AG, int EXTRA_DS, int QMAX>
__device__ __forceinline__ void interleave() {
  constexpr int NRB = S::FN, NRA = S::FM / AG, NMG = S::FN * S::FM / AG;
  if constexpr (AG == 1) {
    constexpr int NR = NRA + NRB, NM = NMG;
    if constexpr (S::STAGES == 3) {
      static_assert(S::NLOAD % 2 == 0, "stage loads must split over the two halves");
      interleave_half<NR + EXTRA_DS, NM, S::NLOAD / 2>();
      interleave_half<NR, NM, S::NLOAD / 2>();
    } else {
      interleave_half<NR + EXTRA_DS, NM, S::NLOAD, QMAX>();
      interleave_half<NR, NM, 0>();
    }
  } else if constexpr (AG == 2) {
    static_assert(S::STAGES == 2, "A-fragment groups only with the 2-stage tile");
    // first half: B + A group 0 (and the loader's reads), A group 1; loads
    // spread over the first half; second half without loads
    constexpr int NV0 = S::NLOAD / 2, NV1 = S::NLOAD - NV0;
    interleave_half<NRB + NRA + EXTRA_DS, NMG, NV0, QMAX>();
    interleave_half<NRA, NMG, NV1, QMAX>();
    interleave_half<NRB + NRA, NMG, 0>();
    interleave_half<NRA, NMG, 0>();
  } else {
    static_assert(AG == 4 && S::STAGES == 2, "A-fragment groups only with the 2-stage tile");
    constexpr int NV = S::NLOAD / 4, NV0 = S::NLOAD - 3 * NV;
    interleave_half<NRB + NRA + EXTRA_DS, NMG, NV0, QMAX>();
    interleave_half<NRA, NMG, NV, QMAX>();
    interleave_half<NRA, NMG, NV, QMAX>();
    interleave_half<NRA, NMG, NV, QMAX>();
    interleave_half<NRB + NRA, NMG, 0>();
    interleave_half<NRA, NMG, 0>();
    interleave_half<NRA, NMG, 0>();
    interleave_half<NRA, NMG, 0>();
  }
}

// The k-loop. `issue(t, sa, sb)` must issue exactly S::NLOAD buffer loads per
// wave for stage t into (sa, sb), out of range when t >= nk, and no other
// vector-memory loads; `issue.prefetch(t)` (called while stage t is
// multiplied) may issue Issue::kDsReads LDS reads whose results the next issue
// uses; Issue::kWideAGroups sets the A-fragment groups of a 320-wide tile;
// Issue::kLoadGap caps the MFMAs between two stage loads of the 2-stage
// tile (0: spread evenly). The stage buffers are distinct LDS objects so the
// compiler can tell them apart when it places its own waits.
//
// 3 stages: stage t sits in buffer t % 3; after the barrier of step t every
// wave is done with buffer (t + 2) % 3, which then receives stage t + 2.
// 2 stages: after the barrier of step t every wave is done with the other
// buffer, which then receives stage t + 1.
template <class S, int BN, bool SPLIT, class Issue>
__device__ __forceinline__ void mainloop(int nk, Issue &issue, lds_u16 *a0, lds_u16 *b0, lds_u16 *a1, lds_u16 *b1,
                                         lds_u16 *a2, lds_u16 *b2, Acc<S> &acc, int wm, int wn, int lane) {
  constexpr int NL = S::NLOAD;
  int t = 0;
#define WIDE_STEP(WAITN, CA, CB, NA, NB, AHEAD)                              \
  {                                                                          \
    WIDE_WAIT_VM_LGKM0(WAITN);                                               \
    WIDE_BARRIER();                                                          \
    issue(t + AHEAD, NA, NB);                                                \
    compute_stage<S, BN, SPLIT>(CA, CB, acc, wm, wn, lane, issue, t);        \
    interleave<S, a_groups<S, Issue>(), Issue::kDsReads, Issue::kLoadGap>(); \
    __builtin_amdgcn_sched_barrier(0);                                       \
    ++t;                                                                     \
  }
  if constexpr (S::STAGES == 3) {
    issue(0, a0, b0);
    issue(1, a1, b1);
    for (; t + 3 <= nk;) {
      WIDE_STEP(NL, a0, b0, a2, b2, 2)
      WIDE_STEP(NL, a1, b1, a0, b0, 2)
      WIDE_STEP(NL, a2, b2, a1, b1, 2)
    }
    if (t < nk) WIDE_STEP(NL, a0, b0, a2, b2, 2)
    if (t < nk) WIDE_STEP(NL, a1, b1, a0, b0, 2)
  } else {
    (void)a2;
    (void)b2;
    issue(0, a0, b0);
    for (; t + 2 <= nk;) {
      WIDE_STEP(0, a0, b0, a1, b1, 1)
      WIDE_STEP(0, a1, b1, a0, b0, 1)
    }
    if (t < nk) WIDE_STEP(0, a0, b0, a1, b1, 1)
  }
#undef WIDE_STEP
  WIDE_WAIT_VM_LGKM0(0);
}

// Workgroup id -> (m-tile, n-tile). The dispatcher deals workgroups to the 8
// XCDs round-robin; when the n-tiles split evenly, XCD x owns n-tiles
// [x NT/8, (x+1) NT/8) for every m-tile (so tiles that exit early are spread
// over all XCDs), visited in groups of GM m-tiles, column by column, so
// concurrently running tiles share A rows and B rows in that XCD's L2.
// Measured on MI355X (Qwen3-14B prefill shapes): GM = 8 suits the GEMM-MN
// raster (gate/up on all-ones masks 2.27 ms against 2.36 at GM = 4 and 2.47
// at GM = 32); the GEMM-K kernel picks GM per tile width and column split
// (its own raster helper states the measured choices).
template <int GM>
__device__ __forceinline__ void tile_of(int L, int MT, int NT, int &mt, int &tn) {
  int x = 0, i = L, NX = NT;
  if (NT % 8 == 0) {
    x = L % 8;
    i = L / 8;
    NX = NT / 8;
  }
  const int per_group = GM * NX;
  const int grp = i / per_group, in = i % per_group;
  const int first = grp * GM;
  const int gm = min(GM, MT - first);
  mt = first + in % gm;
  tn = x * NX + in / gm;
}

}  // namespace eng
}  // namespace wide
