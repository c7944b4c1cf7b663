// Shared device helpers for the gfx950 kernels: bf16 packing, MFMA wrappers,
// wave-level primitives. Internal to libwide.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wide {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// D[16x16] += A[16x32] * B[32x16], bf16 inputs, fp32 accumulate.
// Lane l supplies row (l % 16) of A and column (l % 16) of B, each with 8
// reduction elements; the hardware pairs A's element i of lane l with B's
// element i of lane l, so any reduction-index assignment shared by A and B is
// valid. The result lands in lane l as column (l % 16), rows 4*(l/16) + v.
__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4 &a, const u32x4 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// fp32 -> bf16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint16_t f2bf(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16x2 (low half = a), round to nearest even; one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// 2^x on the transcendental unit (v_exp_f32): no range reduction; results
// below the normal range flush to zero, which softmax weights tolerate.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf2f(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, const u32x4 &v) { *reinterpret_cast<u32x4 *>(p) = v; }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Buffer resource over [base, base + bytes) (raw, stride 0). A load whose
// byte offset lies outside the range returns zeros and touches no memory, so
// predicated gathers can be issued unconditionally (no branch around the
// load, which keeps the compiler's load counters exact across prefetches).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOffNone = 0x80000000u;  // an offset past any valid range

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint64_t bytes) {
  const uint32_t n = bytes > 0x7fffffffull ? 0x7fffffffu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_ld16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Number of set bits of `m` below this lane (a wave-wide exclusive rank).
__device__ __forceinline__ int rank_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// Read-only value shared by the whole wave (keeps it in a scalar register).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

// acc + sum over 8 bf16 pairs of w * x: four v_dot2c_f32_bf16 (exact bf16
// products, fp32 sums). Each element is copied to a scalar before the bit
// cast: hipcc drops the index of a bit cast applied to a vector subscript.
__device__ __forceinline__ float dot8(const u32x4 &w, const u32x4 &x, float acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t we = w[e], xe = x[e];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, we), __builtin_bit_cast(bf16x2, xe), acc, false);
  }
  return acc;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes, the same value in every lane: four DPP steps give
// each 16-lane row its sum (swap neighbours, swap pairs, mirror within 8,
// mirror within 16), then the four row sums are read out. No LDS traffic.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  const int b = __builtin_bit_cast(int, v);
  return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
         (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}

}  // namespace wide
