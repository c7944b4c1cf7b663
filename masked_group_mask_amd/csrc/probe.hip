// Measurement probe: the bf16 MFMA rate this device sustains (the measured
// peak the GEMM and attention figures are compared with, beside the vendor
// figure). Every wave runs 8 independent accumulator chains of
// v_mfma_f32_16x16x32_bf16 (16 x 16 x 32 x 2 FLOPs each) from register
// operands, so nothing but the matrix cores is exercised; the accumulators
// are summed into one float per wave so no work can be dropped.
#include "common.hpp"
#include "launch.hpp"

namespace wide {

constexpr int kProbeChains = 8;

__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float *sink) {
  const int lane = threadIdx.x % kWave;
  u32x4 a = {0x3f803f80u + (uint32_t)lane, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  u32x4 b = {0x3c003c00u, 0x3c003c00u + (uint32_t)lane, 0x3c003c00u, 0x3c003c00u};
  f32x4 acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = mfma16x16x32(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  s = wave_sum(s);
  if (lane == 0) sink[blockIdx.x * 4 + threadIdx.x / kWave] = s;
}

int launch_mfma_probe(int blocks, int iters, float *sink, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, s, iters, sink);
  return check_launch();
}

}  // namespace wide
