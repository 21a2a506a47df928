// Measurement kernel: the MFMA ceiling of the chip, and the clock it holds
// while the matrix pipes are saturated. Not part of the forward path; the
// benchmark runs it beside the GEMMs so their fraction of the published peak
// can be read against what the same instruction reaches with no memory
// traffic at all.
//
// Every wave keeps 8 independent accumulator chains of the path's one bf16
// instruction (v_mfma_f32_16x16x32_bf16) on register operands, so each
// MFMA's issue never waits on the previous one's result. 8 waves per
// workgroup (two per SIMD). Lane 0 of wave 0 reads the shader-clock counter
// and the constant 100 MHz real-time counter before and after the loop; the
// ratio of the two differences is the shader clock during the loop.
#include "common.h"
#include "launch.h"

namespace inv {
namespace {

constexpr int kProbeWaves = 8;
constexpr int kChains = 8;

__global__ __launch_bounds__(64 * kProbeWaves) void mfma_loop_kernel(int64_t iters, uint64_t* __restrict__ clk,
                                                                     float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  // operands that the compiler cannot fold: derived from the lane id at run time
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(float)((lane + e) & 7);
    b[e] = (__bf16)(float)((lane * 3 + e) & 3);
  }
  asm volatile("" : "+v"(a), "+v"(b));
  f32x4 acc[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  const uint64_t c0 = clock64();
  const uint64_t r0 = wall_clock64();
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kChains; ++i) acc[i] = mfma16(a, b, acc[i]);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kChains; ++i) s = s + acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  __syncthreads();
  const uint64_t c1 = clock64();
  const uint64_t r1 = wall_clock64();
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clk[2 * (int64_t)blockIdx.x + 0] = c1 - c0;
    clk[2 * (int64_t)blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

hipError_t launch_mfma_loop(int64_t iters, int groups, uint64_t* clk, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)groups), dim3(64 * kProbeWaves), 0, s, iters, clk, sink);
  return hipGetLastError();
}

}  // namespace inv
