// Measurement support: the MFMA throughput this chip reaches on the instruction the attention
// kernel uses (v_mfma_f32_32x32x16_bf16), and the shader clock while it runs. The spec peak
// (256 CU x 4096 FLOP/clk x 2.4 GHz) assumes the top clock; under a full MFMA load the clock is
// lower, so the attention kernel is also compared against what this loop measures.
//
// Every wave keeps four independent accumulators, so consecutive MFMAs never wait on each other,
// and touches no memory inside the loop. The first lane of each workgroup records the shader
// clock counter (s_memtime) and the constant 100 MHz counter (s_memrealtime) around the loop.
#include "dev_common.h"
#include "pisa_internal.h"

namespace pisa {
namespace {

__global__ __launch_bounds__(256) void mfma_probe(float* __restrict__ out, uint64_t* __restrict__ clk, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.125f * (float)((lane + e) & 7));
    b[e] = (__bf16)(0.0625f * (float)((3 * lane + e) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
    c0 = mfma32(a, b, c0);
    c1 = mfma32(a, b, c1);
    c2 = mfma32(a, b, c2);
    c3 = mfma32(a, b, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int x = 0; x < 16; ++x) s += (c0[x] + c1[x]) + (c2[x] + c3[x]);
  // the end stamps are taken after the results exist (the empty statement consumes s and keeps
  // its place relative to the counter reads)
  asm volatile("" ::"v"(s));
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clk[2 * (size_t)blockIdx.x] = t1 - t0;
    clk[2 * (size_t)blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

hipError_t launch_mfma_probe(int blocks, int iters, float* out, uint64_t* clk, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe, dim3(blocks), dim3(256), 0, s, out, clk, iters);
  return hipGetLastError();
}

}  // namespace pisa
