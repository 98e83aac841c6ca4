// attn_probe.hip - a measurement aid beside the attention kernels: the matrix-core rate the device
// sustains under a load of MFMA instructions alone, and its engine clock meanwhile. The attention
// kernels do not use it; it gives their fraction-of-peak figures a measured ceiling next to the
// published one.
#include "attn_device.h"
#include "attn_internal.h"

namespace sdpa {
namespace {

constexpr int kProbeChains = 4;  // independent accumulator chains per wave

// Every wave runs `iters` rounds of kProbeChains independent 32x32x16 bf16 MFMAs on operands held in
// registers: no memory traffic and no other instruction inside the loop. Lane l's operands are
// A[t] = bf16(x + y * (l + 8t)), B[t] = bf16(x - y * (l + 8t)), t = 0..7. Each thread then writes the
// sum of its 4 x 16 accumulator values to out[block * 256 + thread]; with y = 0 every accumulator
// element gains 16 * bf16(x)^2 per MFMA, so that sum is 1024 * bf16(x)^2 * iters. Thread 0 of each
// workgroup writes the shader-clock ticks (s_memtime) and the 100 MHz reference ticks (s_memrealtime)
// its wave spent in the loop to ticks[2 * block] and ticks[2 * block + 1].
__global__ void __launch_bounds__(256) mfma_probe_kernel(float x, float y, int iters, float* out,
                                                         unsigned long long* ticks) {
  const int lane = threadIdx.x & 63;
  v8bf a, b;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float d = y * (float)(lane + 8 * t);
    a[t] = (__bf16)(x + d);
    b[t] = (__bf16)(x - d);
  }
  v16f acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) acc[c] = v16f{};
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    ticks[2 * (int64_t)blockIdx.x] = c1 - c0;
    ticks[2 * (int64_t)blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

int launch_mfma_probe(int blocks, int iters, float x, float y, float* out, unsigned long long* ticks,
                      void* stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, x, y, iters,
                     out, ticks);
  return (int)hipGetLastError();
}

}  // namespace sdpa
