// attn_probe.hip - measurement aids beside the attention kernels, which do not use them:
//  - the matrix-core rate the device sustains under a load of MFMA instructions alone, and its engine
//    clock meanwhile (a measured ceiling next to the published peak for the fraction-of-peak figures);
//  - an LDS read probe: one wave reading caller-chosen per-lane addresses, run under the bank-conflict
//    counter to find how the LDS serves each read width (the basis of the tile swizzle in
//    attn_device.h);
//  - the kernels' workgroup order (tile_map in attn_device.h) evaluated on the host.
#include "../../include/attn_probe.h"
#include "attn_device.h"
#include "attn_internal.h"

namespace sdpa {
namespace {

constexpr int kProbeChains = 4;  // independent accumulator chains per wave
constexpr int kLdsProbeBytes = ATTN_LDS_PROBE_BYTES;
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

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

// One wave: the LDS array is filled, then every lane whose address is not negative reads 16 (kind 0,
// ds_read_b128), 8 (kind 1, ds_read_b64_tr_b16) or 8 (kind 2, ds_read_b64) bytes at it, 8 times per
// iteration; the address passes through an empty asm statement before each read so no read is merged
// with another. Lane l writes the sum of what it read to out[l].
struct LdsProbeArgs {
  int32_t addr[64];
};
template <int KIND>
__global__ void __launch_bounds__(64) lds_probe_kernel(LdsProbeArgs a, int iters, int32_t* out) {
  __shared__ __attribute__((aligned(1024))) char buf[kLdsProbeBytes];
  for (int i = threadIdx.x; i < kLdsProbeBytes / 16; i += 64)
    reinterpret_cast<v4i*>(buf)[i] = v4i{i, 3 * i, 5 * i, 7 * i};
  __syncthreads();
  const int x0 = a.addr[threadIdx.x];
  int acc = 0;
  if (x0 >= 0) {
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        int x = x0;
        asm volatile("" : "+v"(x));
        if constexpr (KIND == 0) {
          const v4i v = *reinterpret_cast<const v4i*>(buf + x);
          acc += v[0] + v[3];
        } else if constexpr (KIND == 1) {
          const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(buf + x));
          acc += v[0] + v[3];
        } else {
          const v2i v = *reinterpret_cast<const v2i*>(buf + x);
          acc += v[0] + v[1];
        }
      }
    }
  }
  out[threadIdx.x] = acc;
}

}  // namespace

int launch_lds_probe(int kind, const int32_t* lane_addr, int iters, int32_t* out, void* stream) {
  LdsProbeArgs a;
  for (int l = 0; l < 64; ++l) a.addr[l] = lane_addr[l];
  const hipStream_t st = (hipStream_t)stream;
  if (kind == 0) hipLaunchKernelGGL(lds_probe_kernel<0>, dim3(1), dim3(64), 0, st, a, iters, out);
  else if (kind == 1) hipLaunchKernelGGL(lds_probe_kernel<1>, dim3(1), dim3(64), 0, st, a, iters, out);
  else hipLaunchKernelGGL(lds_probe_kernel<2>, dim3(1), dim3(64), 0, st, a, iters, out);
  return (int)hipGetLastError();
}

int launch_mfma_probe(int blocks, int iters, float x, float y, float* out, unsigned long long* ticks,
                      void* stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, x, y, iters,
                     out, ticks);
  return (int)hipGetLastError();
}

void tile_map_host(int i, int units, int tiles, bool reverse, int order, int* unit, int* tile) {
  int u = 0, t = 0;
  tile_map(i, units, tiles, reverse, order, u, t);
  *unit = u;
  *tile = t;
}

}  // namespace sdpa
