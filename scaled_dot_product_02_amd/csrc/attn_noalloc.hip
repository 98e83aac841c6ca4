// attn_noalloc.hip - attn_bwd_noalloc (include/attn.h): the backward for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// attn_bwd takes its workspace (the error word and the two fp32 [Hq x tokens] row arrays of the
// backward) from the caller. This entry point takes it from `scratch`, a file-scope device array of
// ATTN_NOALLOC_MAX_WORKSPACE bytes that every GPU the library runs on holds until the process ends,
// and otherwise runs exactly attn_bwd: the same validation and the same kernels, with the array's
// device address in place of the caller's workspace pointer.
//
// In host code `scratch` names a host-side stand-in, not the device memory: its device address is
// looked up once per device with hipGetSymbolAddress (with that device current) and only that
// address is ever handed to a kernel. Nothing here allocates or frees. Calls on one GPU share its
// array: two calls that overlap in time on one GPU (different streams, no ordering) race on it.
// Nothing in the array has to start at zero: the preprocess writes every row the passes read, and
// every call on a packed batch rewrites the error word first.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "../../include/attn.h"
#include "attn_internal.h"

static_assert(ATTN_NOALLOC_MAX_WORKSPACE % 256 == 0, "whole 256-byte blocks");

static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_MAX_WORKSPACE];

namespace {

constexpr size_t kScratchBytes = ATTN_NOALLOC_MAX_WORKSPACE;
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch` on each device, once looked up

attn_status_t fail(attn_status_t s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  return (attn_status_t)sdpa::fail_status_code(s, buf);
}

// Device address of `scratch` on device `dev`, looked up on the first call for that device with the
// device current (the caller's current device is restored afterwards).
hipError_t scratch_on(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (e2 != hipSuccess) return e2;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" attn_status_t attn_bwd_noalloc(const attn_problem_t* p, const void* q, const void* k, const void* v,
                                          const void* o, const void* d_o, const float* lse, void* dq, void* dk,
                                          void* dv, void* stream) {
  // the problem and size checks need no device: attn_bwd_workspace_bytes is host arithmetic, 0 exactly
  // for a malformed problem
  const size_t need = attn_bwd_workspace_bytes(p);
  if (need == 0)  // a malformed problem: attn_bwd declines it with its reason before any HIP call
    return attn_bwd(p, q, k, v, o, d_o, lse, dq, dk, dv, nullptr, 0, stream);
  if (need > kScratchBytes)
    return fail(ATTN_E_WORKSPACE,
                "the backward needs %zu workspace bytes; attn_bwd_noalloc holds %zu (ATTN_NOALLOC_MAX_WORKSPACE): "
                "call attn_bwd with a caller workspace",
                need, kScratchBytes);
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ATTN_E_HIP, "device of the stream: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ATTN_E_UNSUPPORTED, "device %d is past the %d this entry point serves", dev, kMaxDevices);
  void* ws = nullptr;
  if ((e = scratch_on(dev, &ws)) != hipSuccess)
    return fail(ATTN_E_HIP, "scratch address on device %d: %s", dev, hipGetErrorString(e));
  return attn_bwd(p, q, k, v, o, d_o, lse, dq, dk, dv, ws, kScratchBytes, stream);
}
