// attn_abi.cpp - the C-ABI entry points of include/attn.h: host-side validation, workspace sizing
// and kernel dispatch.
//
// TransformerEngine pull request 3705 (FROST forward provider for context-parallel attention),
// section Execution and supported scope: the steady-state native path binds the current pointers,
// workspace and stream on every call and validates operand and workspace alignment, capacity and
// overlap before launching. Pull request 3527 ("cuDNN FROST attention backend for head_dim in
// (256, 512], with context parallelism"), sections Notes for reviewers and Scope: unsupported
// configurations are declined explicitly with a reason, never served by a different computation.
#include <cmath>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <string>

#include "../../include/attn.h"
#include "../../include/attn_probe.h"
#include "attn_internal.h"

namespace {

thread_local std::string g_last_error;

attn_status_t fail(attn_status_t s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

constexpr size_t kHeader = 256;
constexpr float kLog2eHost = 1.4426950408889634f;

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

struct Info {
  bool packed;
  int64_t nq;   // query rows per head: dense batch*Sq, packed total_q
  int64_t nkv;  // key rows per kv-head
};

// Byte extent [lo, hi) of a [seq, rows, heads, D] tensor described by strides (elements).
struct Extent {
  uintptr_t lo = 0, hi = 0;
  bool huge = false;  // spans more than kMaxExtent bytes (strides or sizes no allocation can have)
  bool empty() const { return hi <= lo; }
};
constexpr __int128 kMaxExtent = (__int128)1 << 62;

Extent extent16(const void* base, const int64_t* st, bool packed, int64_t batch, int64_t rows, int64_t heads,
                int64_t d) {
  Extent e;  // a NULL base still gets its size, so that check_ptr can reject it
  if (rows <= 0 || heads <= 0 || (!packed && batch <= 0)) return e;
  // strides are non-negative (checked before); 128-bit arithmetic cannot overflow here
  __int128 last = (__int128)(rows - 1) * (packed ? st[0] : st[1]) + (__int128)(heads - 1) * (packed ? st[1] : st[2]) +
                  (d - 1);
  if (!packed) last += (__int128)(batch - 1) * st[0];
  if ((last + 1) * 2 > kMaxExtent) {
    e.huge = true;
    return e;
  }
  e.lo = (uintptr_t)base;
  e.hi = e.lo + (uintptr_t)(last + 1) * 2;
  return e;
}

bool overlaps(const Extent& a, const Extent& b) {
  return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, size_t n) { return ((uintptr_t)p % n) == 0; }

// Head dims (pull request 3527, section Scope: any multiple of 8 up to 512, padded to a compiled
// width; an asymmetric Q/K vs V/O pair). head_dim_v = 0 means the same as head_dim.
int head_dim_v(const attn_problem_t* p) { return p->head_dim_v ? p->head_dim_v : p->head_dim; }
// keys per stored dS row of the stored-dS backward: the longest key range rounded up to 64
int64_t ds_row(const attn_problem_t* p) { return ((int64_t)p->max_seqlen_kv + 63) / 64 * 64; }

attn_status_t check_head_dims(const attn_problem_t* p) {
  if (p->head_dim <= 0) return fail(ATTN_E_INVALID, "head_dim %d <= 0", p->head_dim);
  if (p->head_dim_v < 0) return fail(ATTN_E_INVALID, "head_dim_v %d < 0", p->head_dim_v);
  if (p->head_dim % 8 || p->head_dim > 512)
    return fail(ATTN_E_UNSUPPORTED, "head_dim %d is not a multiple of 8 in [8, 512]", p->head_dim);
  if (p->head_dim_v % 8 || p->head_dim_v > 512)
    return fail(ATTN_E_UNSUPPORTED, "head_dim_v %d is not 0 or a multiple of 8 in [8, 512]", p->head_dim_v);
  return ATTN_OK;
}

attn_status_t check_problem(const attn_problem_t* p, Info* info) {
  if (!p) return fail(ATTN_E_INVALID, "problem pointer is NULL");
  if (p->abi_version != ATTN_ABI_VERSION)
    return fail(ATTN_E_UNSUPPORTED, "abi_version %d is not this library's %d", p->abi_version, ATTN_ABI_VERSION);
  if (p->dtype != ATTN_BF16 && p->dtype != ATTN_FP16)
    return fail(ATTN_E_UNSUPPORTED, "dtype %d is not bf16 (0) or fp16 (1)", p->dtype);
  if (p->mask < ATTN_MASK_NONE || p->mask > ATTN_MASK_CAUSAL_BR)
    return fail(ATTN_E_UNSUPPORTED, "mask %d is not none (0), causal top-left (1) or causal bottom-right (2)",
                p->mask);
  if (p->batch < 0) return fail(ATTN_E_INVALID, "batch %d < 0", p->batch);
  if (p->heads_q < 1 || p->heads_kv < 1) return fail(ATTN_E_INVALID, "head counts must be >= 1");
  if (p->heads_q % p->heads_kv)
    return fail(ATTN_E_INVALID, "heads_q %d is not a multiple of heads_kv %d", p->heads_q, p->heads_kv);
  if (attn_status_t st = check_head_dims(p)) return st;
  if (!isfinite(p->scale)) return fail(ATTN_E_INVALID, "scale is not finite");
  if (!(p->scale > 0.f)) return fail(ATTN_E_UNSUPPORTED, "scale %g is not positive", (double)p->scale);
  if (p->max_seqlen_q < 0 || p->max_seqlen_kv < 0) return fail(ATTN_E_INVALID, "negative max_seqlen");
  if (p->window_left < -1) return fail(ATTN_E_INVALID, "window_left %d < -1", p->window_left);
  if (p->flags & ~(ATTN_FLAG_BWD_ATOMIC_DQ | ATTN_FLAG_FWD_EXP_SPLIT | ATTN_FLAG_BWD_STORED_DS))
    return fail(ATTN_E_INVALID, "unknown flags 0x%x", (unsigned)p->flags);
  if (p->window_left >= 0 && p->mask == ATTN_MASK_NONE)
    return fail(ATTN_E_UNSUPPORTED, "window_left %d needs a causal mask (the window is measured from its diagonal)",
                p->window_left);
  // one workgroup per (sequence, head, tile) of at least 64 rows or keys: every grid must fit in 32 bits
  // (units = batch * heads < 2^62 cannot overflow; the product with the tile count is tested by division)
  const int64_t uq = (int64_t)p->batch * p->heads_q, uk = (int64_t)p->batch * p->heads_kv;
  const int64_t tq = ((int64_t)p->max_seqlen_q + 63) / 64, tk = ((int64_t)p->max_seqlen_kv + 63) / 64;
  if ((uq > 0 && tq > INT32_MAX / uq) || (uk > 0 && tk > INT32_MAX / uk))
    return fail(ATTN_E_UNSUPPORTED, "batch x heads x tiles exceed the 32-bit launch grid");
  const bool packed = p->cu_seqlens_q != nullptr;
  if (packed != (p->cu_seqlens_kv != nullptr))
    return fail(ATTN_E_INVALID, "cu_seqlens_q and cu_seqlens_kv must both be set (packed) or both be NULL");
  if (packed) {
    if (p->total_q < 0 || p->total_kv < 0) return fail(ATTN_E_INVALID, "negative total_q/total_kv");
    if (p->total_q > INT32_MAX || p->total_kv > INT32_MAX)
      return fail(ATTN_E_UNSUPPORTED, "packed totals beyond int32 offsets");
    // every sequence is at most max_seqlen long, so the totals are at most batch times that
    if (p->total_q > (int64_t)p->batch * p->max_seqlen_q || p->total_kv > (int64_t)p->batch * p->max_seqlen_kv)
      return fail(ATTN_E_INVALID, "total_q / total_kv exceed batch x max_seqlen");
    if (!aligned(p->cu_seqlens_q, 4) || !aligned(p->cu_seqlens_kv, 4))
      return fail(ATTN_E_ALIGN, "cu_seqlens must be 4-byte aligned");
  }
  const int64_t* strides[4] = {p->q_stride, p->k_stride, p->v_stride, p->o_stride};
  const char* names[4] = {"q", "k", "v", "o"};
  for (int t = 0; t < 4; ++t)
    for (int i = 0; i < (packed ? 2 : 3); ++i) {
      if (strides[t][i] < 0) return fail(ATTN_E_INVALID, "%s_stride[%d] is negative", names[t], i);
      if (strides[t][i] % 8)
        return fail(ATTN_E_ALIGN, "%s_stride[%d] = %lld is not a multiple of 8 elements (16 bytes)", names[t], i,
                    (long long)strides[t][i]);
    }
  // Tiles address rows with 32-bit offsets from a 64-bit tile base: (tile rows <= 128) x row stride
  // must stay below 2^31 elements.
  for (int t = 0; t < 4; ++t) {
    const int64_t row = packed ? strides[t][0] : strides[t][1];
    if (row >= (int64_t(1) << 24))
      return fail(ATTN_E_UNSUPPORTED, "%s row stride %lld is not below 2^24 elements", names[t], (long long)row);
  }
  info->packed = packed;
  info->nq = packed ? p->total_q : (int64_t)p->batch * p->max_seqlen_q;
  info->nkv = packed ? p->total_kv : (int64_t)p->batch * p->max_seqlen_kv;
  // the stored-dS array (2 bytes per query token, head and stored key) must stay below 2^62 bytes
  if ((p->flags & ATTN_FLAG_BWD_STORED_DS) && info->nq > 0 &&
      ds_row(p) > (int64_t(1) << 61) / (info->nq * p->heads_q))
    return fail(ATTN_E_UNSUPPORTED, "the stored-dS workspace (ATTN_FLAG_BWD_STORED_DS) exceeds 2^62 bytes");
  return ATTN_OK;
}

// d: the tensor's head dim (head_dim for Q, K, dQ, dK; head_dim_v for V, O, dO, dV)
Extent ext_q(const attn_problem_t* p, const void* base, const int64_t* st, bool kv, const Info& in, int d) {
  const int64_t rows = in.packed ? (kv ? p->total_kv : p->total_q) : (kv ? p->max_seqlen_kv : p->max_seqlen_q);
  return extent16(base, st, in.packed, p->batch, rows, kv ? p->heads_kv : p->heads_q, d);
}

Extent ext_lse(const attn_problem_t* p, const float* lse, const Info& in) {
  Extent e;
  if (in.nq <= 0) return e;
  if ((__int128)in.nq * p->heads_q * 4 > kMaxExtent) {
    e.huge = true;
    return e;
  }
  e.lo = (uintptr_t)lse;
  e.hi = e.lo + (uintptr_t)(in.nq * p->heads_q) * 4;
  return e;
}

attn_status_t check_ptr(const void* ptr, const Extent& e, const char* name) {
  if (e.huge) return fail(ATTN_E_UNSUPPORTED, "%s spans more than 2^62 bytes", name);
  if (e.empty()) return ATTN_OK;  // nothing is read or written through it
  if (!ptr) return fail(ATTN_E_INVALID, "%s is NULL", name);
  if (!aligned(ptr, 16)) return fail(ATTN_E_ALIGN, "%s is not 16-byte aligned", name);
  return ATTN_OK;
}

sdpa::AttnShape make_shape(const attn_problem_t* p, const Info& in, void* ws, int qtile) {
  sdpa::AttnShape s{};
  s.cu_q = p->cu_seqlens_q;
  s.cu_kv = p->cu_seqlens_kv;
  s.err = in.packed ? (int32_t*)ws : nullptr;
  s.batch = p->batch;
  s.hq = p->heads_q;
  s.hkv = p->heads_kv;
  s.group = p->heads_q / p->heads_kv;
  s.sq = p->max_seqlen_q;
  s.skv = p->max_seqlen_kv;
  s.mask = p->mask;
  s.wl = p->window_left;
  s.dqk = p->head_dim;
  s.dv = head_dim_v(p);
  s.n_qtiles = (p->max_seqlen_q + qtile - 1) / qtile;
  s.total_q = in.packed ? p->total_q : 0;
  s.total_kv = in.packed ? p->total_kv : 0;
  s.scale = p->scale;
  s.scale_log2 = p->scale * kLog2eHost;
  return s;
}

sdpa::TensorAddr addr(const int64_t* st, bool packed) {
  sdpa::TensorAddr a;
  if (packed) {
    a.batch = 0;
    a.row = st[0];
    a.head = st[1];
  } else {
    a.batch = st[0];
    a.row = st[1];
    a.head = st[2];
  }
  return a;
}

sdpa::TensorAddr lse_addr(const attn_problem_t* p, bool packed) {
  sdpa::TensorAddr a;
  if (packed) {  // [total_q, Hq], token-major
    a.batch = 0;
    a.row = p->heads_q;
    a.head = 1;
  } else {  // [B, Hq, Sq]
    a.batch = (int64_t)p->heads_q * p->max_seqlen_q;
    a.row = 1;
    a.head = p->max_seqlen_q;
  }
  return a;
}

}  // namespace

int sdpa::fail_status_code(int s, const char* msg) {
  g_last_error = msg;
  return s;
}

extern "C" {

int32_t attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char* attn_last_error(void) { return g_last_error.c_str(); }

const char* attn_status_str(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_E_INVALID: return "ATTN_E_INVALID";
    case ATTN_E_UNSUPPORTED: return "ATTN_E_UNSUPPORTED";
    case ATTN_E_ALIGN: return "ATTN_E_ALIGN";
    case ATTN_E_OVERLAP: return "ATTN_E_OVERLAP";
    case ATTN_E_WORKSPACE: return "ATTN_E_WORKSPACE";
    case ATTN_E_HIP: return "ATTN_E_HIP";
  }
  return "ATTN_E_UNKNOWN";
}

size_t attn_fwd_workspace_bytes(const attn_problem_t* p) {
  Info in;
  if (check_problem(p, &in) != ATTN_OK) return 0;
  return in.packed ? kHeader : 0;
}

size_t attn_bwd_workspace_bytes(const attn_problem_t* p) {
  Info in;
  if (check_problem(p, &in) != ATTN_OK) return 0;
  size_t n = kHeader + 2 * round256((size_t)in.nq * p->heads_q * sizeof(float));
  if (p->flags & ATTN_FLAG_BWD_ATOMIC_DQ) n += round256((size_t)in.nq * p->heads_q * p->head_dim * sizeof(float));
  if (p->flags & ATTN_FLAG_BWD_STORED_DS) n += round256((size_t)in.nq * p->heads_q * ds_row(p) * 2);
  return n;
}

attn_status_t attn_fwd(const attn_problem_t* p, const void* q, const void* k, const void* v, void* o, float* lse,
                       void* ws, size_t ws_bytes, void* stream) {
  try {
    Info in;
    attn_status_t st = check_problem(p, &in);
    if (st != ATTN_OK) return st;
    const int dqk = p->head_dim, dv = head_dim_v(p);
    if ((p->flags & ATTN_FLAG_FWD_EXP_SPLIT) && sdpa::instance_head_dim(dqk, dv) > 256)
      return fail(ATTN_E_UNSUPPORTED, "the exp split (ATTN_FLAG_FWD_EXP_SPLIT) is built for head dims up to 256, "
                                      "not %d/%d", dqk, dv);
    const Extent eq = ext_q(p, q, p->q_stride, false, in, dqk), ek = ext_q(p, k, p->k_stride, true, in, dqk),
                 ev = ext_q(p, v, p->v_stride, true, in, dv), eo = ext_q(p, o, p->o_stride, false, in, dv),
                 el = ext_lse(p, lse, in);
    if ((st = check_ptr(q, eq, "q")) || (st = check_ptr(k, ek, "k")) || (st = check_ptr(v, ev, "v")) ||
        (st = check_ptr(o, eo, "o")))
      return st;
    if (el.huge) return fail(ATTN_E_UNSUPPORTED, "lse spans more than 2^62 bytes");
    if (!el.empty() && !lse) return fail(ATTN_E_INVALID, "lse is NULL");
    if (!el.empty() && !aligned(lse, 4)) return fail(ATTN_E_ALIGN, "lse is not 4-byte aligned");
    const size_t need = attn_fwd_workspace_bytes(p);
    if (ws_bytes < need) return fail(ATTN_E_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, need);
    if (need && (!ws || !aligned(ws, 256))) return fail(ATTN_E_WORKSPACE, "workspace NULL or not 256-byte aligned");
    Extent ew;
    if (need) {
      ew.lo = (uintptr_t)ws;
      ew.hi = ew.lo + need;
    }
    const Extent* ins[3] = {&eq, &ek, &ev};
    for (const Extent* x : ins) {
      if (overlaps(eo, *x)) return fail(ATTN_E_OVERLAP, "o overlaps an input");
      if (overlaps(el, *x)) return fail(ATTN_E_OVERLAP, "lse overlaps an input");
    }
    if (overlaps(eo, el)) return fail(ATTN_E_OVERLAP, "o overlaps lse");
    if (overlaps(ew, eo) || overlaps(ew, el) || overlaps(ew, eq) || overlaps(ew, ek) || overlaps(ew, ev))
      return fail(ATTN_E_OVERLAP, "workspace overlaps a tensor");
    sdpa::FwdArgs a{};
    const int inst = sdpa::instance_head_dim(dqk, dv);
    a.exp_split = (p->flags & ATTN_FLAG_FWD_EXP_SPLIT) != 0;
    a.s = make_shape(p, in, ws, sdpa::fwd_query_tile(inst));
    if (in.packed) {  // every packed call rewrites the error word from its own offsets
      const int e = sdpa::launch_validate_cu(a.s, stream);
      if (e) return fail(ATTN_E_HIP, "validate launch: %s", hipGetErrorString((hipError_t)e));
    }
    if (p->batch == 0 || in.nq == 0) return ATTN_OK;  // no query row: nothing to write
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.aq = addr(p->q_stride, in.packed);
    a.ak = addr(p->k_stride, in.packed);
    a.av = addr(p->v_stride, in.packed);
    a.ao = addr(p->o_stride, in.packed);
    a.alse = lse_addr(p, in.packed);
    if (a.s.n_qtiles == 0) return ATTN_OK;
    const int e = sdpa::launch_fwd(p->dtype, inst, a, stream);
    if (e) return fail(ATTN_E_HIP, "forward launch: %s", hipGetErrorString((hipError_t)e));
    return ATTN_OK;
  } catch (...) {
    return fail(ATTN_E_INVALID, "internal error");
  }
}

}  // extern "C"

namespace {

attn_status_t bwd_passes(int passes, const attn_problem_t* p, const void* q, const void* k, const void* v,
                         const void* o, const void* d_o, const float* lse, void* dq, void* dk, void* dv, void* ws,
                         size_t ws_bytes, void* stream) {
  try {
    Info in;
    attn_status_t st = check_problem(p, &in);
    if (st != ATTN_OK) return st;
    const int dqk = p->head_dim, dvw = head_dim_v(p);
    const Extent eq = ext_q(p, q, p->q_stride, false, in, dqk), ek = ext_q(p, k, p->k_stride, true, in, dqk),
                 ev = ext_q(p, v, p->v_stride, true, in, dvw), eo = ext_q(p, o, p->o_stride, false, in, dvw),
                 edo = ext_q(p, d_o, p->o_stride, false, in, dvw), el = ext_lse(p, lse, in),
                 edq = ext_q(p, dq, p->q_stride, false, in, dqk), edk = ext_q(p, dk, p->k_stride, true, in, dqk),
                 edv = ext_q(p, dv, p->v_stride, true, in, dvw);
    if ((st = check_ptr(q, eq, "q")) || (st = check_ptr(k, ek, "k")) || (st = check_ptr(v, ev, "v")) ||
        (st = check_ptr(o, eo, "o")) || (st = check_ptr(d_o, edo, "d_o")) || (st = check_ptr(dq, edq, "dq")) ||
        (st = check_ptr(dk, edk, "dk")) || (st = check_ptr(dv, edv, "dv")))
      return st;
    if (el.huge) return fail(ATTN_E_UNSUPPORTED, "lse spans more than 2^62 bytes");
    if (!el.empty() && !lse) return fail(ATTN_E_INVALID, "lse is NULL");
    if (!el.empty() && !aligned(lse, 4)) return fail(ATTN_E_ALIGN, "lse is not 4-byte aligned");
    const size_t need = attn_bwd_workspace_bytes(p);
    if (ws_bytes < need) return fail(ATTN_E_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, need);
    if (!ws || !aligned(ws, 256)) return fail(ATTN_E_WORKSPACE, "workspace NULL or not 256-byte aligned");
    Extent ew;
    ew.lo = (uintptr_t)ws;
    ew.hi = ew.lo + need;
    const Extent* ins[7] = {&eq, &ek, &ev, &eo, &edo, &el, &ew};
    const Extent* outs[3] = {&edq, &edk, &edv};
    const char* onames[3] = {"dq", "dk", "dv"};
    for (int i = 0; i < 3; ++i) {
      for (const Extent* x : ins)
        if (overlaps(*outs[i], *x)) return fail(ATTN_E_OVERLAP, "%s overlaps an input or the workspace", onames[i]);
      for (int j = i + 1; j < 3; ++j)
        if (overlaps(*outs[i], *outs[j])) return fail(ATTN_E_OVERLAP, "%s overlaps %s", onames[i], onames[j]);
    }
    for (int i = 0; i < 6; ++i)
      if (overlaps(ew, *ins[i])) return fail(ATTN_E_OVERLAP, "workspace overlaps an input");
    const bool atomic = (p->flags & ATTN_FLAG_BWD_ATOMIC_DQ) != 0;
    if (atomic && (dqk > 128 || dvw > 128))
      return fail(ATTN_E_UNSUPPORTED, "the single-pass backward (ATTN_FLAG_BWD_ATOMIC_DQ) is built for head dims up "
                  "to 128; head_dim %d, head_dim_v %d", dqk, dvw);
    if (atomic && passes == sdpa::kPassDqPre)
      return fail(ATTN_E_UNSUPPORTED, "attn_bwd_dq_preprocess has no single-pass form (ATTN_FLAG_BWD_ATOMIC_DQ): "
                  "call attn_bwd_preprocess, attn_bwd_dkdv, attn_bwd_dq");
    const bool stored_ds = (p->flags & ATTN_FLAG_BWD_STORED_DS) != 0;
    if (stored_ds && sdpa::instance_head_dim(dqk, dvw) <= 256)
      return fail(ATTN_E_UNSUPPORTED, "the stored-dS backward (ATTN_FLAG_BWD_STORED_DS) is built for head dims above "
                  "256; head_dim %d, head_dim_v %d", dqk, dvw);
    if (stored_ds && ds_row(p) >= (int64_t(1) << 24))
      return fail(ATTN_E_UNSUPPORTED, "the stored-dS backward (ATTN_FLAG_BWD_STORED_DS) takes key lengths below 2^24");
    if (stored_ds && passes == sdpa::kPassDqPre)
      return fail(ATTN_E_UNSUPPORTED, "attn_bwd_dq_preprocess has no stored-dS form (ATTN_FLAG_BWD_STORED_DS): "
                  "call attn_bwd_preprocess, attn_bwd_dkdv, attn_bwd_dq");
    sdpa::BwdArgs a{};
    const int inst = sdpa::instance_head_dim(dqk, dvw);
    a.s = make_shape(p, in, ws, sdpa::bwd_query_tile(inst));
    if (in.packed) {  // every packed call (each pass on its own too) rewrites the error word first
      const int e = sdpa::launch_validate_cu(a.s, stream);
      if (e) return fail(ATTN_E_HIP, "validate launch: %s", hipGetErrorString((hipError_t)e));
    }
    if (p->batch == 0 || (in.nq == 0 && in.nkv == 0)) return ATTN_OK;

    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.d_o = d_o;
    a.lse = lse;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.nrows = in.nq;
    a.rowsum = (float*)((char*)ws + kHeader);
    a.lse2 = (float*)((char*)ws + kHeader + round256((size_t)in.nq * p->heads_q * sizeof(float)));
    a.atomic_dq = atomic ? 1 : 0;
    a.dq_acc = atomic ? (float*)((char*)ws + kHeader + 2 * round256((size_t)in.nq * p->heads_q * sizeof(float)))
                      : nullptr;
    a.ds = stored_ds
               ? (unsigned short*)((char*)ws + kHeader + 2 * round256((size_t)in.nq * p->heads_q * sizeof(float)))
               : nullptr;
    a.ds_ld = ds_row(p);
    a.n_dsqtiles = (p->max_seqlen_q + 63) / 64;
    a.aq = addr(p->q_stride, in.packed);
    a.ak = addr(p->k_stride, in.packed);
    a.av = addr(p->v_stride, in.packed);
    a.ao = addr(p->o_stride, in.packed);
    a.alse = lse_addr(p, in.packed);
    const int kt = sdpa::bwd_key_tile(inst);
    a.n_kvtiles = (p->max_seqlen_kv + kt - 1) / kt;
    const int e = sdpa::launch_bwd(p->dtype, inst, a, passes, stream);
    if (e) return fail(ATTN_E_HIP, "backward launch: %s", hipGetErrorString((hipError_t)e));
    return ATTN_OK;
  } catch (...) {
    return fail(ATTN_E_INVALID, "internal error");
  }
}

}  // namespace

extern "C" {

attn_status_t attn_bwd(const attn_problem_t* p, const void* q, const void* k, const void* v, const void* o,
                       const void* d_o, const float* lse, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                       void* stream) {
  return bwd_passes(sdpa::kPassAll, p, q, k, v, o, d_o, lse, dq, dk, dv, ws, ws_bytes, stream);
}

attn_status_t attn_bwd_preprocess(const attn_problem_t* p, const void* q, const void* k, const void* v,
                                  const void* o, const void* d_o, const float* lse, void* dq, void* dk, void* dv,
                                  void* ws, size_t ws_bytes, void* stream) {
  return bwd_passes(sdpa::kPassPre, p, q, k, v, o, d_o, lse, dq, dk, dv, ws, ws_bytes, stream);
}

attn_status_t attn_bwd_dkdv(const attn_problem_t* p, const void* q, const void* k, const void* v, const void* o,
                            const void* d_o, const float* lse, void* dq, void* dk, void* dv, void* ws,
                            size_t ws_bytes, void* stream) {
  return bwd_passes(sdpa::kPassDkdv, p, q, k, v, o, d_o, lse, dq, dk, dv, ws, ws_bytes, stream);
}

attn_status_t attn_bwd_dq(const attn_problem_t* p, const void* q, const void* k, const void* v, const void* o,
                          const void* d_o, const float* lse, void* dq, void* dk, void* dv, void* ws,
                          size_t ws_bytes, void* stream) {
  return bwd_passes(sdpa::kPassDq, p, q, k, v, o, d_o, lse, dq, dk, dv, ws, ws_bytes, stream);
}

attn_status_t attn_bwd_dq_preprocess(const attn_problem_t* p, const void* q, const void* k, const void* v,
                                     const void* o, const void* d_o, const float* lse, void* dq, void* dk,
                                     void* dv, void* ws, size_t ws_bytes, void* stream) {
  return bwd_passes(sdpa::kPassDqPre, p, q, k, v, o, d_o, lse, dq, dk, dv, ws, ws_bytes, stream);
}

}  // extern "C"

extern "C" {

// Merge of per-chunk results (include/attn.h). Only the query side of the problem is validated.
attn_status_t attn_merge(const attn_problem_t* p, int32_t n_parts, const void* const* o_parts,
                         const float* const* lse_parts, void* o, float* lse, void* stream) {
  try {
    if (!p) return fail(ATTN_E_INVALID, "problem pointer is NULL");
    if (p->abi_version != ATTN_ABI_VERSION)
      return fail(ATTN_E_UNSUPPORTED, "abi_version %d is not this library's %d", p->abi_version, ATTN_ABI_VERSION);
    if (p->dtype != ATTN_BF16 && p->dtype != ATTN_FP16)
      return fail(ATTN_E_UNSUPPORTED, "dtype %d is not bf16 (0) or fp16 (1)", p->dtype);
    if (p->batch < 0) return fail(ATTN_E_INVALID, "batch %d < 0", p->batch);
    if (p->heads_q < 1) return fail(ATTN_E_INVALID, "heads_q must be >= 1");
    if (attn_status_t hs = check_head_dims(p)) return hs;
    const int dv = head_dim_v(p);  // the width of O
    if (p->max_seqlen_q < 0) return fail(ATTN_E_INVALID, "negative max_seqlen_q");
    if (n_parts < 1 || n_parts > ATTN_MERGE_MAX_PARTS)
      return fail(ATTN_E_INVALID, "n_parts %d is not in [1, %d]", n_parts, ATTN_MERGE_MAX_PARTS);
    if (!o_parts || !lse_parts) return fail(ATTN_E_INVALID, "o_parts or lse_parts array is NULL");
    Info in;
    in.packed = p->cu_seqlens_q != nullptr;
    if (in.packed && (p->total_q < 0 || p->total_q > INT32_MAX))
      return fail(ATTN_E_INVALID, "total_q %lld out of range", (long long)p->total_q);
    in.nq = in.packed ? p->total_q : (int64_t)p->batch * p->max_seqlen_q;
    in.nkv = 0;
    // at least 4 (row, head) pairs per workgroup: the grid fits in 32 bits
    if (in.nq > (int64_t)INT32_MAX * 4 / p->heads_q)
      return fail(ATTN_E_UNSUPPORTED, "rows x heads exceed the 32-bit launch grid");
    for (int i = 0; i < (in.packed ? 2 : 3); ++i) {
      if (p->o_stride[i] < 0) return fail(ATTN_E_INVALID, "o_stride[%d] is negative", i);
      if (p->o_stride[i] % 8)
        return fail(ATTN_E_ALIGN, "o_stride[%d] = %lld is not a multiple of 8 elements (16 bytes)", i,
                    (long long)p->o_stride[i]);
    }
    const Extent eo = ext_q(p, o, p->o_stride, false, in, dv), el = ext_lse(p, lse, in);
    attn_status_t st = check_ptr(o, eo, "o");
    if (st) return st;
    if (el.huge) return fail(ATTN_E_UNSUPPORTED, "lse spans more than 2^62 bytes");
    if (!el.empty() && !lse) return fail(ATTN_E_INVALID, "lse is NULL");
    if (!el.empty() && !aligned(lse, 4)) return fail(ATTN_E_ALIGN, "lse is not 4-byte aligned");
    if (overlaps(eo, el)) return fail(ATTN_E_OVERLAP, "o overlaps lse");
    for (int k = 0; k < n_parts; ++k) {
      const Extent ok = ext_q(p, o_parts[k], p->o_stride, false, in, dv), lk = ext_lse(p, lse_parts[k], in);
      if ((st = check_ptr(o_parts[k], ok, "o_parts[k]"))) return st;
      if (!lk.empty() && !lse_parts[k]) return fail(ATTN_E_INVALID, "lse_parts[%d] is NULL", k);
      if (!lk.empty() && !aligned(lse_parts[k], 4)) return fail(ATTN_E_ALIGN, "lse_parts[%d] is not 4-byte aligned", k);
      // an output may be exactly one of the parts (same base and layout); any other overlap is refused
      if (overlaps(eo, ok) && o != o_parts[k]) return fail(ATTN_E_OVERLAP, "o partially overlaps o_parts[%d]", k);
      if (overlaps(el, lk) && lse != lse_parts[k])
        return fail(ATTN_E_OVERLAP, "lse partially overlaps lse_parts[%d]", k);
      if (overlaps(eo, lk)) return fail(ATTN_E_OVERLAP, "o overlaps lse_parts[%d]", k);
      if (overlaps(el, ok)) return fail(ATTN_E_OVERLAP, "lse overlaps o_parts[%d]", k);
    }
    if (in.nq <= 0 || (!in.packed && p->batch == 0)) return ATTN_OK;

    sdpa::MergeArgs a{};
    for (int k = 0; k < n_parts; ++k) {
      a.o_parts[k] = o_parts[k];
      a.lse_parts[k] = lse_parts[k];
    }
    a.o = o;
    a.lse = lse;
    a.n_parts = n_parts;
    a.hq = p->heads_q;
    a.sq = p->max_seqlen_q;
    a.packed = in.packed ? 1 : 0;
    a.dv = dv;
    a.nrows = in.nq * p->heads_q;
    a.ao = addr(p->o_stride, in.packed);
    a.alse = lse_addr(p, in.packed);
    const int e = sdpa::launch_merge(p->dtype, sdpa::instance_head_dim(dv, dv), a, stream);
    if (e) return fail(ATTN_E_HIP, "merge launch: %s", hipGetErrorString((hipError_t)e));
    return ATTN_OK;
  } catch (...) {
    return fail(ATTN_E_INVALID, "internal error");
  }
}

// Matrix-core rate probe (include/attn_probe.h): a measurement aid, not part of the attention path.
attn_status_t attn_mfma_probe(int32_t blocks, int32_t iters, float x, float y, float* out, size_t out_bytes,
                              uint64_t* ticks, size_t ticks_bytes, void* stream) {
  try {
    if (blocks < 1 || blocks > ATTN_PROBE_MAX_BLOCKS)
      return fail(ATTN_E_INVALID, "blocks %d is not in [1, %d]", blocks, ATTN_PROBE_MAX_BLOCKS);
    if (iters < 1 || iters > ATTN_PROBE_MAX_ITERS)
      return fail(ATTN_E_INVALID, "iters %d is not in [1, %d]", iters, ATTN_PROBE_MAX_ITERS);
    if (!std::isfinite(x) || !std::isfinite(y)) return fail(ATTN_E_INVALID, "x and y must be finite");
    if (!out || !ticks) return fail(ATTN_E_INVALID, "out or ticks is NULL");
    if (!aligned(out, 4)) return fail(ATTN_E_ALIGN, "out is not 4-byte aligned");
    if (!aligned(ticks, 8)) return fail(ATTN_E_ALIGN, "ticks is not 8-byte aligned");
    if (out_bytes < (size_t)blocks * 256 * sizeof(float))
      return fail(ATTN_E_WORKSPACE, "out holds %zu bytes, %zu needed", out_bytes, (size_t)blocks * 256 * sizeof(float));
    if (ticks_bytes < (size_t)blocks * 2 * sizeof(uint64_t))
      return fail(ATTN_E_WORKSPACE, "ticks holds %zu bytes, %zu needed", ticks_bytes,
                  (size_t)blocks * 2 * sizeof(uint64_t));
    const uintptr_t o0 = (uintptr_t)out, o1 = o0 + (size_t)blocks * 256 * sizeof(float);
    const uintptr_t t0 = (uintptr_t)ticks, t1 = t0 + (size_t)blocks * 2 * sizeof(uint64_t);
    if (o0 < t1 && t0 < o1) return fail(ATTN_E_OVERLAP, "out overlaps ticks");
    const int e = sdpa::launch_mfma_probe(blocks, iters, x, y, out, (unsigned long long*)ticks, stream);
    if (e) return fail(ATTN_E_HIP, "probe launch: %s", hipGetErrorString((hipError_t)e));
    return ATTN_OK;
  } catch (...) {
    return fail(ATTN_E_INVALID, "internal error");
  }
}

attn_status_t attn_lds_probe(int32_t kind, const int32_t* lane_addr, int32_t iters, int32_t* out, size_t out_bytes,
                             void* stream) {
  try {
    if (kind < ATTN_LDS_READ_B128 || kind > ATTN_LDS_READ_B64) return fail(ATTN_E_INVALID, "unknown read kind %d", kind);
    if (iters < 1 || iters > ATTN_LDS_PROBE_MAX_ITERS)
      return fail(ATTN_E_INVALID, "iters %d is not in [1, %d]", iters, ATTN_LDS_PROBE_MAX_ITERS);
    if (!lane_addr || !out) return fail(ATTN_E_INVALID, "lane_addr or out is NULL");
    if (!aligned(out, 4)) return fail(ATTN_E_ALIGN, "out is not 4-byte aligned");
    if (out_bytes < 64 * sizeof(int32_t)) return fail(ATTN_E_WORKSPACE, "out holds %zu bytes, 256 needed", out_bytes);
    const int width = kind == ATTN_LDS_READ_B128 ? 16 : 8;
    for (int l = 0; l < 64; ++l) {
      const int32_t x = lane_addr[l];
      if (x < 0) continue;
      if (x % width) return fail(ATTN_E_ALIGN, "lane %d address %d is not a multiple of %d", l, x, width);
      if (x > ATTN_LDS_PROBE_BYTES - width)
        return fail(ATTN_E_INVALID, "lane %d address %d: the read passes the %d-byte array", l, x, ATTN_LDS_PROBE_BYTES);
    }
    const int e = sdpa::launch_lds_probe(kind, lane_addr, iters, out, stream);
    if (e) return fail(ATTN_E_HIP, "probe launch: %s", hipGetErrorString((hipError_t)e));
    return ATTN_OK;
  } catch (...) {
    return fail(ATTN_E_INVALID, "internal error");
  }
}

attn_status_t attn_tile_order_probe(int32_t units, int32_t tiles, int32_t reverse, int32_t order, int32_t* unit_out,
                                    int32_t* tile_out, size_t n) {
  static_assert(ATTN_ORDER_TILE_MAJOR == sdpa::kOrderTileMajor && ATTN_ORDER_QUERY == sdpa::kOrderQuery &&
                    ATTN_ORDER_GROUPED == sdpa::kOrderGrouped, "order codes");
  if (units < 1 || tiles < 1 || (int64_t)units * tiles > ATTN_TILE_ORDER_PROBE_MAX)
    return fail(ATTN_E_INVALID, "units %d x tiles %d is not in [1, %d]", units, tiles, ATTN_TILE_ORDER_PROBE_MAX);
  if (reverse != 0 && reverse != 1) return fail(ATTN_E_INVALID, "reverse must be 0 or 1");
  if (order < ATTN_ORDER_TILE_MAJOR || order > ATTN_ORDER_GROUPED) return fail(ATTN_E_INVALID, "unknown order %d", order);
  if (!unit_out || !tile_out) return fail(ATTN_E_INVALID, "unit_out or tile_out is NULL");
  if (n != (size_t)units * (size_t)tiles) return fail(ATTN_E_INVALID, "n = %zu, units x tiles = %lld", n, (long long)units * tiles);
  for (int i = 0; i < units * tiles; ++i) sdpa::tile_map_host(i, units, tiles, reverse != 0, order, unit_out + i, tile_out + i);
  return ATTN_OK;
}

}  // extern "C"
