// attn_internal.h - parameter blocks passed from the host dispatcher (attn_abi.cpp) to the
// kernels (attn_kernels.hip). Not part of the public ABI.
#pragma once
#include <stdint.h>

namespace sdpa {

// Workgroup orders of tile_map (attn_device.h); the values are those of attn_probe.h's ATTN_ORDER_*.
constexpr int kOrderTileMajor = 0, kOrderQuery = 1, kOrderGrouped = 2;

// Addressing of one [sequence, head, D] tensor. Element (b, s, h, d) of a dense tensor lives at
// base + b*batch + s*row + h*head + d; for a packed tensor the sequence start token cu[b] replaces
// the batch term: base + (cu[b] + s)*row + h*head + d.
struct TensorAddr {
  int64_t batch;
  int64_t row;
  int64_t head;
};

struct AttnShape {
  const int32_t* cu_q;   // device, packed batches only (else nullptr)
  const int32_t* cu_kv;  // device, packed batches only (else nullptr)
  int32_t* err;          // device error word (packed batches) or nullptr
  int32_t batch, hq, hkv, group;  // group = hq / hkv
  int32_t sq, skv;                // dense lengths, or the host-side maxima for packed batches
  int32_t mask;                   // attn_mask_t
  int32_t wl;                     // sliding window below the diagonal, -1 = none (causal masks only)
  int32_t dqk, dv;                // head dims of Q/K and of V/O (multiples of 8, <= the kernel's D)
  int32_t n_qtiles;               // ceil(sq / query tile) of the launched kernel
  int64_t total_q, total_kv;      // packed token counts (for NaN fill on device errors)
  float scale;                    // softmax scale
  float scale_log2;               // scale * log2(e)
};

struct FwdArgs {
  AttnShape s;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  TensorAddr aq, ak, av, ao;
  TensorAddr alse;  // LSE addressing (d term absent)
  int32_t exp_split;  // ATTN_FLAG_FWD_EXP_SPLIT: a quarter of the interior tiles' exponentials on the VALU
};

struct BwdArgs {
  AttnShape s;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* d_o;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* rowsum;  // workspace: D = rowsum(dO * O), [hq][nrows]
  float* lse2;    // workspace: LSE * log2(e) (+inf for empty rows), [hq][nrows]
  int64_t nrows;  // dense: batch * sq; packed: total_q
  TensorAddr aq, ak, av, ao, alse;
  int32_t n_kvtiles;  // ceil(skv / key tile) of the dK/dV kernel
  int32_t atomic_dq;  // single-pass backward: dQ accumulated in dq_acc with fp32 atomics
  float* dq_acc;      // workspace (atomic_dq only): fp32 [nrows][hq][dqk]
  // stored-dS backward (D = 512 instances): the dK/dV pass stores dS (in dtype) into ds, and the dQ pass
  // is the product dQ = scale * dS K. ds: workspace [hq][nrows][ds_ld]; ds_ld = max key length rounded
  // up to 64; n_dsqtiles = ceil(sq / 64), the query tiles of that product. nullptr: recompute dQ.
  unsigned short* ds;
  int64_t ds_ld;
  int32_t n_dsqtiles;
};

// Merge of per-chunk results (attn_merge): nrows = query rows * hq independent (row, head) pairs.
constexpr int kMergeMaxParts = 8;
struct MergeArgs {
  const void* o_parts[kMergeMaxParts];
  const float* lse_parts[kMergeMaxParts];
  void* o;
  float* lse;
  int32_t n_parts;
  int32_t hq, sq;     // sq: dense sequence length (unused for packed)
  int32_t packed;
  int32_t dv;         // head dim of O (multiple of 8, <= the kernel's D)
  int64_t nrows;      // tokens * hq
  TensorAddr ao, alse;
};

// Launchers (attn_kernels.hip). Return hipError_t as int. head_dim is the compiled width a call runs
// on (instance_head_dim); heads narrower than it (s.dqk, s.dv) run on the padded instances.
int instance_head_dim(int dqk, int dv);  // smallest of 64, 128, 256, 512 holding both, 0 if none
int launch_validate_cu(const AttnShape& s, void* stream);
int launch_fwd(int dtype, int head_dim, const FwdArgs& a, void* stream);
// Backward passes selected by bit: 1 = preprocess, 2 = dK/dV pass, 4 = dQ pass, 8 = the dQ pass with
// the preprocess folded in (the same as 1 | 4). Preprocess and dQ together run fused for D <= 256.
// With a.atomic_dq (head dims up to 128): 1 = preprocess with the zeroing of dq_acc, 2 = the single-pass
// kernel (dK, dV and the atomic dQ accumulation), 4 = the conversion of dq_acc into dQ; 8 is not used.
enum { kPassPre = 1, kPassDkdv = 2, kPassDq = 4, kPassDqPre = 8, kPassAll = 7 };
int launch_bwd(int dtype, int head_dim, const BwdArgs& a, int passes, void* stream);
int launch_merge(int dtype, int head_dim, const MergeArgs& a, void* stream);
// Matrix-core rate probe (attn_probe.hip): blocks x 256 threads, iters rounds of four MFMAs per wave.
int launch_lds_probe(int kind, const int32_t* lane_addr, int iters, int32_t* out, void* stream);
// attn_device.h's workgroup order, evaluated on the host (attn_tile_order_probe)
void tile_map_host(int i, int units, int tiles, bool reverse, int order, int* unit, int* tile);
int launch_mfma_probe(int blocks, int iters, float x, float y, float* out, unsigned long long* ticks,
                      void* stream);
int fwd_query_tile(int head_dim);
// Records the reason attn_last_error() returns on this thread and returns s (attn_abi.cpp); for entry
// points defined in other sources.
int fail_status_code(int s, const char* msg);
int bwd_key_tile(int head_dim);
int bwd_query_tile(int head_dim);

}  // namespace sdpa
