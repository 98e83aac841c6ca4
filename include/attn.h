/*
 * attn.h - C-ABI of the MI355X (gfx950) fused scaled-dot-product attention engine.
 *
 * The operation is the one the three pages turn on:
 *   TransformerEngine pull request 3527, "cuDNN FROST attention backend for head_dim in (256, 512],
 *   with context parallelism" - sections Approach, Verification and Scope: fused attention
 *   S = scale * Q K^T, one of the masks no_mask / causal / causal_bottom_right, softmax, O = P V,
 *   and a backward producing dQ, dK, dV; GQA and MHA; bshd-style layouts; head dims that are
 *   multiples of 8 up to 512, padded to a compiled width, and the asymmetric Q/K vs V/O pair the
 *   forward engine there lists.
 *   TransformerEngine pull request 3705 (FROST forward provider for context-parallel attention) -
 *   section Execution and supported scope: compact packed (THD) batches described by zero-based
 *   cumulative sequence lengths with no holes, checked on the device on every execution; the
 *   forward returns fp32 Stats that are natural logarithms, token-major for packed batches, and
 *   the backward consumes them; operand/workspace alignment, capacity and overlap are validated;
 *   the caller binds pointers, workspace and stream on every call.
 *   TransformerEngine pull request 3693, "Switch to Python binding for cuDNN frontend" - review
 *   comments on the fused-attention wrapper: Stats are [tq, h] for packed inputs and [b, h, sq]
 *   for dense ones; the attention scale is an fp32 value passed by value.
 *
 * Ownership: the caller allocates every buffer (inputs, outputs, workspace). The library allocates
 * nothing, frees nothing, never synchronises, keeps no pointer after a call returns and holds no
 * global mutable state apart from a thread-local error string and the device array that
 * attn_bwd_noalloc uses in place of a caller workspace (see there). Calls on different streams are
 * independent as long as their outputs and workspaces are distinct.
 *
 * Errors: every problem that is knowable on the host is reported before any launch, as a status
 * code with a reason in attn_last_error(); nothing is written in that case. An unsupported
 * feature is ATTN_E_UNSUPPORTED, never a silent fallback to another computation. HIP launch
 * failures are ATTN_E_HIP (read with hipGetLastError, no synchronisation). Malformed packed
 * sequence lengths (only visible on the device) set the workspace error word (see below) and the
 * kernels then fill every output with NaN. No C++ exception crosses this boundary.
 */
#ifndef SDPA02_ATTN_H
#define SDPA02_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 4

typedef enum {
  ATTN_OK = 0,
  ATTN_E_INVALID = 1,     /* malformed argument: null pointer, bad size, bad stride, ...       */
  ATTN_E_UNSUPPORTED = 2, /* well-formed but outside what is built (head_dim, dtype, ...)      */
  ATTN_E_ALIGN = 3,       /* a pointer or stride breaks the 16-byte alignment rule             */
  ATTN_E_OVERLAP = 4,     /* an output overlaps an input, another output or the workspace     */
  ATTN_E_WORKSPACE = 5,   /* workspace smaller than attn_*_workspace_bytes() or misaligned     */
  ATTN_E_HIP = 6          /* a kernel launch failed                                            */
} attn_status_t;

typedef enum { ATTN_BF16 = 0, ATTN_FP16 = 1 } attn_dtype_t;

/* Mask vocabulary of pull request 3527, section Scope. For query i and key j of one sequence
 * (both zero-based, lengths Sq and Skv):
 *   ATTN_MASK_NONE       every key is allowed
 *   ATTN_MASK_CAUSAL_TL  causal, top-left aligned:     allowed iff j <= i
 *   ATTN_MASK_CAUSAL_BR  causal, bottom-right aligned: allowed iff j <= i + (Skv - Sq)
 * The bottom-right band is what a context-parallel rank holding the last Sq queries of a sequence
 * needs on its trimmed KV range (pull request 3527, section Approach). A query row with no allowed
 * key gets O = 0, LSE = -inf and a zero gradient.
 * Sliding window (attn_problem_t.window_left = W >= 0, causal masks only; pull request 3527, section
 * Scope: windows measured against the top-left or bottom-right diagonal): key j is allowed for query
 * i iff i + delta - W <= j <= i + delta, with delta = 0 (TL) or Skv - Sq (BR): every query sees its
 * diagonal key and the W keys before it. W = -1 means no window. A window with ATTN_MASK_NONE has no
 * diagonal to measure from and is ATTN_E_UNSUPPORTED. */
typedef enum { ATTN_MASK_NONE = 0, ATTN_MASK_CAUSAL_TL = 1, ATTN_MASK_CAUSAL_BR = 2 } attn_mask_t;

/* One attention problem. All tensors have a contiguous head dimension (stride 1).
 *
 * Head dims (pull request 3527, section Scope: the backward engine there serves any multiple of 8
 * up to 512 by padding to its compiled width, and the forward engine lists the pair (192, 128)):
 * Q, K, dQ, dK have head_dim = D_qk elements per row, V, O, dO, dV have D_v = head_dim_v (or
 * head_dim when head_dim_v is 0); each is a multiple of 8 in [8, 512]. A call runs on the smallest
 * compiled width of 64, 128, 256, 512 that holds both, computing narrower heads as if padded with
 * zero columns: nothing is copied, no workspace is added and no byte past a row's D is read or
 * written. Below, D stands for the tensor's own head dim.
 *
 * Dense batches (cu_seqlens_q == cu_seqlens_kv == NULL): Q, O, dO, dQ are logically [B, Sq, Hq, D]
 * and K, V, dK, dV are [B, Skv, Hkv, D], with element strides (batch, sequence, head) given in
 * *_stride[0..2]; Sq = max_seqlen_q, Skv = max_seqlen_kv for every batch element. This covers
 * bshd, sbhd and bhsd storage. LSE is contiguous fp32 [B, Hq, Sq].
 *
 * Packed (THD) batches (both cu_seqlens non-NULL): Q, O, dO, dQ are [total_q, Hq, D] and K, V, dK,
 * dV are [total_kv, Hkv, D], with strides (token, head) in *_stride[0..1] (index 2 unused).
 * Sequence b owns tokens cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (and likewise for K/V); both
 * arrays are device int32[batch + 1], zero-based, non-decreasing, ending at total_q / total_kv,
 * with every sequence length <= max_seqlen_q / max_seqlen_kv and a non-empty KV range wherever the
 * query range is non-empty. LSE is contiguous fp32 [total_q, Hq] (token-major).
 *
 * Row strides (sequence stride for dense, token stride for packed) must be below 2^24 elements,
 * and batch * heads * ceil(max_seqlen / 64) must stay below 2^31 for the query side (heads_q) and
 * the key side (heads_kv): one workgroup per tile of at least 64 rows or keys; beyond that the call
 * is ATTN_E_UNSUPPORTED.
 * Grouped-query attention: q-head h reads kv-head h / (heads_q / heads_kv).
 * dQ/dK/dV use the strides of Q/K/V; dO uses the strides of O. */
typedef struct attn_problem {
  int32_t abi_version; /* must be ATTN_ABI_VERSION                                   */
  int32_t dtype;       /* attn_dtype_t: element type of Q, K, V, O, dO, dQ, dK, dV    */
  int32_t mask;        /* attn_mask_t                                                 */
  float scale;         /* > 0; multiplies Q K^T before masking and softmax (1/sqrt(D) usually) */
  int32_t batch;       /* dense batch size or number of packed sequences (>= 0)       */
  int32_t heads_q;     /* Hq >= 1                                                     */
  int32_t heads_kv;    /* Hkv >= 1, Hq % Hkv == 0                                     */
  int32_t head_dim;    /* D_qk: head dim of Q, K (multiple of 8 in [8, 512])         */
  int32_t max_seqlen_q;  /* dense: Sq; packed: an upper bound of every query length   */
  int32_t max_seqlen_kv; /* dense: Skv; packed: an upper bound of every key length    */
  const int32_t* cu_seqlens_q;  /* device int32[batch + 1] or NULL (dense)            */
  const int32_t* cu_seqlens_kv; /* device int32[batch + 1] or NULL (dense)            */
  int64_t total_q;     /* packed: cu_seqlens_q[batch] (tokens in Q); dense: ignored   */
  int64_t total_kv;    /* packed: cu_seqlens_kv[batch]; dense: ignored                */
  int64_t q_stride[3]; /* element strides, see above                                  */
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
  int32_t window_left; /* sliding window below the causal diagonal (see above); -1 = none (ABI 2) */
  int32_t head_dim_v;  /* D_v: head dim of V, O (multiple of 8 in [8, 512]); 0 = head_dim (ABI 3) */
  int32_t flags;       /* ATTN_FLAG_* bits; 0 = the defaults (ABI 4)                         */
} attn_problem_t;

/* Single-pass backward (pull request 3527, section Scope: the backward there has no deterministic mode at
 * all; this engine's default backward is deterministic and this flag trades that for speed). With the flag
 * the dK/dV pass also forms dQ += scale * dS K for its key tile and adds it with fp32 atomics into a
 * workspace buffer, so the scores and dP are computed once per allowed pair instead of twice (the default
 * dQ pass recomputes them). dQ then depends on the order of those additions: results agree with the
 * default backward to fp32 rounding, not bit for bit. Head dims up to 128 (both head_dim and head_dim_v);
 * wider heads are ATTN_E_UNSUPPORTED. The workspace grows by 4 * head_dim bytes per query row and q-head.
 * The forward ignores the flag. With it, the backward passes are: attn_bwd_preprocess (D, LSE in log2
 * units, and the zeroing of the dQ buffer), attn_bwd_dkdv (dK, dV and the dQ accumulation) and attn_bwd_dq
 * (dQ = the scaled buffer rounded to dtype), in that order; attn_bwd runs the three;
 * attn_bwd_dq_preprocess is ATTN_E_UNSUPPORTED. */
#define ATTN_FLAG_BWD_ATOMIC_DQ 1

/* Exp split in the forward (pull request 3705, section Follow-up causal THD forward kernel optimization:
 * a quarter of the softmax exponentials on interior tiles moved from the transcendental unit to an FMA
 * implementation). With the flag, on every key tile that needs no mask one in four of each lane's
 * exponentials is computed as 2^n * p(x - n), n = rint(x), p a degree-5 polynomial (Cody-Waite reduction,
 * relative error below 2.0e-7, the transcendental unit's is about the same), the others by the unit.
 * Results agree with the default forward to fp32 rounding of P, not bit for bit. Head dims up to 256
 * (both head_dim and head_dim_v); wider heads are ATTN_E_UNSUPPORTED. Measured slower on gfx950 (its
 * exponential unit overlaps the VALU and is not the limit), so off by default. The backward ignores the
 * flag. */
#define ATTN_FLAG_FWD_EXP_SPLIT 2

/* Stored-dS backward (pull request 3527, section Known limitations: the backward workspace there grows
 * super-linearly with sequence length, the price this mode pays too; the default keeps it linear). dQ =
 * scale * dS K is the gradient every backward here evaluates; with the flag the dK/dV pass also stores
 * dS = P * (dP - D), rounded to dtype, for every allowed (query, key) pair
 * into the workspace, and the dQ pass becomes the product dQ = scale * dS K over each query row's allowed
 * keys, instead of recomputing S and dP (2 * head_dim FLOP per pair instead of 6 * head_dim). Results are
 * deterministic; dQ agrees with the default backward to the rounding of its summation order, dK and dV
 * are bitwise the default ones. Head dims above 256 (head_dim or head_dim_v), the instances whose dQ
 * recompute costs more than reading dS back; narrower heads are ATTN_E_UNSUPPORTED. The workspace grows
 * by 2 * heads_q * (query tokens) * ceil(max_seqlen_kv / 64) * 64 bytes (about 2.1 GB for 16 heads at
 * 8192 x 8192), so attn_bwd_noalloc takes only small problems with it. With the flag the passes run as
 * attn_bwd_preprocess, attn_bwd_dkdv, attn_bwd_dq, in that order (dq reads the dS that dkdv stored in the
 * same workspace); attn_bwd runs the three; attn_bwd_dq_preprocess is ATTN_E_UNSUPPORTED. The forward
 * ignores the flag. */
#define ATTN_FLAG_BWD_STORED_DS 4

/* Workspace (pull request 3705, section Execution and supported scope: the caller binds the workspace
 * on every call; pull request 3527, section Known limitations: the backward workspace there grows
 * super-linearly, here it is linear in tokens). Its first 256 bytes are a header whose int32 at
 * offset 0 is the device error word: every call on a packed batch (attn_fwd, attn_bwd and each
 * backward pass on its own) first rewrites it from this call's cu_seqlens, 0 when they are valid,
 * otherwise a nonzero code (bit 0: first offset not zero; bit 1: decreasing offsets; bit 2: last
 * offset differs from total_q/total_kv; bit 3: a length exceeds max_seqlen; bit 4: queries without
 * keys), so no pre-clearing is needed and a stale word from another call is never trusted. Dense
 * calls neither read nor write it. Dense forward calls need no workspace (0 bytes; ws may be NULL).
 * The backward workspace is linear in the number of query tokens: header + two fp32 [Hq x tokens]
 * arrays (row sums D = rowsum(dO * O), and LSE in log2 units), with ATTN_FLAG_BWD_ATOMIC_DQ an fp32
 * [tokens x Hq x head_dim] dQ buffer, and with ATTN_FLAG_BWD_STORED_DS a dtype [Hq x tokens x
 * ceil(max_seqlen_kv / 64) * 64] dS array (the one workspace that is not linear in tokens). Sizes are
 * multiples of 256. */
size_t attn_fwd_workspace_bytes(const attn_problem_t* p);
size_t attn_bwd_workspace_bytes(const attn_problem_t* p);

/* Forward (pull request 3527, sections Approach and Scope: fused attention with the mask vocabulary
 * above; pull request 3705, section Execution and supported scope: the forward returns fp32 Stats in
 * natural log, token-major for packed batches):
 * O = softmax(mask(scale * Q K^T)) V and LSE = log(sum_j exp(S_ij)) (natural log, fp32).
 * q, k, v: device inputs in p->dtype; o: device output (O's strides); lse: device fp32 output;
 * ws: device workspace of ws_bytes >= attn_fwd_workspace_bytes(p), 256-byte aligned;
 * stream: the hipStream_t to launch on (NULL = the default stream). Pointers and strides must
 * be 16-byte aligned (strides multiples of 8 elements); lse 4-byte aligned. Every element of o and
 * lse is written (rows with no allowed key: O = 0, LSE = -inf). */
attn_status_t attn_fwd(const attn_problem_t* p, const void* q, const void* k, const void* v, void* o,
                       float* lse, void* ws, size_t ws_bytes, void* stream);

/* Backward (pull request 3527, sections Approach and Scope: the backward of the same fused attention,
 * producing dQ, dK, dV; pull request 3705, section Execution and supported scope: the backward
 * consumes the forward's natural-log Stats): given dO, returns dQ, dK, dV of the forward above,
 * recomputing P from the saved LSE.
 * o and lse must be the forward's outputs for the same q, k, v (O is used for the row sums
 * D = rowsum(dO * O)); d_o uses O's strides. dK and dV of kv-head g sum over the q-heads of
 * g's group. Every element of dq, dk, dv is written (keys that no query sees get zeros). The result
 * is bitwise deterministic: every output element has one writer and a fixed summation order. */
attn_status_t attn_bwd(const attn_problem_t* p, const void* q, const void* k, const void* v, const void* o,
                       const void* d_o, const float* lse, void* dq, void* dk, void* dv, void* ws,
                       size_t ws_bytes, void* stream);

/* The passes of the backward as separate calls with attn_bwd's arguments (each validates the whole
 * argument list the same way). The method's backward consists of these steps (pull request 3527,
 * section Approach; pull request 3705, section Execution and supported scope, for the Stats it
 * reads): preprocess D = rowsum(dO * O) (and LSE in log2 units, +inf for rows with no key) into the
 * workspace; the dK/dV pass, which writes dk and dv; the dQ pass, which writes dq. dkdv and dq read
 * what preprocess left in the same workspace for the same problem and inputs, so they must follow it
 * on the same stream (or after an event); they are independent of each other. Each call on a packed
 * batch rewrites the error word from its own cu_seqlens first. attn_bwd_dq_preprocess is the dQ pass
 * with the preprocess folded in (it writes the workspace's D and LSE rows for attn_bwd_dkdv, which
 * must follow it): attn_bwd runs attn_bwd_dq_preprocess then attn_bwd_dkdv for head dims up to 256,
 * and the three passes in the order preprocess, dkdv, dq for wider heads. Every split computes the
 * same quantities (up to the summation order of D). Splitting them lets a caller time or overlap the
 * passes. */
attn_status_t attn_bwd_preprocess(const attn_problem_t* p, const void* q, const void* k, const void* v,
                                  const void* o, const void* d_o, const float* lse, void* dq, void* dk, void* dv,
                                  void* ws, size_t ws_bytes, void* stream);
attn_status_t attn_bwd_dkdv(const attn_problem_t* p, const void* q, const void* k, const void* v, const void* o,
                            const void* d_o, const float* lse, void* dq, void* dk, void* dv, void* ws,
                            size_t ws_bytes, void* stream);
attn_status_t attn_bwd_dq(const attn_problem_t* p, const void* q, const void* k, const void* v, const void* o,
                          const void* d_o, const float* lse, void* dq, void* dk, void* dv, void* ws,
                          size_t ws_bytes, void* stream);
attn_status_t attn_bwd_dq_preprocess(const attn_problem_t* p, const void* q, const void* k, const void* v,
                                     const void* o, const void* d_o, const float* lse, void* dq, void* dk,
                                     void* dv, void* ws, size_t ws_bytes, void* stream);

/* The backward without a caller workspace, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Same arguments, validation,
 * kernels and results as attn_bwd (bitwise), except that the workspace is a library-owned device array
 * of ATTN_NOALLOC_MAX_WORKSPACE bytes that each GPU the library runs on holds from the first call until
 * the process ends; its device address is looked up once per device. Nothing is allocated or freed.
 * A problem whose attn_bwd_workspace_bytes() exceeds ATTN_NOALLOC_MAX_WORKSPACE (more than about 2M
 * query rows x heads) is declined with ATTN_E_WORKSPACE before any HIP call. Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (different streams without ordering
 * between them) race on it and must not be issued; calls ordered on one stream are safe. The array
 * keeps the last call's contents; nothing in it has to start at zero. */
#define ATTN_NOALLOC_MAX_WORKSPACE (16u << 20)
attn_status_t attn_bwd_noalloc(const attn_problem_t* p, const void* q, const void* k, const void* v, const void* o,
                               const void* d_o, const float* lse, void* dq, void* dk, void* dv, void* stream);

/* Merge of attention results over disjoint key chunks: the combination step of the p2p (ring)
 * context-parallel mode, which shards the keys across steps (pull request 3527, section Scope), with
 * neutral statistics for empty blocks (pull request 3693, Description). o_parts[k], lse_parts[k]
 * (k < n_parts, 1 <= n_parts <= ATTN_MERGE_MAX_PARTS; host arrays of device pointers) are attn_fwd
 * results for the same queries against disjoint key sets, laid out as attn_fwd writes O (p->o_stride)
 * and LSE. Writes, per query row and head,
 *   LSE = log(sum_k exp(LSE_k))                (natural log, fp32)
 *   O   = sum_k exp(LSE_k - LSE) * O_k         (fp32 arithmetic, rounded to p->dtype)
 * into o (p->o_stride) and lse. Parts with LSE_k = -inf contribute nothing; rows where every part is
 * -inf get O = 0, LSE = -inf. The result equals one attn_fwd over the union of the key sets (up to the
 * rounding of the parts), and merging is associative, so any number of chunks can be merged in steps.
 * Only the query side of p is used: abi_version, dtype, batch, heads_q, head_dim and head_dim_v (O
 * has head_dim_v elements per row, or head_dim when head_dim_v is 0), max_seqlen_q, o_stride, and
 * for packed batches cu_seqlens_q (marks the layout; not read) and total_q. o may be
 * exactly one of the o_parts and lse exactly one of the lse_parts (in-place accumulation); any other
 * overlap of an output with an input or with the other output is ATTN_E_OVERLAP. No workspace. */
#define ATTN_MERGE_MAX_PARTS 8
attn_status_t attn_merge(const attn_problem_t* p, int32_t n_parts, const void* const* o_parts,
                         const float* const* lse_parts, void* o, float* lse, void* stream);

const char* attn_status_str(attn_status_t s); /* static string naming the status code          */
const char* attn_last_error(void);            /* thread-local reason for this thread's last error */
int32_t attn_abi_version(void);               /* ATTN_ABI_VERSION of the built library           */

#ifdef __cplusplus
}
#endif

#endif /* SDPA02_ATTN_H */
