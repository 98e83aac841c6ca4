// attn_kernels.hip - fused scaled-dot-product attention, forward and backward, for gfx950.
//
// The computation (TransformerEngine pull request 3527, "cuDNN FROST attention backend for
// head_dim in (256, 512], with context parallelism", sections Approach and Scope; pull request
// 3705, section Execution and supported scope):
//   forward   S = scale * Q K^T, mask, online softmax in the log2 domain, O = P V, and the per-row
//             natural-log LSE (fp32 Stats) that the backward consumes;
//   backward  preprocess D = rowsum(dO * O); a dK/dV pass (one workgroup per key tile, looping
//             over the query tiles and q-heads that see it); a dQ pass (one workgroup per query
//             tile, looping over the key tiles it sees). Both passes recompute P = exp(S - LSE)
//             from the saved LSE. No atomics: every output element has exactly one writer, so
//             results are deterministic.
//
// Masks: interior tiles take no mask; only tiles that cross the causal diagonal, the sequence
// tails or (bottom-right) the empty-row region are masked element by element; tiles that are
// fully masked for a whole workgroup are never loaded, and a wave skips the MFMAs of a tile that
// is fully masked for its own rows.
//
// K/V (forward, dQ pass) and Q/dO (dK/dV pass) tiles are streamed HBM -> LDS with
// global_load_lds_dwordx4 into a two-stage ring, one barrier per tile; LDS rows are XOR-swizzled
// in 16-byte chunks. Operands whose contraction index runs along LDS rows are fetched with the
// LDS transpose read (ds_read_b64_tr_b16).
#include <hip/hip_runtime.h>
#include <math.h>

#include "attn_device.h"
#include "attn_internal.h"

namespace sdpa {

typedef unsigned short us;

__device__ __forceinline__ int64_t seq_off(const TensorAddr& t, bool packed, int b, int64_t tok0) {
  return packed ? tok0 * t.row : (int64_t)b * t.batch;
}

struct Seq {
  int sq, skv;
  int64_t tq0, tk0;
};

__device__ __forceinline__ Seq seq_info(const AttnShape& s, int b) {
  Seq r;
  if (s.cu_q) {
    const int a0 = s.cu_q[b], a1 = s.cu_q[b + 1], k0 = s.cu_kv[b], k1 = s.cu_kv[b + 1];
    r.sq = a1 - a0;
    r.skv = k1 - k0;
    r.tq0 = a0;
    r.tk0 = k0;
  } else {
    r.sq = s.sq;
    r.skv = s.skv;
    r.tq0 = 0;
    r.tk0 = 0;
  }
  return r;
}

// Query-side walk of the dK/dV passes: query tiles qt0 .. qt0+nq-1 of each q-head of a GQA group in
// turn, one step per loaded tile. Running pointers to the tile's Q and dO rows and to the head's
// lse2 / D rows replace a division and several 64-bit products per tile.
template <int BQ, bool REV = false>
struct QueryWalk {  // REV: each q-head's tiles from the last one down (the D = 512 dK/dV pass)
  const us *qh, *oh, *qp, *op;
  const float *l2, *rs;
  int64_t qstep, ostep, qhead, ohead, nrows;
  int qt, qt0, qt_end;
  __device__ __forceinline__ QueryWalk(const BwdArgs& a, bool packed, int b, const Seq& sq, int h0, int qt0_, int nq)
      : qstep((int64_t)BQ * a.aq.row), ostep((int64_t)BQ * a.ao.row), qhead(a.aq.head), ohead(a.ao.head),
        nrows(a.nrows), qt(REV ? qt0_ + nq - 1 : qt0_), qt0(qt0_), qt_end(qt0_ + nq) {
    qh = (const us*)a.q + seq_off(a.aq, packed, b, sq.tq0) + (int64_t)h0 * a.aq.head;
    oh = (const us*)a.d_o + seq_off(a.ao, packed, b, sq.tq0) + (int64_t)h0 * a.ao.head;
    qp = qh + qt * qstep;
    op = oh + qt * ostep;
    const int64_t row0 = (int64_t)h0 * a.nrows + (packed ? sq.tq0 : (int64_t)b * a.s.sq);
    l2 = a.lse2 + row0;
    rs = a.rowsum + row0;
  }
  __device__ __forceinline__ void next() {
    if constexpr (REV) {
      qp -= qstep;
      op -= ostep;
      if (qt-- == qt0) {  // next q-head of the group
        qt = qt_end - 1;
        qh += qhead;
        oh += ohead;
        qp = qh + qt * qstep;
        op = oh + qt * ostep;
        l2 += nrows;
        rs += nrows;
      }
    } else {
      qp += qstep;
      op += ostep;
      if (++qt == qt_end) {  // next q-head of the group
        qt = qt0;
        qh += qhead;
        oh += ohead;
        qp = qh + qt0 * qstep;
        op = oh + qt0 * ostep;
        l2 += nrows;
        rs += nrows;
      }
    }
  }
};

// HBM -> LDS copy of one tile of two tensors X and Y (ROWS rows of D 16-bit elements each, rows
// stored with swizzled 16-byte chunks) by one wave: its NDMA 64-lane slots, slot wslot*NDMA + i
// covering 64 consecutive chunks. Each copy is a uniform 64-bit tile base plus a 32-bit per-lane
// byte offset (row strides < 2^24 elements, checked by the host), the scalar-base form of the load.
// KEEP: the per-lane offsets of full tiles stay in registers (2*NDMA of them); otherwise each tile
// clamps the lane's row and forms its offsets (a few VALU operations per copy) where registers are
// short. A tile that runs past the sequence end clamps each row to its last valid row (the repeated
// rows are masked by the kernels).
// PAD: X and Y rows hold only xd / yd (<= D, multiples of 8) elements; a lane whose chunk lies
// beyond that copies nothing (its LDS slot keeps the zeros the kernel wrote there at start), so no
// byte past a row's real width is read. The chunk of slot i depends on its row (swizzle), hence
// one bit per slot.
template <int D, int ROWS, int NDMA, bool KEEP = true, bool PAD = false>
struct TileDma {
  static constexpr int CH = D / 8;
  static_assert((ROWS * CH) % (NDMA * 64) == 0, "a tile is a whole number of wave slots");
  static_assert(NDMA <= 32, "one mask bit per slot");
  unsigned xo[KEEP ? NDMA : 1], yo[KEEP ? NDMA : 1];
  int slot0, lane;
  unsigned xrs, yrs;
  unsigned xm, ym;  // PAD: bit i set when slot i's chunk lies inside X's / Y's real width
  __device__ __forceinline__ TileDma(int wslot, int lane_, int64_t xrow, int64_t yrow, int xd = D, int yd = D)
      : slot0(wslot * NDMA * 64), lane(lane_), xrs((unsigned)xrow), yrs((unsigned)yrow), xm(0), ym(0) {
    if constexpr (KEEP) {
#pragma unroll
      for (int i = 0; i < NDMA; ++i) offsets(lane, i, ROWS, xo[i], yo[i]);
    }
    if constexpr (PAD) {
#pragma unroll
      for (int i = 0; i < NDMA; ++i) {
        const int L = slot0 + i * 64 + lane;
        const int c = (L % CH) ^ sw_key<D>(L / CH);
        xm |= (8 * c < xd ? 1u : 0u) << i;
        ym |= (8 * c < yd ? 1u : 0u) << i;
      }
    }
  }
  // byte offsets of slot i's chunk for this lane, its row clamped to last
  __device__ __forceinline__ void offsets(int ln, int i, int last, unsigned& xb, unsigned& yb) const {
    const int L = slot0 + i * 64 + ln;
    const int r = L / CH;
    const unsigned c = (unsigned)((L % CH) ^ sw_key<D>(r));
    const unsigned rc = (unsigned)min(r, last);
    xb = (rc * xrs + c * 8) * 2;
    yb = (rc * yrs + c * 8) * 2;
  }
  // xt, yt: the tile's first rows; last: index of the tile's last valid row (>= 0)
  __device__ __forceinline__ void copy(const us* xt, const us* yt, int last, us* xs, us* ys) const {
    const bool full = last >= ROWS - 1;
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      unsigned xb, yb;
      if (KEEP && full) {  // opaque: keeps the 32-bit offset (not a hoisted 64-bit copy) in the load
        xb = (unsigned)opaque((int)xo[KEEP ? i : 0]);
        yb = (unsigned)opaque((int)yo[KEEP ? i : 0]);
      } else {
        offsets(lane, i, last, xb, yb);
      }
      if (!PAD || ((xm >> i) & 1u)) dma16(xt, xb, xs + (slot0 + i * 64) * 8);
      if (!PAD || ((ym >> i) & 1u)) dma16(yt, yb, ys + (slot0 + i * 64) * 8);
    }
  }
};

template <typename T> __device__ __forceinline__ us nan_bits();
template <> __device__ __forceinline__ us nan_bits<__bf16>() { return 0x7FC0; }
template <> __device__ __forceinline__ us nan_bits<_Float16>() { return 0x7E00; }

template <typename T> __device__ __forceinline__ float to_f32(short x) {
  return (float)__builtin_bit_cast(T, x);
}

__device__ __forceinline__ int64_t flat_block() {
  return blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
}
__device__ __forceinline__ int64_t flat_grid_threads() {
  return (int64_t)gridDim.x * gridDim.y * gridDim.z * blockDim.x;
}

// Fill a packed [tokens, heads, d] tensor with NaN (grid-stride over all workgroups).
template <typename T>
__device__ void fill_nan_rows(void* base, const TensorAddr& a, int64_t tokens, int heads, int d) {
  const int CH = d / 8;
  v8s nanv;
  for (int i = 0; i < 8; ++i) nanv[i] = (short)nan_bits<T>();
  const int64_t n = tokens * heads * CH;
  for (int64_t i = flat_block() * blockDim.x + threadIdx.x; i < n; i += flat_grid_threads()) {
    const int64_t t = i / (heads * CH);
    const int rem = (int)(i % (heads * CH));
    *reinterpret_cast<v8s*>((us*)base + t * a.row + (int64_t)(rem / CH) * a.head + (rem % CH) * 8) = nanv;
  }
}

// Heads narrower than the kernel's D (PAD instances) are computed as if padded with zero columns:
// zero columns add nothing to Q K^T or dO V^T, and the padded columns of O, dQ, dK, dV are never
// stored. A chunk of 8 elements starting at column col is inside a head of width d (a multiple of 8)
// or wholly outside it.
template <bool PAD>
__device__ __forceinline__ v8s ld_chunk(const us* p, int col, int d) {
  if (PAD && col >= d) return v8s{};
  return *reinterpret_cast<const v8s*>(p);
}
// Zero N 16-bit LDS elements with the whole workgroup (the caller then synchronises).
template <int N>
__device__ __forceinline__ void zero_lds(us* p) {
  static_assert(N % 8 == 0, "whole 16-byte chunks");
  for (int i = threadIdx.x; i < N / 8; i += blockDim.x) reinterpret_cast<v8s*>(p)[i] = v8s{};
}

// ------------------------------------------------------------------------------------------
// Device check of packed sequence offsets (pull request 3705, section Execution and supported
// scope: compactness checked on the GPU on every execution). One workgroup; writes the error
// word unconditionally so no pre-clearing is needed.
// ------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) validate_cu_kernel(AttnShape s) {
  __shared__ int flag;
  if (threadIdx.x == 0) flag = 0;
  __syncthreads();
  int f = 0;
  for (int b = threadIdx.x; b < s.batch; b += blockDim.x) {
    const int q0 = s.cu_q[b], q1 = s.cu_q[b + 1], k0 = s.cu_kv[b], k1 = s.cu_kv[b + 1];
    if (q1 < q0 || k1 < k0) f |= 2;
    if (q1 - q0 > s.sq || k1 - k0 > s.skv) f |= 8;
    if (q1 > q0 && k1 == k0) f |= 16;
  }
  if (threadIdx.x == 0) {
    if (s.cu_q[0] != 0 || s.cu_kv[0] != 0) f |= 1;
    if ((int64_t)s.cu_q[s.batch] != s.total_q || (int64_t)s.cu_kv[s.batch] != s.total_kv) f |= 4;
  }
  if (f) atomicOr(&flag, f);
  __syncthreads();
  if (threadIdx.x == 0) *s.err = flag;
}

// ------------------------------------------------------------------------------------------
// Forward. Workgroup = 4 waves = 128 query rows of one (sequence, q-head); wave w owns rows
// q0 + 32w .. +31. Per key tile of BN keys the wave computes S^T = K Q^T with 32x32x16 MFMAs
// (A = K rows from LDS, B = its Q fragment held in VGPRs), so lane l holds query l%32 and half
// of the tile's keys: the row max/sum need one exchange between lanes l and l^32 (permlane swap).
// The accumulator layout of S^T is fed straight back as the B operand of O^T += V^T P^T (k slots
// permuted consistently), with V^T fetched by transpose reads.
//
// Softmax in the log2 domain with a lazy reference: P = exp2(S*c - m_ref) where m_ref is the
// row's scaled running max at the last rescale; the O accumulator and row sum are rescaled only
// when some row's max has grown by more than 2^8 since (wave-uniform branch), so P <= 2^8.
// This is exact in real arithmetic (the reference cancels in O / l and LSE = m_ref + log2 l).
// MINW = minimum waves per SIMD requested from the compiler (2 lets two workgroups share a CU so
// one wave's softmax overlaps another's MFMAs).
// ------------------------------------------------------------------------------------------
constexpr float kRescaleThreshold = 8.0f;

// EXPS: the optional exp split (ATTN_FLAG_FWD_EXP_SPLIT), one in four of each lane's exponentials on tiles
// without a mask computed by exp2_poly.
template <int D, int BN, int MINW, typename T, bool PAD, bool EXPS = false>
__global__ void __launch_bounds__(256, MINW) attn_fwd_kernel(FwdArgs a) {
  constexpr int BM = 128;
  constexpr int CH = D / 8;
  constexpr int TILE = BN * D;               // 16-bit elements of one K or V tile
  constexpr int NDMA = TILE * 2 / 1024 / 4;  // 16-byte DMA instructions per wave per tensor
  static_assert(NDMA >= 1 && (TILE * 2) % 4096 == 0, "tile must split evenly over 4 waves");
  __shared__ __attribute__((aligned(1024))) us smem[2 * 2 * TILE];
  const AttnShape& s = a.s;
  const bool packed = s.cu_q != nullptr;
  if (packed && *s.err) {
    fill_nan_rows<T>(a.o, a.ao, s.total_q, s.hq, s.dv);
    for (int64_t i = flat_block() * blockDim.x + threadIdx.x; i < s.total_q * s.hq; i += flat_grid_threads())
      a.lse[(i / s.hq) * a.alse.row + (i % s.hq) * a.alse.head] = __builtin_nanf("");
    return;
  }
  const int lane = threadIdx.x & 63, w = wave_id();
  const int hh = lane >> 5, lrow = lane & 31;
  int u, qt, b, h;
  tile_order(s.batch * s.hq, s.n_qtiles, s.mask != 0, u, qt, kOrderQuery);
  q_unit(u, s.batch, s.hkv, s.group, b, h);
  const int g = h / s.group;
  const Seq sq = seq_info(s, b);
  const int q0 = qt * BM;
  if (q0 >= sq.sq) return;
  const int delta = s.mask == 2 ? sq.skv - sq.sq : 0;
  const int kv_end = s.mask != 0 ? min(sq.skv, q0 + BM + delta) : sq.skv;
  const int n_tiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  // first key tile inside some row's sliding window (0 without a window)
  const int j0 = s.wl >= 0 ? max(0, q0 + delta - s.wl) / BN : 0;

  const us* qg = (const us*)a.q + seq_off(a.aq, packed, b, sq.tq0) + (int64_t)h * a.aq.head;
  const us* kg = (const us*)a.k + seq_off(a.ak, packed, b, sq.tk0) + (int64_t)g * a.ak.head;
  const us* vg = (const us*)a.v + seq_off(a.av, packed, b, sq.tk0) + (int64_t)g * a.av.head;
  const int qw0 = q0 + 32 * w;
  const int qi = qw0 + lrow;
  const float c = s.scale_log2;

  v8s qf[D / 16];
  {
    const us* p = qg + (int64_t)min(qi, sq.sq - 1) * a.aq.row + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = ld_chunk<PAD>(p + 16 * kk, 16 * kk + 8 * hh, s.dqk);
  }
  v16f oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = v16f{};
  float m_ref = -__builtin_inff();  // scaled (log2-domain) reference of this row
  float l_run = 0.f;                // this lane's half of the row sum, relative to m_ref

  const TileDma<D, BN, NDMA, true, PAD> dma(w, lane, a.ak.row, a.av.row, s.dqk, s.dv);
  auto issue = [&](int tile, int stage) {
    us* ks = smem + stage * 2 * TILE;
    us* vs = ks + TILE;
    const int kv0 = tile * BN;
    dma.copy(kg + (int64_t)kv0 * a.ak.row, vg + (int64_t)kv0 * a.av.row, sq.skv - 1 - kv0, ks, vs);
  };

  const int G = lane >> 4, rr = (lane >> 2) & 3, c4 = lane & 3;
  // LDS addressing (see sw_key). K rows (A of S^T): row 32kb + lrow, chunk 2kk + hh -> the lane's
  // bit hh is folded into its key, so the element offset is krow + 32kb*D + ((16kk) ^ kkey).
  // V^T by transpose reads: k-chunk cp of key block kb covers keys 32kb + 8cp + 4hh + 0..3 and the
  // same + 16 (both halves share a key); chunk 4dt + (2(G&1) + c4/2) with the lane part folded in.
  const int krow = lrow * D, kkey = (sw_key<D>(lrow) ^ hh) << 3;
  const int vrow = (4 * hh + rr) * D + 4 * (c4 & 1);
  int vkey[2];
#pragma unroll
  for (int cp = 0; cp < 2; ++cp) vkey[cp] = (sw_key<D>(8 * cp + 4 * hh + rr) ^ (2 * (G & 1) + (c4 >> 1))) << 3;
  if constexpr (PAD) {
    zero_lds<2 * 2 * TILE>(smem);
    __syncthreads();
  }
  if (j0 < n_tiles) issue(j0, j0 & 1);
  for (int j = j0; j < n_tiles; ++j) {
    wait_vmem();
    __syncthreads();
    if (j + 1 < n_tiles) issue(j + 1, (j + 1) & 1);
    const int sb = (j & 1) * 4 * TILE;  // stage, bytes; K tile at sb, V tile at sb + 2*TILE
    const int kv0 = j * BN;
    if (s.mask != 0 && kv0 > qw0 + 31 + delta) continue;  // tile fully masked for this wave
    if (s.wl >= 0 && kv0 + BN - 1 < qw0 + delta - s.wl) continue;  // tile before this wave's windows
    const bool need_mask = (kv0 + BN > sq.skv) || (s.mask != 0 && kv0 + BN - 1 > qw0 + delta) ||
                           (s.wl >= 0 && kv0 < qw0 + 31 + delta - s.wl);

    // per-tile byte bases: the stage and row parts never touch the swizzled chunk bits, so each read
    // below is one XOR with a constant (plus an immediate offset)
    const int kb_ = opaque(2 * (krow + kkey)) + sb;
    const int vb0 = opaque(2 * (vrow + vkey[0])) + sb + 2 * TILE, vb1 = opaque(2 * (vrow + 8 * D + vkey[1])) + sb + 2 * TILE;
    v16f sacc[BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) sacc[kb] = v16f{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {  // alternate accumulators between dependent MFMAs
        const v8s kf = lds_read16_at(smem, (kb_ ^ (32 * kk)) + 64 * kb * D);
        sacc[kb] = Elem<T>::mma32(Elem<T>::cast(kf), Elem<T>::cast(qf[kk]), sacc[kb]);
      }
    // schedule: the K-fragment reads run two ahead of the MFMAs that consume them
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // mask 0x100: LDS reads
#pragma unroll
    for (int i = 0; i < D / 16 * BN / 32 - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // mask 0x008: MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    // row max of the raw scores (scale c > 0); this lane's keys are kv0 + 32kb + 8(jr/4) + 4hh + jr%4
    // (one branch per tile: a mask test inside the unrolled loop becomes one branch per element)
    float mt = -__builtin_inff();
    if (need_mask) {
      const int lim = min(sq.skv - 1, s.mask == 0 ? sq.skv : qi + delta) - kv0 - 4 * hh;
      const int lo = s.wl >= 0 ? qi + delta - s.wl - kv0 - 4 * hh : -(1 << 30);  // window start
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int jr = 0; jr < 16; ++jr) {
          const int off = 32 * kb + 8 * (jr >> 2) + (jr & 3);
          const float x = off <= lim && off >= lo ? sacc[kb][jr] : -__builtin_inff();
          sacc[kb][jr] = x;
          mt = fmaxf(mt, x);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int jr = 0; jr < 16; ++jr) mt = fmaxf(mt, sacc[kb][jr]);
    }
    const float m_new = pair32_max(mt) * c;
    if (wave_any(m_new > m_ref + kRescaleThreshold)) {
      const float ref = fmaxf(m_ref, m_new);
      // 0 when m_ref = -inf; rows still without any key keep ref = -inf (O and l are 0 there)
      const float alpha = ref == -__builtin_inff() ? 0.f : fast_exp2(m_ref - ref);
      m_ref = ref;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
    }
    const float m_use = m_ref == -__builtin_inff() ? 0.f : m_ref;  // rows with no key yet: every P is 0
    if (EXPS && !need_mask) {  // exp split: one in four of the lane's exponentials on the VALU
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int jr = 0; jr < 16; ++jr) {
          const float x = __builtin_fmaf(sacc[kb][jr], c, -m_use);
          const float p = (jr & 3) == 3 ? exp2_poly(x) : fast_exp2(x);
          sacc[kb][jr] = p;
          l_run += p;
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int jr = 0; jr < 16; ++jr) {
          const float p = fast_exp2(__builtin_fmaf(sacc[kb][jr], c, -m_use));
          sacc[kb][jr] = p;
          l_run += p;
        }
    }
    // O^T += V^T P^T, 16 keys per MFMA: k-chunk cp of block kb takes S^T registers 4cp..4cp+3 and
    // 8+4cp..8+4cp+3, i.e. keys 32kb + 8cp + 4hh + 0..3 and the same + 16
#pragma unroll
    for (int cb = 0; cb < BN / 16; ++cb) {
      const int kb = cb >> 1, cp = cb & 1;
      const auto pb = pack8<T>(sacc[kb][4 * cp + 0], sacc[kb][4 * cp + 1], sacc[kb][4 * cp + 2],
                               sacc[kb][4 * cp + 3], sacc[kb][8 + 4 * cp + 0], sacc[kb][8 + 4 * cp + 1],
                               sacc[kb][8 + 4 * cp + 2], sacc[kb][8 + 4 * cp + 3]);
      const int vb = cp ? vb1 : vb0;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int o1 = (vb ^ (64 * dt)) + 64 * kb * D;
        const v4s lo = lds_read_tr_at(smem, o1);
        const v4s hi = lds_read_tr_at(smem, o1 + 32 * D);
        oacc[dt] = Elem<T>::mma32(Elem<T>::cast(cat44(lo, hi)), pb, oacc[dt]);
      }
    }
  }

  const float lt = pair32_sum(l_run);
  if (qi < sq.sq) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    T* op = (T*)a.o + seq_off(a.ao, packed, b, sq.tq0) + (int64_t)h * a.ao.head + (int64_t)qi * a.ao.row;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        typename Elem<T>::op4 v;
        v[0] = Elem<T>::cvt(oacc[dt][4 * q4 + 0] * inv);
        v[1] = Elem<T>::cvt(oacc[dt][4 * q4 + 1] * inv);
        v[2] = Elem<T>::cvt(oacc[dt][4 * q4 + 2] * inv);
        v[3] = Elem<T>::cvt(oacc[dt][4 * q4 + 3] * inv);
        if (!PAD || 32 * dt + 8 * q4 + 4 * hh < s.dv)
          *reinterpret_cast<typename Elem<T>::op4*>(op + 32 * dt + 8 * q4 + 4 * hh) = v;
      }
    if (hh == 0) {
      float* lp = a.lse + seq_off(a.alse, packed, b, sq.tq0) + (int64_t)h * a.alse.head + (int64_t)qi * a.alse.row;
      *lp = lt > 0.f ? (m_ref + __builtin_log2f(lt)) * kLn2 : -__builtin_inff();
    }
  }
}

// ------------------------------------------------------------------------------------------
// Forward for D = 512. A 32-row query block with all of its D in one wave needs Q (D/4 registers)
// plus the O accumulator (D/2) — more than the 256 registers that keep two waves per SIMD (at D = 256
// they fit, and attn_fwd_kernel serves it). So each 32-row block is shared by a wave pair: wave w (w < 4) and w + 4 own
// rows q0 + 32*(w&3) .. +31, and wave half hf = w/4 owns head-dim columns [hf*D/2, (hf+1)*D/2).
// Per key tile (BN = 32 keys) each wave computes the partial S^T over its half of D, the pair
// swaps partials through LDS (fp32) and adds own + partner (commutative: both waves hold the same
// bits), then both run the identical softmax and each accumulates O^T for its half of D. Every
// wave executes every barrier; a wave pair with no allowed key in a tile skips only its MFMAs.
// ------------------------------------------------------------------------------------------
template <int D, typename T, bool PAD>
__global__ void __launch_bounds__(512, 1) attn_fwd_split_kernel(FwdArgs a) {
  constexpr int BM = 128, BN = 32, NW = 8, DH = D / 2;
  constexpr int CH = D / 8;
  constexpr int TILE = BN * D;
  constexpr int NDMA = TILE * 2 / 1024 / NW;
  static_assert(NDMA >= 1 && (TILE * 2) % (1024 * NW) == 0, "tile must split evenly over 8 waves");
  __shared__ __attribute__((aligned(1024))) us smem[2 * 2 * TILE];
  __shared__ __attribute__((aligned(16))) float xch[NW * 16 * 64];  // partial S^T per wave
  const AttnShape& s = a.s;
  const bool packed = s.cu_q != nullptr;
  if (packed && *s.err) {
    fill_nan_rows<T>(a.o, a.ao, s.total_q, s.hq, s.dv);
    for (int64_t i = flat_block() * blockDim.x + threadIdx.x; i < s.total_q * s.hq; i += flat_grid_threads())
      a.lse[(i / s.hq) * a.alse.row + (i % s.hq) * a.alse.head] = __builtin_nanf("");
    return;
  }
  const int lane = threadIdx.x & 63, w = wave_id();
  const int pw = w & 3, hf = w >> 2;
  const int hh = lane >> 5, lrow = lane & 31;
  int u, qt, b, h;
  tile_order(s.batch * s.hq, s.n_qtiles, s.mask != 0, u, qt, kOrderQuery);
  q_unit(u, s.batch, s.hkv, s.group, b, h);
  const int g = h / s.group;
  const Seq sq = seq_info(s, b);
  const int q0 = qt * BM;
  if (q0 >= sq.sq) return;
  const int delta = s.mask == 2 ? sq.skv - sq.sq : 0;
  const int kv_end = s.mask != 0 ? min(sq.skv, q0 + BM + delta) : sq.skv;
  const int n_tiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  // first key tile inside some row's sliding window (0 without a window)
  const int j0 = s.wl >= 0 ? max(0, q0 + delta - s.wl) / BN : 0;

  const us* qg = (const us*)a.q + seq_off(a.aq, packed, b, sq.tq0) + (int64_t)h * a.aq.head;
  const us* kg = (const us*)a.k + seq_off(a.ak, packed, b, sq.tk0) + (int64_t)g * a.ak.head;
  const us* vg = (const us*)a.v + seq_off(a.av, packed, b, sq.tk0) + (int64_t)g * a.av.head;
  const int qw0 = q0 + 32 * pw;
  const int qi = qw0 + lrow;
  const float c = s.scale_log2;

  v8s qf[DH / 16];  // this wave's half of the row: d = hf*DH + 16kk + 8hh + t
  {
    const us* p = qg + (int64_t)min(qi, sq.sq - 1) * a.aq.row + hf * DH + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < DH / 16; ++kk) qf[kk] = ld_chunk<PAD>(p + 16 * kk, hf * DH + 16 * kk + 8 * hh, s.dqk);
  }
  v16f oacc[DH / 32];
#pragma unroll
  for (int dt = 0; dt < DH / 32; ++dt) oacc[dt] = v16f{};
  float m_ref = -__builtin_inff();
  float l_run = 0.f;

  const TileDma<D, BN, NDMA, (D < 512), PAD> dma(w, lane, a.ak.row, a.av.row, s.dqk, s.dv);  // registers are short at D = 512
  auto issue = [&](int tile, int stage) {
    us* ks = smem + stage * 2 * TILE;
    us* vs = ks + TILE;
    const int kv0 = tile * BN;
    dma.copy(kg + (int64_t)kv0 * a.ak.row, vg + (int64_t)kv0 * a.av.row, sq.skv - 1 - kv0, ks, vs);
  };

  float* mine = xch + w * 1024;
  const float* other = xch + (w ^ 4) * 1024;
  const int G = lane >> 4, rr = (lane >> 2) & 3, c4 = lane & 3;
  // same addressing as the D <= 128 forward, shifted by this wave's half of D (whole 16-chunk groups,
  // untouched by the swizzle)
  const int krow = lrow * D + hf * DH, kkey = (sw_key<D>(lrow) ^ hh) << 3;
  const int vrow = (4 * hh + rr) * D + 4 * (c4 & 1) + hf * DH;
  int vkey[2];
#pragma unroll
  for (int cp = 0; cp < 2; ++cp) vkey[cp] = (sw_key<D>(8 * cp + 4 * hh + rr) ^ (2 * (G & 1) + (c4 >> 1))) << 3;
  if constexpr (PAD) {
    zero_lds<2 * 2 * TILE>(smem);
    __syncthreads();
  }
  if (j0 < n_tiles) issue(j0, j0 & 1);
  for (int j = j0; j < n_tiles; ++j) {
    wait_vmem();
    __syncthreads();
    if (j + 1 < n_tiles) issue(j + 1, (j + 1) & 1);
    // per-stage byte bases: the stage, row and half-of-D parts never touch the bits the XOR constants
    // below flip, so each read is one XOR plus an immediate offset
    const int sbb = 4 * (j & 1) * TILE;
    const int kb_ = opaque(2 * (krow + kkey)) + sbb;
    const int vb0 = opaque(2 * (vrow + vkey[0])) + sbb + 2 * TILE, vb1 = opaque(2 * (vrow + 8 * D + vkey[1])) + sbb + 2 * TILE;
    const int kv0 = j * BN;
    const bool active = (s.mask == 0 || kv0 <= qw0 + 31 + delta) &&
                        (s.wl < 0 || kv0 + BN - 1 >= qw0 + delta - s.wl);  // same for both waves of a pair
    v16f sacc = v16f{};
    if (active && (!PAD || hf * DH < s.dqk)) {  // a half of D wholly past D_qk adds 0 to S
#pragma unroll
      for (int kk = 0; kk < DH / 16; ++kk) {
        const v8s kf = lds_read16_at(smem, kb_ ^ (32 * kk));
        sacc = Elem<T>::mma32(Elem<T>::cast(kf), Elem<T>::cast(qf[kk]), sacc);
      }
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {  // 4 floats per lane per group: conflict-free 16-byte writes
        v4f t4 = {sacc[4 * q4], sacc[4 * q4 + 1], sacc[4 * q4 + 2], sacc[4 * q4 + 3]};
        *reinterpret_cast<v4f*>(mine + (q4 * 64 + lane) * 4) = t4;
      }
    } else if (active) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) *reinterpret_cast<v4f*>(mine + (q4 * 64 + lane) * 4) = v4f{};
    }
    __syncthreads();
    if (!active) continue;
    if (PAD && hf * DH >= s.dv) continue;  // all of this wave's O columns lie past D_v: nothing to compute
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const v4f t4 = *reinterpret_cast<const v4f*>(other + (q4 * 64 + lane) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) sacc[4 * q4 + i] += t4[i];
    }
    // Mask, one branch per tile (the same for both waves of a pair): key kv0 + 8(jr/4) + 4hh + jr%4 is
    // allowed iff its offset 8(jr/4) + jr%4 lies in [lo, lim] (relative to kv0 + 4hh).
    const bool need_mask = (kv0 + BN > sq.skv) || (s.mask != 0 && kv0 + BN - 1 > qw0 + delta) ||
                           (s.wl >= 0 && kv0 < qw0 + 31 + delta - s.wl);
    float mt = -__builtin_inff();
    if (need_mask) {
      // (opaque: the index arithmetic stays inside the branch instead of being hoisted onto every tile)
      const int lim = opaque((s.mask != 0 ? min(sq.skv - 1, qi + delta) : sq.skv - 1) - kv0 - 4 * hh);
      const int lo = s.wl >= 0 ? qi + delta - s.wl - kv0 - 4 * hh : -(1 << 30);  // window start
#pragma unroll
      for (int jr = 0; jr < 16; ++jr) {
        const int off = 8 * (jr >> 2) + (jr & 3);
        const float x = (off <= lim && off >= lo) ? sacc[jr] : -__builtin_inff();
        sacc[jr] = x;
        mt = fmaxf(mt, x);
      }
    } else {
#pragma unroll
      for (int jr = 0; jr < 16; ++jr) mt = fmaxf(mt, sacc[jr]);
    }
    const float m_new = pair32_max(mt) * c;
    // lazy rescale (rare; wave-uniform, and the same in both waves of a pair, which hold the same S)
    if (wave_any(m_new > m_ref + kRescaleThreshold)) {
      const float ref = fmaxf(m_ref, m_new);
      // 0 when m_ref = -inf; rows still without any key keep ref = -inf (O and l are 0 there)
      const float alpha = ref == -__builtin_inff() ? 0.f : fast_exp2(m_ref - ref);
      m_ref = ref;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DH / 32; ++dt) oacc[dt] *= alpha;
    }
    const float m_use = m_ref == -__builtin_inff() ? 0.f : m_ref;
#pragma unroll
    for (int jr = 0; jr < 16; ++jr) {
      const float p = fast_exp2(__builtin_fmaf(sacc[jr], c, -m_use));
      sacc[jr] = p;
      l_run += p;
    }
#pragma unroll
    for (int cp = 0; cp < 2; ++cp) {
      const auto pb = pack8<T>(sacc[4 * cp + 0], sacc[4 * cp + 1], sacc[4 * cp + 2], sacc[4 * cp + 3],
                               sacc[8 + 4 * cp + 0], sacc[8 + 4 * cp + 1], sacc[8 + 4 * cp + 2], sacc[8 + 4 * cp + 3]);
      const int vb = cp ? vb1 : vb0;
#pragma unroll
      for (int dt = 0; dt < DH / 32; ++dt) {
        const int o1 = vb ^ (64 * dt);
        const v4s lo = lds_read_tr_at(smem, o1);
        const v4s hi = lds_read_tr_at(smem, o1 + 32 * D);
        oacc[dt] = Elem<T>::mma32(Elem<T>::cast(cat44(lo, hi)), pb, oacc[dt]);
      }
    }
  }

  const float lt = pair32_sum(l_run);
  if (qi < sq.sq) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    T* op = (T*)a.o + seq_off(a.ao, packed, b, sq.tq0) + (int64_t)h * a.ao.head + (int64_t)qi * a.ao.row + hf * DH;
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        typename Elem<T>::op4 v;
        v[0] = Elem<T>::cvt(oacc[dt][4 * q4 + 0] * inv);
        v[1] = Elem<T>::cvt(oacc[dt][4 * q4 + 1] * inv);
        v[2] = Elem<T>::cvt(oacc[dt][4 * q4 + 2] * inv);
        v[3] = Elem<T>::cvt(oacc[dt][4 * q4 + 3] * inv);
        if (!PAD || hf * DH + 32 * dt + 8 * q4 + 4 * hh < s.dv)
          *reinterpret_cast<typename Elem<T>::op4*>(op + 32 * dt + 8 * q4 + 4 * hh) = v;
      }
    if (hh == 0 && hf == 0) {
      float* lp = a.lse + seq_off(a.alse, packed, b, sq.tq0) + (int64_t)h * a.alse.head + (int64_t)qi * a.alse.row;
      *lp = lt > 0.f ? (m_ref + __builtin_log2f(lt)) * kLn2 : -__builtin_inff();
    }
  }
}

// ------------------------------------------------------------------------------------------
// Backward preprocess: D = rowsum(dO * O) in fp32 and LSE * log2(e) (+inf for rows with no key,
// so that exp2(S*c - lse2) is exactly 0 there), both stored head-major [hq][nrows]. HBM-bound.
// ------------------------------------------------------------------------------------------
template <int D, typename T>
__global__ void __launch_bounds__(256) attn_bwd_pre_kernel(BwdArgs a) {
  const AttnShape& s = a.s;
  const bool packed = s.cu_q != nullptr;
  if (packed && *s.err) return;
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int64_t total = a.nrows * s.hq;
  const int64_t R = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.f;
  int64_t t = 0, lofs = 0;
  int h = 0;
  if (R < total) {
    t = R / s.hq;
    h = (int)(R % s.hq);
    int64_t oofs;
    if (packed) {
      oofs = t * a.ao.row + (int64_t)h * a.ao.head;
      lofs = t * a.alse.row + (int64_t)h * a.alse.head;
    } else {
      const int64_t bb = t / s.sq, si = t % s.sq;
      oofs = bb * a.ao.batch + si * a.ao.row + (int64_t)h * a.ao.head;
      lofs = bb * a.alse.batch + si * a.alse.row + (int64_t)h * a.alse.head;
    }
    if (8 * c < s.dv) {  // lanes past a narrower head's width contribute 0
      const v8s o8 = *reinterpret_cast<const v8s*>((const us*)a.o + oofs + 8 * c);
      const v8s d8 = *reinterpret_cast<const v8s*>((const us*)a.d_o + oofs + 8 * c);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += to_f32<T>(o8[i]) * to_f32<T>(d8[i]);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (R < total && c == 0) {
    a.rowsum[(int64_t)h * a.nrows + t] = acc;
    const float l = a.lse[lofs];
    a.lse2[(int64_t)h * a.nrows + t] = l == -__builtin_inff() ? __builtin_inff() : l * kLog2e;
  }
}

// ------------------------------------------------------------------------------------------
// Backward dK/dV pass. Workgroup = 4 waves = BKV = 64*KB keys of one (sequence, kv-head); wave w
// owns 16*KB keys whose K and V fragments stay in VGPRs. It loops over every q-head of the GQA
// group and every query tile that sees its keys (64 rows for D <= 128, computed as 32-row halves
// under one barrier, else 32); Q, dO, lse2 and D of the tile stream through LDS. With 16x16x32 MFMAs:
//   S = Q K^T, dP = dO V^T   (A = Q / dO rows from LDS, B = K / V fragments): lane = key
//   P = exp2(S*c - lse2), dS = P (dP - D)
//   dV += P^T dO, dK += dS^T Q  (A = the P / dS accumulators as they are, B = dO / Q by transpose
//   reads). dK is scaled once at the end; keys no query sees get exact zeros.
// ------------------------------------------------------------------------------------------
template <int D, int KB, int MINW, typename T, bool PAD>
__global__ void __launch_bounds__(256, MINW) attn_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NW = 4, KW = 16 * KB, BKV = NW * KW, BQ = D <= 128 ? 64 : 32, QH = BQ / 32, CH = D / 8;
  constexpr int QTILE = BQ * D;
  constexpr int NDMA = QTILE * 2 / 1024 / NW;
  static_assert(NDMA >= 1, "query tile must split over 4 waves");
  constexpr int STAGE = 2 * QTILE + 2 * 64 * 2;  // Q, dO tiles, then lse2[64] and D[64] as floats
  __shared__ __attribute__((aligned(1024))) us smem[2 * STAGE];
  const AttnShape& s = a.s;
  const bool packed = s.cu_q != nullptr;
  if (packed && *s.err) {
    fill_nan_rows<T>(a.dk, a.ak, s.total_kv, s.hkv, s.dqk);
    fill_nan_rows<T>(a.dv, a.av, s.total_kv, s.hkv, s.dv);
    return;
  }
  const int lane = threadIdx.x & 63, w = wave_id();
  const int G = lane >> 4, l16 = lane & 15, rr = (lane >> 2) & 3, cc = lane & 3;
  int u, kt;
  tile_order(s.batch * s.hkv, a.n_kvtiles, false, u, kt, packed ? kOrderTileMajor : kOrderGrouped);
  const int b = u / s.hkv, g = u % s.hkv;
  const Seq sq = seq_info(s, b);
  kt = end_aligned(kt, a.n_kvtiles, sq.skv, BKV);
  if (kt < 0) return;
  const int k0 = kt * BKV;
  if (k0 >= sq.skv) return;
  const int kw0 = k0 + w * KW;
  const int delta = s.mask == 2 ? sq.skv - sq.sq : 0;
  const int q_lo = s.mask != 0 ? max(0, k0 - delta) : 0;
  const int qt0 = q_lo / BQ;
  // with a sliding window, rows past k0 + BKV - 1 - delta + W see none of these keys
  const int q_hi = s.wl >= 0 ? k0 + BKV - 1 - delta + s.wl : sq.sq - 1;
  const int nq = q_hi < 0 ? 0 : max(0, min((sq.sq + BQ - 1) / BQ, q_hi / BQ + 1) - qt0);
  const int n_it = nq * s.group;

  const us* kg = (const us*)a.k + seq_off(a.ak, packed, b, sq.tk0) + (int64_t)g * a.ak.head;
  const us* vg = (const us*)a.v + seq_off(a.av, packed, b, sq.tk0) + (int64_t)g * a.av.head;
  v8s kf[KB][D / 32], vf[KB][D / 32];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int64_t r = min(kw0 + 16 * kb + l16, sq.skv - 1);
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      kf[kb][kk] = ld_chunk<PAD>(kg + r * a.ak.row + 32 * kk + 8 * G, 32 * kk + 8 * G, s.dqk);
      vf[kb][kk] = ld_chunk<PAD>(vg + r * a.av.row + 32 * kk + 8 * G, 32 * kk + 8 * G, s.dv);
    }
  }
  v4f dk[KB][D / 16], dv[KB][D / 16];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      dk[kb][dt] = v4f{};
      dv[kb][dt] = v4f{};
    }

  const TileDma<D, BQ, NDMA, (D != 128), PAD> dma(w, lane, a.aq.row, a.ao.row, s.dqk, s.dv);  // registers are short at D = 128
  QueryWalk<BQ> ld(a, packed, b, sq, g * s.group, qt0, nq);
  const int qt_end = qt0 + nq;
  auto issue = [&](int stage) {
    const int qs0 = ld.qt * BQ;
    us* qs = smem + stage * STAGE;
    us* dos = qs + QTILE;
    float* l2s = reinterpret_cast<float*>(dos + QTILE);
    float* rss = l2s + 64;
    dma.copy(ld.qp, ld.op, sq.sq - 1 - qs0, qs, dos);
    const int r = min(qs0 + lane, sq.sq - 1);
    if (w == 0) dma4(ld.l2, 4u * r, l2s);
    if (w == 1) dma4(ld.rs, 4u * r, rss);
    ld.next();
  };

  // LDS offsets (elements; the reads take twice these in bytes). Row reads: Q/dO row 16m + l16, logical
  // chunk 4kk + G at ((stage + rrow + rkey) ^ 32kk) + 16m*D; transpose reads: rows 4G + rr (+16), chunk
  // 2dt + cc/2 at (stage + trow + tkey) ^ 16dt (+16D). The swizzled chunk bits (element bits
  // 3..log2(D)-1) are the only bits the keys and the XOR constants touch; the stage, row and tile offsets
  // are zero there, so adding them first and XOR-ing after gives the same offset: one XOR per read.
  const int rrow = l16 * D, rkey = (sw_key<D>(l16) ^ G) << 3;
  const int trow = (4 * G + rr) * D + 4 * (cc & 1), tkey = (sw_key<D>(4 * G + rr) ^ (cc >> 1)) << 3;
  static_assert((STAGE & (D - 1)) == 0 && (QTILE & (D - 1)) == 0, "stage offsets must leave the chunk bits alone");
  int qt_c = qt0;  // query tile of the iteration
  if constexpr (PAD) {
    zero_lds<2 * STAGE>(smem);
    __syncthreads();
  }
  if (n_it > 0) issue(0);
  for (int it = 0; it < n_it; ++it) {
    wait_vmem();
    __syncthreads();
    if (it + 1 < n_it) issue((it + 1) & 1);
    const int sb = (it & 1) * STAGE;
    const int qs0 = qt_c * BQ;
    qt_c = qt_c + 1 == qt_end ? qt0 : qt_c + 1;
    if (kw0 >= sq.skv) continue;
#pragma unroll
   for (int qh = 0; qh < QH; ++qh) {  // 32-row half of the tile
    const int qs = qs0 + 32 * qh;
    if (qs >= sq.sq) continue;
    if (s.mask != 0 && qs + 31 + delta < kw0) continue;  // no row of the half sees these keys
    if (s.wl >= 0 && qs + delta - s.wl > kw0 + KW - 1) continue;  // every row's window starts later
    const bool need_mask = (qs + 32 > sq.sq) || (kw0 + KW > sq.skv) || (s.mask != 0 && qs + delta < kw0 + KW - 1) ||
                           (s.wl >= 0 && qs + 31 + delta - s.wl > kw0);
    const int hb = 2 * sb + 64 * D * qh;  // byte offset of the half's first row
    const int rb = opaque(2 * (rrow + rkey)) + hb, tb = opaque(2 * (trow + tkey)) + hb;
    const float* l2s = reinterpret_cast<const float*>(smem + sb + 2 * QTILE) + 32 * qh;
    const float* rss = l2s + 64;
    v4f sv[2][KB], dp[2][KB];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        sv[qb][kb] = v4f{};
        dp[qb][kb] = v4f{};
      }
    // D <= 128: the S and dP products of each row block interleaved (four accumulator chains). D = 256
    // (one 16-key block per wave): S first, its exponentials then issued beside the dP products below, so
    // the transcendental unit runs under the matrix core (measured 3.8 % faster there, 3-5 % slower at
    // D = 128, where the interleaved order keeps more independent products in flight)
    constexpr bool SFIRST = D >= 256;
    if constexpr (SFIRST) {  // consecutive S products alternate the two row blocks' accumulators
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const v8s qa = lds_read16_at(smem, (rb ^ (64 * kk)) + 32 * qb * D);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
            sv[qb][kb] = Elem<T>::mma16(Elem<T>::cast(qa), Elem<T>::cast(kf[kb][kk]), sv[qb][kb]);
        }
    } else {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
          const int o = (rb ^ (64 * kk)) + 32 * qb * D;
          const v8s qa = lds_read16_at(smem, o);
          const v8s da = lds_read16_at(smem, o + 2 * QTILE);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            sv[qb][kb] = Elem<T>::mma16(Elem<T>::cast(qa), Elem<T>::cast(kf[kb][kk]), sv[qb][kb]);
            dp[qb][kb] = Elem<T>::mma16(Elem<T>::cast(da), Elem<T>::cast(vf[kb][kk]), dp[qb][kb]);
          }
        }
    }
    if (need_mask) {  // one branch per tile (a test inside the unrolled loop branches per element)
      // (opaque: the index arithmetic stays inside the branch instead of being hoisted onto every tile)
      const int ql = opaque(qs + 4 * G), kl = opaque(kw0 + l16);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int q = ql + 16 * qb + i;
            const int key = kl + 16 * kb;
            const bool ok = q < sq.sq && key < sq.skv && (s.mask == 0 || key <= q + delta) &&
                             (s.wl < 0 || key >= q + delta - s.wl);
            sv[qb][kb][i] = ok ? sv[qb][kb][i] : -__builtin_inff();  // exp2 -> exactly 0
          }
    }
    if constexpr (SFIRST) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {  // exponent arguments (their row values are in the stage already)
        const v4f l2 = *reinterpret_cast<const v4f*>(l2s + 16 * qb + 4 * G);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[qb][kb][i] = sv[qb][kb][i] * s.scale_log2 - l2[i];
      }
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const v8s da = lds_read16_at(smem, (rb ^ (64 * kk)) + 32 * qb * D + 2 * QTILE);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
            dp[qb][kb] = Elem<T>::mma16(Elem<T>::cast(da), Elem<T>::cast(vf[kb][kk]), dp[qb][kb]);
        }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[qb][kb][i] = fast_exp2(sv[qb][kb][i]);
#pragma unroll
      for (int i = 0; i < D / 32 * 2 * KB; ++i) {  // one exponential beside each dP product
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // mask 0x008: MFMA
        __builtin_amdgcn_sched_group_barrier(0x400, 1, 0);  // mask 0x400: transcendental
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const v4f dr = *reinterpret_cast<const v4f*>(rss + 16 * qb + 4 * G);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) dp[qb][kb][i] = sv[qb][kb][i] * (dp[qb][kb][i] - dr[i]);
      }
    } else {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const v4f l2 = *reinterpret_cast<const v4f*>(l2s + 16 * qb + 4 * G);
        const v4f dr = *reinterpret_cast<const v4f*>(rss + 16 * qb + 4 * G);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = fast_exp2(sv[qb][kb][i] * s.scale_log2 - l2[i]);
            sv[qb][kb][i] = p;
            dp[qb][kb][i] = p * (dp[qb][kb][i] - dr[i]);
          }
      }
    }
    typename Elem<T>::op8 pa[KB], sa[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      pa[kb] = pack8<T>(sv[0][kb][0], sv[0][kb][1], sv[0][kb][2], sv[0][kb][3], sv[1][kb][0], sv[1][kb][1],
                        sv[1][kb][2], sv[1][kb][3]);
      sa[kb] = pack8<T>(dp[0][kb][0], dp[0][kb][1], dp[0][kb][2], dp[0][kb][3], dp[1][kb][0], dp[1][kb][1],
                        dp[1][kb][2], dp[1][kb][3]);
    }
    // dO and Q fragments of column group dt + 1 are read before the products of group dt, so each
    // group's LDS latency overlaps the previous group's MFMAs (two fragment sets in flight)
    v8s dob = cat44(lds_read_tr_at(smem, tb + 2 * QTILE), lds_read_tr_at(smem, tb + 2 * QTILE + 32 * D));
    v8s qbt = cat44(lds_read_tr_at(smem, tb), lds_read_tr_at(smem, tb + 32 * D));
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      v8s dob_n = dob, qbt_n = qbt;
      if (dt + 1 < D / 16) {
        const int o1 = tb ^ (32 * (dt + 1));
        dob_n = cat44(lds_read_tr_at(smem, o1 + 2 * QTILE), lds_read_tr_at(smem, o1 + 2 * QTILE + 32 * D));
        qbt_n = cat44(lds_read_tr_at(smem, o1), lds_read_tr_at(smem, o1 + 32 * D));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        dv[kb][dt] = Elem<T>::mma16(pa[kb], Elem<T>::cast(dob), dv[kb][dt]);
        dk[kb][dt] = Elem<T>::mma16(sa[kb], Elem<T>::cast(qbt), dk[kb][dt]);
      }
      __builtin_amdgcn_sched_barrier(0);
      dob = dob_n;
      qbt = qbt_n;
    }
   }
  }

  T* dkp = (T*)a.dk + seq_off(a.ak, packed, b, sq.tk0) + (int64_t)g * a.ak.head;
  T* dvp = (T*)a.dv + seq_off(a.av, packed, b, sq.tk0) + (int64_t)g * a.av.head;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kw0 + 16 * kb + 4 * G + i;
      if (key < sq.skv) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          if (!PAD || 16 * dt + l16 < s.dqk)
            dkp[(int64_t)key * a.ak.row + 16 * dt + l16] = Elem<T>::cvt(dk[kb][dt][i] * s.scale);
          if (!PAD || 16 * dt + l16 < s.dv) dvp[(int64_t)key * a.av.row + 16 * dt + l16] = Elem<T>::cvt(dv[kb][dt][i]);
        }
      }
    }
}

// ------------------------------------------------------------------------------------------
// Backward dQ pass. Workgroup = 4 waves = 64*QB query rows of one (sequence, q-head); wave w owns
// 16*QB rows whose Q and dO fragments stay in VGPRs. K/V tiles (64 or 32 keys, see BK) stream
// through LDS.
//   S^T = K Q^T, dP^T = V dO^T  (A = K / V rows from LDS, B = Q / dO fragments): lane = query
//   P = exp2(S*c - lse2), dS = P (dP - D)            (lse2, D are per-lane scalars)
//   dQ += dS K                  (A = the dS accumulators, B = K by transpose reads)
// ------------------------------------------------------------------------------------------
// PRE: the pass also does the preprocess for its own rows (it holds their dO already): it loads O
// beside dO, forms D = rowsum(dO * O) and LSE * log2(e), uses them and stores them for the dK/dV pass,
// which then runs after it. Every query row of every head belongs to exactly one query tile.
template <int D, int QB, int MINW, typename T, bool PAD, bool PRE = false>
__global__ void __launch_bounds__(256, MINW) attn_bwd_dq_kernel(BwdArgs a) {
  // key tiles of BK = 64 (D <= 128) or 32 keys, processed as 32-key halves: a larger tile halves the
  // barriers, waits and copy issues per key at the same register use
  constexpr int NW = 4, QW = 16 * QB, BMQ = NW * QW, BK = D <= 128 ? 64 : 32, KH = BK / 32, CH = D / 8;
  constexpr int KTILE = BK * D;
  constexpr int NDMA = KTILE * 2 / 1024 / NW;
  static_assert(NDMA >= 1, "key tile must split over 4 waves");
  __shared__ __attribute__((aligned(1024))) us smem[2 * 2 * KTILE];
  const AttnShape& s = a.s;
  const bool packed = s.cu_q != nullptr;
  if (packed && *s.err) {
    fill_nan_rows<T>(a.dq, a.aq, s.total_q, s.hq, s.dqk);
    return;
  }
  const int lane = threadIdx.x & 63, w = wave_id();
  const int G = lane >> 4, l16 = lane & 15, rr = (lane >> 2) & 3, cc = lane & 3;
  int u, qt, b, h;
  tile_order(s.batch * s.hq, s.n_qtiles, s.mask != 0, u, qt, kOrderQuery);
  q_unit(u, s.batch, s.hkv, s.group, b, h);
  const int g = h / s.group;
  const Seq sq = seq_info(s, b);
  const int q0 = qt * BMQ;
  if (q0 >= sq.sq) return;
  const int delta = s.mask == 2 ? sq.skv - sq.sq : 0;
  const int kv_end = s.mask != 0 ? min(sq.skv, q0 + BMQ + delta) : sq.skv;
  const int n_tiles = kv_end > 0 ? (kv_end + BK - 1) / BK : 0;
  // first key tile inside some row's sliding window (0 without a window)
  const int j0 = s.wl >= 0 ? max(0, q0 + delta - s.wl) / BK : 0;
  const int qw0 = q0 + w * QW;
  const int64_t rowbase = packed ? sq.tq0 : (int64_t)b * s.sq;

  const us* qg = (const us*)a.q + seq_off(a.aq, packed, b, sq.tq0) + (int64_t)h * a.aq.head;
  const us* dg = (const us*)a.d_o + seq_off(a.ao, packed, b, sq.tq0) + (int64_t)h * a.ao.head;
  const us* kg = (const us*)a.k + seq_off(a.ak, packed, b, sq.tk0) + (int64_t)g * a.ak.head;
  const us* vg = (const us*)a.v + seq_off(a.av, packed, b, sq.tk0) + (int64_t)g * a.av.head;
  v8s qf[QB][D / 32], df[QB][D / 32];
  float l2[QB], dr[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int64_t r = min(qw0 + 16 * qb + l16, sq.sq - 1);
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      qf[qb][kk] = ld_chunk<PAD>(qg + r * a.aq.row + 32 * kk + 8 * G, 32 * kk + 8 * G, s.dqk);
      df[qb][kk] = ld_chunk<PAD>(dg + r * a.ao.row + 32 * kk + 8 * G, 32 * kk + 8 * G, s.dv);
    }
    if constexpr (!PRE) {
      l2[qb] = a.lse2[(int64_t)h * a.nrows + rowbase + r];
      dr[qb] = a.rowsum[(int64_t)h * a.nrows + rowbase + r];
    }
  }
  if constexpr (PRE) {
    // lanes l16, l16 + 16, l16 + 32, l16 + 48 hold a row's dO between them (chunks 32kk + 8G)
    const us* og = (const us*)a.o + seq_off(a.ao, packed, b, sq.tq0) + (int64_t)h * a.ao.head;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int q = qw0 + 16 * qb + l16;
      const int64_t r = min(q, sq.sq - 1);
      float part = 0.f;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const v8s o8 = ld_chunk<PAD>(og + r * a.ao.row + 32 * kk + 8 * G, 32 * kk + 8 * G, s.dv);
#pragma unroll
        for (int i = 0; i < 8; ++i) part += to_f32<T>(o8[i]) * to_f32<T>(df[qb][kk][i]);
      }
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      dr[qb] = part;
      const int64_t lofs = packed ? (rowbase + r) * a.alse.row + (int64_t)h * a.alse.head
                                  : (int64_t)b * a.alse.batch + r * a.alse.row + (int64_t)h * a.alse.head;
      const float l = a.lse[lofs];
      l2[qb] = l == -__builtin_inff() ? __builtin_inff() : l * kLog2e;
      if (G == 0 && q < sq.sq) {
        a.rowsum[(int64_t)h * a.nrows + rowbase + r] = dr[qb];
        a.lse2[(int64_t)h * a.nrows + rowbase + r] = l2[qb];
      }
    }
  }
  v4f dq[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) dq[qb][dt] = v4f{};

  const TileDma<D, BK, NDMA, true, PAD> dma(w, lane, a.ak.row, a.av.row, s.dqk, s.dv);
  auto issue = [&](int tile, int stage) {
    us* ks = smem + stage * 2 * KTILE;
    us* vs = ks + KTILE;
    const int kv0 = tile * BK;
    dma.copy(kg + (int64_t)kv0 * a.ak.row, vg + (int64_t)kv0 * a.av.row, sq.skv - 1 - kv0, ks, vs);
  };

  // K/V rows 16m + l16, chunk 4kk + G -> element rrow + 16m*D + ((32kk) ^ rkey); transpose reads: rows
  // 4G + rr (+16), chunk 2dt + cc/2 -> trow + ((16dt) ^ tkey) (lane chunk bits folded into the keys). The
  // reads below take these in bytes from a per-half base, one XOR each (see there).
  const int rrow = l16 * D, rkey = (sw_key<D>(l16) ^ G) << 3;
  const int trow = (4 * G + rr) * D + 4 * (cc & 1), tkey = (sw_key<D>(4 * G + rr) ^ (cc >> 1)) << 3;
  static_assert(((2 * KTILE) & (D - 1)) == 0, "stage offsets must leave the chunk bits alone");
  if constexpr (PAD) {
    zero_lds<2 * 2 * KTILE>(smem);
    __syncthreads();
  }
  if (j0 < n_tiles) issue(j0, j0 & 1);
  for (int j = j0; j < n_tiles; ++j) {
    wait_vmem();
    __syncthreads();
    if (j + 1 < n_tiles) issue(j + 1, (j + 1) & 1);
#pragma unroll
   for (int kh = 0; kh < KH; ++kh) {  // 32-key half of the tile
    // per-half byte bases: the stage, half and row parts never touch the swizzled chunk bits, so each
    // read below is one XOR with a constant plus an immediate offset
    const int hb = 4 * (j & 1) * KTILE + 64 * kh * D;
    const int rb = opaque(2 * (rrow + rkey)) + hb, tb = opaque(2 * (trow + tkey)) + hb;
    const int kv0 = j * BK + 32 * kh;
    if (s.mask != 0 && kv0 > qw0 + QW - 1 + delta) continue;
    if (s.wl >= 0 && kv0 + 31 < qw0 + delta - s.wl) continue;  // keys before this wave's windows
    const bool need_mask = (kv0 + 32 > sq.skv) || (s.mask != 0 && kv0 + 31 > qw0 + delta) ||
                           (s.wl >= 0 && kv0 < qw0 + QW - 1 + delta - s.wl);

    // D <= 128: the S and dP products interleaved per K/V fragment pair. D = 256: the S products first, then
    // the dP products with the exponentials of S issued beside them, so the transcendental unit runs under
    // the matrix core (measured 3.3 % faster there, 3-4 % slower at D <= 128)
    constexpr bool SFIRST = D >= 256;
    v4f st[2][QB], dpt[2][QB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        st[kb][qb] = v4f{};
        dpt[kb][qb] = v4f{};
      }
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const int o = (rb ^ (64 * kk)) + 32 * kb * D;
        const v8s ka = lds_read16_at(smem, o);
        v8s va;
        if constexpr (!SFIRST) va = lds_read16_at(smem, o + 2 * KTILE);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          st[kb][qb] = Elem<T>::mma16(Elem<T>::cast(ka), Elem<T>::cast(qf[qb][kk]), st[kb][qb]);
          if constexpr (!SFIRST)
            dpt[kb][qb] = Elem<T>::mma16(Elem<T>::cast(va), Elem<T>::cast(df[qb][kk]), dpt[kb][qb]);
        }
      }
    }
    if constexpr (SFIRST) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
          const v8s va = lds_read16_at(smem, (rb ^ (64 * kk)) + 32 * kb * D + 2 * KTILE);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            dpt[kb][qb] = Elem<T>::mma16(Elem<T>::cast(va), Elem<T>::cast(df[qb][kk]), dpt[kb][qb]);
        }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[kb][qb][i] = fast_exp2(st[kb][qb][i] * s.scale_log2 - l2[qb]);
    if constexpr (SFIRST) {
#pragma unroll
      for (int i = 0; i < D / 32 * 2 * QB; ++i) {  // one exponential beside each dP product
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // mask 0x008: MFMA
        __builtin_amdgcn_sched_group_barrier(0x400, 1, 0);  // mask 0x400: transcendental
      }
    }
    if (need_mask) {  // one branch per tile (a test inside the unrolled loop branches per element)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int q = qw0 + 16 * qb + l16;
            const int key = kv0 + 16 * kb + 4 * G + i;
            const bool ok = key < sq.skv && (s.mask == 0 || key <= q + delta) && (s.wl < 0 || key >= q + delta - s.wl);
            st[kb][qb][i] = ok ? st[kb][qb][i] : 0.f;
          }
    }
    typename Elem<T>::op8 dsa[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float ds[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) ds[kb][i] = st[kb][qb][i] * (dpt[kb][qb][i] - dr[qb]);
      dsa[qb] = pack8<T>(ds[0][0], ds[0][1], ds[0][2], ds[0][3], ds[1][0], ds[1][1], ds[1][2], ds[1][3]);
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const int o1 = tb ^ (32 * dt);
      const v8s kbt = cat44(lds_read_tr_at(smem, o1), lds_read_tr_at(smem, o1 + 32 * D));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) dq[qb][dt] = Elem<T>::mma16(dsa[qb], Elem<T>::cast(kbt), dq[qb][dt]);
    }
   }
  }

  T* dqp = (T*)a.dq + seq_off(a.aq, packed, b, sq.tq0) + (int64_t)h * a.aq.head;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = qw0 + 16 * qb + 4 * G + i;
      if (q < sq.sq) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
          if (!PAD || 16 * dt + l16 < s.dqk)
            dqp[(int64_t)q * a.aq.row + 16 * dt + l16] = Elem<T>::cvt(dq[qb][dt][i] * s.scale);
      }
    }
}

// ------------------------------------------------------------------------------------------
// Backward for D = 512. One wave cannot hold 16 keys' K and V fragments (128 registers) plus their
// dK and dV accumulators (256), nor 16 query rows' Q and dO (128) plus dQ (128), within the 256
// registers that keep two waves per SIMD. So both passes pair waves (8 waves per workgroup):
//
// dK/dV: the pair (w, w+4) owns 16 keys. Wave w holds K, computes S = Q K^T and P = exp2(S*c - lse2),
// hands P (fp32) to its partner through LDS and accumulates dV += P^T dO. Wave w+4 holds V, computes
// dP = dO V^T, takes P, forms dS = P (dP - D) and accumulates dK += dS^T Q. Both do 4*D MFMA work
// per pair. dQ: the pair owns 16 query rows; wave w holds Q and computes P, wave w+4 holds dO and
// computes dP, they swap (fp32), both form the same dS, and each accumulates half of dQ's columns.
// Every wave executes every barrier; a pair whose keys / rows see nothing in a tile skips its MFMAs.
// ------------------------------------------------------------------------------------------
template <int D, typename T, bool PAD, bool STORE_DS = false>
__global__ void __launch_bounds__(512, 1) attn_bwd_dkdv_pair_kernel(BwdArgs a) {
  constexpr int NW = 8, KW = 16, BKV = 4 * KW, BQ = 32, CH = D / 8;
  constexpr int QTILE = BQ * D;
  constexpr int NDMA = QTILE * 2 / 1024 / NW;
  static_assert(NDMA >= 1, "query tile must split over 8 waves");
  // Q, dO tiles, then lse2[64] and D[64] as floats, padded so that a stage offset leaves the chunk bits
  // of a row alone (the reads below XOR them into per-stage byte bases)
  constexpr int STAGE = 2 * QTILE + D;
  static_assert((STAGE & (D - 1)) == 0 && 2 * 64 * 2 <= D, "stage padding");
  __shared__ __attribute__((aligned(1024))) us smem[2 * STAGE];
  __shared__ __attribute__((aligned(16))) float xch[4 * 2 * 64 * 4];  // P per pair: [qb][lane][4]
  __shared__ __attribute__((aligned(16))) us dsst[STORE_DS ? 4 * 32 * 16 : 8];  // STORE_DS: dS per pair, [row][key]
  const AttnShape& s = a.s;
  const bool packed = s.cu_q != nullptr;
  if (packed && *s.err) {
    fill_nan_rows<T>(a.dk, a.ak, s.total_kv, s.hkv, s.dqk);
    fill_nan_rows<T>(a.dv, a.av, s.total_kv, s.hkv, s.dv);
    return;
  }
  const int lane = threadIdx.x & 63, w = wave_id();
  const int pr = w & 3, role = w >> 2;  // role 0: K, S, P, dV; role 1: V, dP, dS, dK
  const int G = lane >> 4, l16 = lane & 15, rr = (lane >> 2) & 3, cc = lane & 3;
  int u, kt;
  tile_order(s.batch * s.hkv, a.n_kvtiles, false, u, kt, packed ? kOrderTileMajor : kOrderGrouped);
  const int b = u / s.hkv, g = u % s.hkv;
  const Seq sq = seq_info(s, b);
  kt = end_aligned(kt, a.n_kvtiles, sq.skv, BKV);
  if (kt < 0) return;
  const int k0 = kt * BKV;
  if (k0 >= sq.skv) return;
  const int kw0 = k0 + pr * KW;
  const int delta = s.mask == 2 ? sq.skv - sq.sq : 0;
  const int q_lo = s.mask != 0 ? max(0, k0 - delta) : 0;
  const int qt0 = q_lo / BQ;
  // with a sliding window, rows past k0 + BKV - 1 - delta + W see none of these keys
  const int q_hi = s.wl >= 0 ? k0 + BKV - 1 - delta + s.wl : sq.sq - 1;
  const int nq = q_hi < 0 ? 0 : max(0, min((sq.sq + BQ - 1) / BQ, q_hi / BQ + 1) - qt0);
  const int n_it = nq * s.group;

  // role 0 keeps K, role 1 keeps V (B operands: key kw0 + l16, d = 32kk + 8G + t)
  const us* kvg = role == 0 ? (const us*)a.k + seq_off(a.ak, packed, b, sq.tk0) + (int64_t)g * a.ak.head
                            : (const us*)a.v + seq_off(a.av, packed, b, sq.tk0) + (int64_t)g * a.av.head;
  const int64_t kvrow = role == 0 ? a.ak.row : a.av.row;
  v8s kvf[D / 32];
  {
    const int64_t r = min(kw0 + l16, sq.skv - 1);
    const int kvd = role == 0 ? s.dqk : s.dv;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) kvf[kk] = ld_chunk<PAD>(kvg + r * kvrow + 32 * kk + 8 * G, 32 * kk + 8 * G, kvd);
  }
  v4f acc[D / 16];  // dV (role 0) or dK (role 1): key kw0 + 4G + i, d = 16dt + l16
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = v4f{};

  const TileDma<D, BQ, NDMA, true, PAD> dma(w, lane, a.aq.row, a.ao.row, s.dqk, s.dv);
  // query tiles from the last one down: the workgroups an XCD runs together (key blocks of one kv-head) then
  // read the same Q/dO tile at about the same time, from L2, instead of each starting at its own diagonal
  QueryWalk<BQ, true> ld(a, packed, b, sq, g * s.group, qt0, nq);
  const int qt_end = qt0 + nq;
  auto issue = [&](int stage) {
    const int qs0 = ld.qt * BQ;
    us* qs = smem + stage * STAGE;
    us* dos = qs + QTILE;
    float* l2s = reinterpret_cast<float*>(dos + QTILE);
    float* rss = l2s + 64;
    dma.copy(ld.qp, ld.op, sq.sq - 1 - qs0, qs, dos);
    const int r = min(qs0 + lane, sq.sq - 1);
    if (w == 0) dma4(ld.l2, 4u * r, l2s);
    if (w == 1) dma4(ld.rs, 4u * r, rss);
    ld.next();
  };

  // Q/dO rows 16m + l16, chunk 4kk + G -> element rrow + 16m*D + ((32kk) ^ rkey); transpose reads: rows
  // 4G + rr (+16), chunk 2dt + cc/2 -> trow + ((16dt) ^ tkey) (lane chunk bits folded into the keys). The
  // reads take these in bytes from per-stage bases, one XOR each.
  const int rrow = l16 * D, rkey = (sw_key<D>(l16) ^ G) << 3;
  const int trow = (4 * G + rr) * D + 4 * (cc & 1), tkey = (sw_key<D>(4 * G + rr) ^ (cc >> 1)) << 3;
  float* pbuf = xch + pr * 2 * 64 * 4;
  const int64_t rowbase = packed ? sq.tq0 : (int64_t)b * s.sq;  // the sequence's first query token

  int qt_c = qt_end - 1, hq_c = g * s.group;  // query tile and q-head of the iteration (tiles walked downwards)

  // stored-dS backward (STORE_DS, an instance of its own: the default one keeps its registers): the
  // role-1 wave of a pair puts the dS of an iteration (rounded to T: the values of its dK product) into
  // its [32 row][16 key] LDS buffer and, after the next barrier, reads it back 8 keys of a row per lane
  // and writes them out as one 16-byte run, so that the copy wait before that barrier does not also wait
  // for these stores and no register stays live across the S/dP products. Key 16a + 8c + 4h + j of a
  // 32-key block goes to position 16c + 8a + 4h + j (the order attn_bwd_dq_ds_kernel reads; a pair of
  // waves holds one a); rows past the sequence end are not stored.
  int ds_qs0 = 0, ds_h = 0;
  bool ds_pending = false;
  auto store_ds = [&]() {
    if (!STORE_DS || !ds_pending) return;
    const int r = lane >> 1, c = lane & 1;  // row r, keys 8c .. 8c + 7 of the pair
    const v8s x = *reinterpret_cast<const v8s*>(dsst + pr * 512 + r * 16 + 8 * c);
    if (ds_qs0 + r < sq.sq) {
      T* dsp = reinterpret_cast<T*>(a.ds) + ((int64_t)ds_h * a.nrows + rowbase + ds_qs0 + r) * a.ds_ld +
               (kw0 - (kw0 & 31)) + 16 * c + 8 * ((kw0 >> 4) & 1);
      *reinterpret_cast<v8s*>(dsp) = x;  // plain store: the two pairs' runs of a 32-byte sector merge in L2
    }
    ds_pending = false;
  };
  if constexpr (PAD) {
    zero_lds<2 * STAGE>(smem);
    __syncthreads();
  }
  if (n_it > 0) issue(0);
  for (int it = 0; it < n_it; ++it) {
    wait_vmem();
    __syncthreads();
    if (it + 1 < n_it) issue((it + 1) & 1);
    store_ds();
    // per-stage byte bases of this wave's row reads (Q for role 0, dO for role 1) and transpose reads
    // (dO for role 0, Q for role 1): one XOR with a constant per read, the rest in immediate offsets
    const int sbb = 2 * (it & 1) * STAGE;
    const int rb = opaque(2 * (rrow + rkey)) + sbb + (role == 0 ? 0 : 2 * QTILE);
    const int tb = opaque(2 * (trow + tkey)) + sbb + (role == 0 ? 2 * QTILE : 0);
    const us* qs = smem + (it & 1) * STAGE;
    const us* dos = qs + QTILE;
    const float* l2s = reinterpret_cast<const float*>(dos + QTILE);
    const float* rss = l2s + 64;
    const int qs0 = qt_c * BQ, h_c = hq_c;
    if (qt_c == qt0) {
      qt_c = qt_end - 1;
      ++hq_c;
    } else {
      --qt_c;
    }
    const bool active = kw0 < sq.skv && (s.mask == 0 || qs0 + BQ - 1 + delta >= kw0) &&
                        (s.wl < 0 || qs0 + delta - s.wl <= kw0 + KW - 1);
    const bool need_mask = (qs0 + BQ > sq.sq) || (kw0 + KW > sq.skv) || (s.mask != 0 && qs0 + delta < kw0 + KW - 1) ||
                           (s.wl >= 0 && qs0 + BQ - 1 + delta - s.wl > kw0);
    v4f sv[2];  // role 0: S then P; role 1: dP then dS
    if (active) {
      // the two 16-row blocks alternate (two independent accumulator chains) and the Q / dO fragments
      // are read RA products ahead: the two waves of a SIMD move in step here and cannot hide each
      // other's LDS latency
      constexpr int NT = 2 * (D / 32), RA = 4;
      v8s rbuf[RA];
#pragma unroll
      for (int i = 0; i < RA; ++i) rbuf[i] = lds_read16_at(smem, (rb ^ (64 * (i >> 1))) + 32 * (i & 1) * D);
      sv[0] = v4f{};
      sv[1] = v4f{};
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const v8s x = rbuf[t % RA];
        __builtin_amdgcn_sched_barrier(0);
        sv[t & 1] = Elem<T>::mma16(Elem<T>::cast(x), Elem<T>::cast(kvf[t >> 1]), sv[t & 1]);
        __builtin_amdgcn_sched_barrier(0);
        if (t + RA < NT) {
          const int u = t + RA;
          rbuf[t % RA] = lds_read16_at(smem, (rb ^ (64 * (u >> 1))) + 32 * (u & 1) * D);
        }
      }
      if (role == 0) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const v4f l2 = *reinterpret_cast<const v4f*>(l2s + 16 * qb + 4 * G);
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[qb][i] = fast_exp2(sv[qb][i] * s.scale_log2 - l2[i]);
        }
        if (need_mask) {  // one branch per tile (a test inside the unrolled loop branches per element)
          const int ql = opaque(qs0 + 4 * G), key = opaque(kw0 + l16);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int q = ql + 16 * qb + i;
              const bool ok = q < sq.sq && key < sq.skv && (s.mask == 0 || key <= q + delta) &&
                              (s.wl < 0 || key >= q + delta - s.wl);
              sv[qb][i] = ok ? sv[qb][i] : 0.f;
            }
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) *reinterpret_cast<v4f*>(pbuf + (qb * 64 + lane) * 4) = sv[qb];
      }
    }
    __syncthreads();
    if (!active) continue;
    if (role == 1) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const v4f pv = *reinterpret_cast<const v4f*>(pbuf + (qb * 64 + lane) * 4);
        const v4f dr = *reinterpret_cast<const v4f*>(rss + 16 * qb + 4 * G);
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[qb][i] = pv[i] * (sv[qb][i] - dr[i]);
      }
    }
    const auto pa = pack8<T>(sv[0][0], sv[0][1], sv[0][2], sv[0][3], sv[1][0], sv[1][1], sv[1][2], sv[1][3]);
    if (STORE_DS && role == 1) {  // rows 16qb + 4G + i of key l16 into the pair's buffer
      const auto pd = __builtin_bit_cast(v8s, pa);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i) dsst[pr * 512 + (16 * qb + 4 * G + i) * 16 + l16] = (us)pd[4 * qb + i];
      ds_qs0 = qs0;
      ds_h = h_c;
      ds_pending = true;
    }
    // dV += P^T dO ; dK += dS^T Q
    if constexpr (STORE_DS) {
      // the fragments of product dt + 1 are read while product dt runs (kept in that order by scheduling
      // barriers: with the dS staging this instance holds more registers, and the compiler would
      // otherwise read each fragment just before its product)
      v8s bt = cat44(lds_read_tr_at(smem, tb), lds_read_tr_at(smem, tb + 32 * D));
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        v8s bn;
        if (dt + 1 < D / 16) {
          const int o1 = tb ^ (32 * (dt + 1));
          bn = cat44(lds_read_tr_at(smem, o1), lds_read_tr_at(smem, o1 + 32 * D));
        }
        __builtin_amdgcn_sched_barrier(0);
        acc[dt] = Elem<T>::mma16(pa, Elem<T>::cast(bt), acc[dt]);
        __builtin_amdgcn_sched_barrier(0);
        if (dt + 1 < D / 16) bt = bn;
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const int o1 = tb ^ (32 * dt);
        const v8s bt = cat44(lds_read_tr_at(smem, o1), lds_read_tr_at(smem, o1 + 32 * D));
        acc[dt] = Elem<T>::mma16(pa, Elem<T>::cast(bt), acc[dt]);
      }
    }
  }

  store_ds();
  T* outp = role == 0 ? (T*)a.dv + seq_off(a.av, packed, b, sq.tk0) + (int64_t)g * a.av.head
                      : (T*)a.dk + seq_off(a.ak, packed, b, sq.tk0) + (int64_t)g * a.ak.head;
  const int64_t orow = role == 0 ? a.av.row : a.ak.row;
  const float oscale = role == 0 ? 1.f : s.scale;
  const int od = role == 0 ? s.dv : s.dqk;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = kw0 + 4 * G + i;
    if (key < sq.skv) {
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        if (!PAD || 16 * dt + l16 < od) outp[(int64_t)key * orow + 16 * dt + l16] = Elem<T>::cvt(acc[dt][i] * oscale);
    }
  }
}

template <int D, typename T, bool PAD>
__global__ void __launch_bounds__(512, 1) attn_bwd_dq_pair_kernel(BwdArgs a) {
  constexpr int NW = 8, QW = 16, BMQ = 4 * QW, BK = 32, CH = D / 8, DH = D / 2;
  constexpr int KTILE = BK * D;
  constexpr int NDMA = KTILE * 2 / 1024 / NW;
  static_assert(NDMA >= 1, "key tile must split over 8 waves");
  __shared__ __attribute__((aligned(1024))) us smem[2 * 2 * KTILE];
  __shared__ __attribute__((aligned(16))) float xch[NW * 2 * 64 * 4];  // P (role 0) / dP (role 1): [kb][lane][4]
  const AttnShape& s = a.s;
  const bool packed = s.cu_q != nullptr;
  if (packed && *s.err) {
    fill_nan_rows<T>(a.dq, a.aq, s.total_q, s.hq, s.dqk);
    return;
  }
  const int lane = threadIdx.x & 63, w = wave_id();
  const int pr = w & 3, role = w >> 2;  // role 0: Q, S, P; role 1: dO, dP. Role r accumulates dQ columns [r*DH, r*DH + DH)
  const int G = lane >> 4, l16 = lane & 15, rr = (lane >> 2) & 3, cc = lane & 3;
  int u, qt, b, h;
  tile_order(s.batch * s.hq, s.n_qtiles, s.mask != 0, u, qt, kOrderQuery);
  q_unit(u, s.batch, s.hkv, s.group, b, h);
  const int g = h / s.group;
  const Seq sq = seq_info(s, b);
  const int q0 = qt * BMQ;
  if (q0 >= sq.sq) return;
  const int delta = s.mask == 2 ? sq.skv - sq.sq : 0;
  const int kv_end = s.mask != 0 ? min(sq.skv, q0 + BMQ + delta) : sq.skv;
  const int n_tiles = kv_end > 0 ? (kv_end + BK - 1) / BK : 0;
  // first key tile inside some row's sliding window (0 without a window)
  const int j0 = s.wl >= 0 ? max(0, q0 + delta - s.wl) / BK : 0;
  const int qw0 = q0 + pr * QW;
  const int64_t rowbase = packed ? sq.tq0 : (int64_t)b * s.sq;

  const us* qdg = role == 0 ? (const us*)a.q + seq_off(a.aq, packed, b, sq.tq0) + (int64_t)h * a.aq.head
                            : (const us*)a.d_o + seq_off(a.ao, packed, b, sq.tq0) + (int64_t)h * a.ao.head;
  const int64_t qdrow = role == 0 ? a.aq.row : a.ao.row;
  const us* kg = (const us*)a.k + seq_off(a.ak, packed, b, sq.tk0) + (int64_t)g * a.ak.head;
  const us* vg = (const us*)a.v + seq_off(a.av, packed, b, sq.tk0) + (int64_t)g * a.av.head;
  v8s qdf[D / 32];
  float l2, dr;
  {
    const int64_t r = min(qw0 + l16, sq.sq - 1);
    const int qdd = role == 0 ? s.dqk : s.dv;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) qdf[kk] = ld_chunk<PAD>(qdg + r * qdrow + 32 * kk + 8 * G, 32 * kk + 8 * G, qdd);
    l2 = a.lse2[(int64_t)h * a.nrows + rowbase + r];
    dr = a.rowsum[(int64_t)h * a.nrows + rowbase + r];
  }
  v4f dq[DH / 16];  // rows qw0 + 4G + i, columns role*DH + 16dt + l16
#pragma unroll
  for (int dt = 0; dt < DH / 16; ++dt) dq[dt] = v4f{};

  const TileDma<D, BK, NDMA, true, PAD> dma(w, lane, a.ak.row, a.av.row, s.dqk, s.dv);
  // issue() is called for tiles j0, j0 + 1, ... in order: running tile pointers
  const int64_t kstep = (int64_t)BK * a.ak.row, vstep = (int64_t)BK * a.av.row;
  const us* k_ld = kg + j0 * kstep;
  const us* v_ld = vg + j0 * vstep;
  auto issue = [&](int tile, int stage) {
    us* ks = smem + stage * 2 * KTILE;
    us* vs = ks + KTILE;
    const int kv0 = tile * BK;
    dma.copy(k_ld, v_ld, sq.skv - 1 - kv0, ks, vs);
    k_ld += kstep;
    v_ld += vstep;
  };

  const int rrow = l16 * D, rkey = (sw_key<D>(l16) ^ G) << 3;
  const int trow = (4 * G + rr) * D + 4 * (cc & 1) + role * DH, tkey = (sw_key<D>(4 * G + rr) ^ (cc >> 1)) << 3;
  float* mine = xch + w * 2 * 64 * 4;
  const float* other = xch + (w ^ 4) * 2 * 64 * 4;

  if constexpr (PAD) {
    zero_lds<2 * 2 * KTILE>(smem);
    __syncthreads();
  }
  if (j0 < n_tiles) issue(j0, j0 & 1);
  for (int j = j0; j < n_tiles; ++j) {
    wait_vmem();
    __syncthreads();
    if (j + 1 < n_tiles) issue(j + 1, (j + 1) & 1);
    // per-stage byte bases (K rows for role 0, V rows for role 1; K transposed for both): one XOR per read
    const int sbb = 4 * (j & 1) * KTILE;
    const int rb = opaque(2 * (rrow + rkey)) + sbb + (role == 0 ? 0 : 2 * KTILE), tb = opaque(2 * (trow + tkey)) + sbb;
    const int kv0 = j * BK;
    const bool active = (s.mask == 0 || kv0 <= qw0 + QW - 1 + delta) && (s.wl < 0 || kv0 + BK - 1 >= qw0 + delta - s.wl);
    const bool need_mask = (kv0 + BK > sq.skv) || (s.mask != 0 && kv0 + BK - 1 > qw0 + delta) ||
                           (s.wl >= 0 && kv0 < qw0 + QW - 1 + delta - s.wl);
    v4f st[2];  // S^T -> P (role 0) or dP^T (role 1): key kv0 + 16kb + 4G + i, query qw0 + l16
    if (active) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        st[kb] = v4f{};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
          st[kb] = Elem<T>::mma16(Elem<T>::cast(lds_read16_at(smem, (rb ^ (64 * kk)) + 32 * kb * D)),
                                  Elem<T>::cast(qdf[kk]), st[kb]);
      }
      if (role == 0) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) st[kb][i] = fast_exp2(st[kb][i] * s.scale_log2 - l2);
        if (need_mask) {  // one branch per tile (a test inside the unrolled loop branches per element)
          const int q = opaque(qw0 + l16), kl = opaque(kv0 + 4 * G);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = kl + 16 * kb + i;
              const bool ok = key < sq.skv && (s.mask == 0 || key <= q + delta) && (s.wl < 0 || key >= q + delta - s.wl);
              st[kb][i] = ok ? st[kb][i] : 0.f;
            }
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) *reinterpret_cast<v4f*>(mine + (kb * 64 + lane) * 4) = st[kb];
    }
    __syncthreads();
    if (!active) continue;
    float ds[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const v4f ot = *reinterpret_cast<const v4f*>(other + (kb * 64 + lane) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = role == 0 ? st[kb][i] : ot[i];
        const float dpv = role == 0 ? ot[i] : st[kb][i];
        ds[kb][i] = p * (dpv - dr);
      }
    }
    const auto dsa = pack8<T>(ds[0][0], ds[0][1], ds[0][2], ds[0][3], ds[1][0], ds[1][1], ds[1][2], ds[1][3]);
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
      const int o1 = tb ^ (32 * dt);
      const v8s kbt = cat44(lds_read_tr_at(smem, o1), lds_read_tr_at(smem, o1 + 32 * D));
      dq[dt] = Elem<T>::mma16(dsa, Elem<T>::cast(kbt), dq[dt]);
    }
  }

  T* dqp = (T*)a.dq + seq_off(a.aq, packed, b, sq.tq0) + (int64_t)h * a.aq.head + role * DH;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = qw0 + 4 * G + i;
    if (q < sq.sq) {
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt)
        if (!PAD || role * DH + 16 * dt + l16 < s.dqk)
          dqp[(int64_t)q * a.aq.row + 16 * dt + l16] = Elem<T>::cvt(dq[dt][i] * s.scale);
    }
  }
}

// ------------------------------------------------------------------------------------------
// dQ of the stored-dS backward (opt-in, ATTN_FLAG_BWD_STORED_DS, D = 512 instances): the dK/dV pass has
// stored dS (rounded to T) for every allowed pair, so dQ = scale * dS K is a plain product over each
// query row's allowed keys, 2*D FLOP per pair instead of the 6*D the recomputing dQ pass executes (its
// S and dP products are 4*D of them, which at D = 512 take longer than reading the stored dS back).
// Workgroup = 4 waves = 64 query rows of one (sequence, q-head), two workgroups per CU: wave w takes
// rows 32*(w%2) .. +31 and dQ columns 256*(w/2) .. +255, as dQ^T += K^T dS^T with 32x32x16 MFMAs (A = K^T
// by transpose reads of the LDS tile, the same reads as the forward's V^T at D = 256; B = this lane's row
// of dS, 8 keys per lane). Key tiles of 32 keys x 512 columns (two 32 x 256 halves, 64 KB for the
// two-stage ring) stream through LDS; dS tiles go through a three-stage LDS ring, copied two steps ahead,
// since they come from HBM rather than from the L2 that serves K. dS is stored in a [q-head][query
// token][ds_ld] array; inside each 32-key block key 16a + 8c + 4h + j sits at position 16c + 8a + 4h + j
// (a 16-byte run per dK/dV wave pair), so the lane (row, half h) of k-step c takes two 8-byte pieces,
// keys 8c + 4h + j and the same + 16, in the order the K^T operand delivers the keys. The dK/dV pass
// writes every allowed pair; a tile that holds a pair outside the mask (or past the key range) replaces
// those dS values by zeros, whatever the workspace holds there.
template <typename T, bool PAD>
__global__ void __launch_bounds__(256, 2) attn_bwd_dq_ds_kernel(BwdArgs a) {
  constexpr int DH = 256, BM = 64, BN = 32;
  constexpr int TILE = BN * DH;             // 16-bit elements of one key half-tile
  constexpr int NDMA = TILE * 2 / 1024 / 4;  // 16-byte copies per wave per half
  static_assert(NDMA >= 1, "half tile must split over 4 waves");
  constexpr int R = 3;            // dS stages: a tile's dS is copied R - 1 steps ahead (HBM latency)
  constexpr int DST = BM * BN;    // 16-bit elements of one dS tile (64 rows x 32 keys, 64-byte rows)
  __shared__ __attribute__((aligned(1024))) us smem[2 * 2 * TILE];
  __shared__ __attribute__((aligned(1024))) us dsm[R * DST];
  const AttnShape& s = a.s;
  const bool packed = s.cu_q != nullptr;
  if (packed && *s.err) {
    fill_nan_rows<T>(a.dq, a.aq, s.total_q, s.hq, s.dqk);
    return;
  }
  const int lane = threadIdx.x & 63, w = wave_id();
  const int hf = w >> 1, wr = w & 1;  // column half and row block of this wave
  const int hh = lane >> 5, lrow = lane & 31;
  int u, qt, b, h;
  tile_order(s.batch * s.hq, a.n_dsqtiles, s.mask != 0, u, qt, kOrderQuery);
  q_unit(u, s.batch, s.hkv, s.group, b, h);
  const int g = h / s.group;
  const Seq sq = seq_info(s, b);
  const int q0 = qt * BM;
  if (q0 >= sq.sq) return;
  const int delta = s.mask == 2 ? sq.skv - sq.sq : 0;
  const int kv_end = s.mask != 0 ? min(sq.skv, q0 + BM + delta) : sq.skv;
  const int n_tiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  // first key tile inside some row's sliding window (0 without a window)
  const int j0 = s.wl >= 0 ? max(0, q0 + delta - s.wl) / BN : 0;
  const int qw0 = q0 + 32 * wr, qi = qw0 + lrow;
  // a wave whose column half lies wholly past D_qk has nothing to compute (it still copies and waits)
  const bool cols = hf * DH < s.dqk;

  const us* kg = (const us*)a.k + seq_off(a.ak, packed, b, sq.tk0) + (int64_t)g * a.ak.head;
  const int64_t rowbase = packed ? sq.tq0 : (int64_t)b * s.sq;
  // dS tiles (the workgroup's 64 rows x 32 keys) are copied into an R-stage LDS ring, one 16-byte chunk
  // per lane: row r = 16w + lane/4 takes physical chunk lane%4, which holds logical chunk (lane%4) ^
  // ((r >> 2) & 3), so that the operand reads below (32 rows, one chunk each) spread over all banks.
  // Rows past the sequence end copy the last row (never stored).
  const us* dsbase = a.ds + ((int64_t)h * a.nrows + rowbase + q0) * a.ds_ld;
  const int crow = 16 * w + (lane >> 2);
  const unsigned coff = (unsigned)((min(crow, sq.sq - 1 - q0) * a.ds_ld + 8 * ((lane & 3) ^ ((crow >> 2) & 3))) * 2);
  auto issue_ds = [&](int tile) { dma16(dsbase, coff + (unsigned)(tile * BN * 2), dsm + (tile % R) * DST + w * 512); };
  // operand of k-step c: row 32wr + lrow, the 8-byte half hh of logical chunks 2c (keys 8c + 4hh + j) and
  // 2c + 1 (the same + 16)
  const int orow = 32 * wr + lrow, oswz = (orow >> 2) & 3;

  const TileDma<DH, BN, NDMA, true, PAD> dma(w, lane, a.ak.row, a.ak.row, min(s.dqk, DH), max(0, s.dqk - DH));
  auto issue = [&](int tile, int stage) {
    us* xs = smem + stage * 2 * TILE;
    const us* kt = kg + (int64_t)tile * BN * a.ak.row;
    dma.copy(kt, kt + DH, sq.skv - 1 - tile * BN, xs, xs + TILE);
  };

  // K^T operand: the forward's V^T transpose reads at D = 256 (k-chunk c: keys 8c + 4hh + 0..3 and the
  // same + 16), from this wave's column half
  const int G = lane >> 4, rr = (lane >> 2) & 3, c4 = lane & 3;
  const int vrow = (4 * hh + rr) * DH + 4 * (c4 & 1);
  int vb[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
    vb[c] = opaque(2 * (vrow + 8 * c * DH + ((sw_key<DH>(8 * c + 4 * hh + rr) ^ (2 * (G & 1) + (c4 >> 1))) << 3))) +
            hf * 2 * TILE;

  v16f acc[DH / 32];
#pragma unroll
  for (int dt = 0; dt < DH / 32; ++dt) acc[dt] = v16f{};
  if constexpr (PAD) {
    zero_lds<2 * 2 * TILE>(smem);
    __syncthreads();
  }
  // copy order: K tile j + 1, then dS tile j + R - 1 (issued after the barrier of step j), so the wait
  // that opens step j + 1 lets the last dS copy stay in flight (vmcnt(1)) whenever one was issued
  bool ds_ahead = false;
  if (j0 < n_tiles) {
    issue(j0, j0 & 1);
#pragma unroll
    for (int t = 0; t < R - 1; ++t)
      if (j0 + t < n_tiles) issue_ds(j0 + t);
    ds_ahead = j0 + 1 < n_tiles;
  }
  for (int j = j0; j < n_tiles; ++j) {
    if (ds_ahead) wait_vmem_but1();
    else wait_vmem();
    __syncthreads();
    if (j + 1 < n_tiles) issue(j + 1, (j + 1) & 1);
    ds_ahead = j + R - 1 < n_tiles;
    if (ds_ahead) issue_ds(j + R - 1);
    const int kv0 = j * BN;
    const bool skip = !cols || (s.mask != 0 && kv0 > qw0 + 31 + delta) ||  // tile fully masked for this wave
                      (s.wl >= 0 && kv0 + BN - 1 < qw0 + delta - s.wl);      // tile before this wave's windows
    if (!skip) {
      const bool need_mask = (kv0 + BN > sq.skv) || (s.mask != 0 && kv0 + BN - 1 > qw0 + delta) ||
                             (s.wl >= 0 && kv0 < qw0 + 31 + delta - s.wl);
      v8s d[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int rb = 2 * ((j % R) * DST + orow * BN) + 8 * hh;
        d[c] = cat44(lds_read8_at(dsm, rb + 16 * ((2 * c) ^ oswz)), lds_read8_at(dsm, rb + 16 * ((2 * c + 1) ^ oswz)));
      }
      if (need_mask) {  // one branch per tile: element e of k-step c is key kv0 + 16(e/4) + 8c + 4hh + e%4
        const int lim = min(sq.skv - 1, s.mask == 0 ? sq.skv : qi + delta) - kv0 - 4 * hh;
        const int lo = s.wl >= 0 ? qi + delta - s.wl - kv0 - 4 * hh : -(1 << 30);
        const bool row_ok = qi < sq.sq;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int off = 16 * (e >> 2) + 8 * c + (e & 3);
            d[c][e] = row_ok && off <= lim && off >= lo ? d[c][e] : (short)0;
          }
      }
      const int sb = (j & 1) * 4 * TILE;  // stage, bytes
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < DH / 32; ++dt) {
          const int o1 = (vb[c] ^ (64 * dt)) + sb;
          const v4s lo = lds_read_tr_at(smem, o1);
          const v4s hi = lds_read_tr_at(smem, o1 + 32 * DH);
          acc[dt] = Elem<T>::mma32(Elem<T>::cast(cat44(lo, hi)), Elem<T>::cast(d[c]), acc[dt]);
        }
    }
  }

  if (cols && qi < sq.sq) {
    T* dqp = (T*)a.dq + seq_off(a.aq, packed, b, sq.tq0) + (int64_t)h * a.aq.head + (int64_t)qi * a.aq.row + hf * DH;
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        typename Elem<T>::op4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = Elem<T>::cvt(acc[dt][4 * q4 + e] * s.scale);
        if (!PAD || hf * DH + 32 * dt + 8 * q4 + 4 * hh < s.dqk)
          *reinterpret_cast<typename Elem<T>::op4*>(dqp + 32 * dt + 8 * q4 + 4 * hh) = v;
      }
  }
}

// ------------------------------------------------------------------------------------------
// Single-pass backward (opt-in, ATTN_FLAG_BWD_ATOMIC_DQ), head dims up to 128. The dK/dV pass also
// forms dQ += scale * dS K for its key tile and adds it with fp32 atomics into a workspace buffer
// (dq_acc, zeroed by the preprocess, scaled and rounded by attn_bwd_dq_convert_kernel), so S and dP are
// computed once per allowed pair instead of twice: 10*D FLOP executed per pair instead of 14*D. The
// order in which key tiles add into a dQ row is not fixed, so dQ is not bitwise deterministic in this
// mode (the pages' own backward has no deterministic mode either: pull request 3527, section Scope).
//
// Workgroup = 8 waves = 128 keys of one (sequence, kv-head); wave pair (p, p + 4) owns 32 keys (two
// 16-key blocks). Wave p (role 0) holds their K and computes S = Q K^T, P = exp2(S*c - lse2), hands P
// (fp32) to its partner through LDS and accumulates dV += P^T dO. Wave p + 4 (role 1) holds V, computes
// dP = dO V^T, takes P, forms dS = P (dP - D), writes dS (rounded to T) into LDS and accumulates
// dK += dS^T Q. Query tiles of 64 rows stream through LDS (Q, dO, lse2, D). The dQ product of a tile
// needs every pair's dS, so it runs one iteration later, after the barrier that starts the next tile:
// wave w takes query rows 32*(w/4) .. +31 of the previous tile and d-columns 16*DBW*(w%4) .. over all
// 128 keys (A = dS by transpose reads of the [key][row] LDS buffer, B = its K columns, held in registers
// with lane = column, 8 keys per lane), then adds the 32 x 16*DBW result into dq_acc with vector
// atomics (one instruction covers 4 rows x 16 consecutive floats). The roles interleave so that one
// wave's matrix products overlap the other's vector work on the same SIMD:
//   role 0:  S -> P -> LDS  | barrier |  dQ(prev) -> dV
//   role 1:  dP -> dQ(prev) | barrier |  dS -> LDS -> dK
// dS is double-buffered in LDS (the dQ product of tile t reads buffer t&1 while dS of tile t+1 goes to
// the other buffer); P is single-buffered (written after one barrier, read before the next).
// dS buffer layout: row = key (128), 64 row elements = 16 chunks of 4 (8 bytes); chunk c of key row r is
// stored at chunk c ^ (((r >> 1) & 3) << 2), so both the dS writes (16 consecutive keys x 4 consecutive
// chunks per instruction) and the transpose reads (the same shape) spread over all banks.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ int ds_chunk_off(int key, int chunk) {  // element offset in one dS buffer
  return key * 64 + ((chunk ^ (((key >> 1) & 3) << 2)) << 2);
}

__device__ __forceinline__ void atomic_add_f32(float* p, float v) {
  __builtin_amdgcn_global_atomic_fadd_f32((__attribute__((address_space(1))) float*)p, v);
}

template <int D, typename T, bool PAD>
__global__ void __launch_bounds__(512, 1) attn_bwd_fused_kernel(BwdArgs a) {
  static_assert(D == 64 || D == 128, "the single-pass backward is built for head dims up to 128");
  constexpr int NW = 8, KW = 32, BKV = 4 * KW, BQ = 64, NDB = D / 16, DBW = NDB / 4;
  constexpr int QTILE = BQ * D;
  constexpr int NDMA = QTILE * 2 / 1024 / NW;
  static_assert(NDMA >= 1, "query tile must split over 8 waves");
  constexpr int STAGE = 2 * QTILE + 2 * 64 * 2;  // Q, dO tiles, then lse2[64] and D[64] as floats
  __shared__ __attribute__((aligned(1024))) us smem[2 * STAGE];
  __shared__ __attribute__((aligned(16))) float pbuf[4 * 8 * 64 * 4];  // P per pair: [pair][m][kb][lane][4]
  __shared__ __attribute__((aligned(16))) us dsbuf[2 * BKV * BQ];      // dS, two buffers of [key][row]
  const AttnShape& s = a.s;
  const bool packed = s.cu_q != nullptr;
  if (packed && *s.err) {
    fill_nan_rows<T>(a.dk, a.ak, s.total_kv, s.hkv, s.dqk);
    fill_nan_rows<T>(a.dv, a.av, s.total_kv, s.hkv, s.dv);
    return;
  }
  const int lane = threadIdx.x & 63, w = wave_id();
  const int pr = w & 3, role = w >> 2;
  const int G = lane >> 4, l16 = lane & 15, rr = (lane >> 2) & 3, cc = lane & 3;
  int u, kt;
  tile_order(s.batch * s.hkv, a.n_kvtiles, false, u, kt, packed ? kOrderTileMajor : kOrderGrouped);
  const int b = u / s.hkv, g = u % s.hkv;
  const Seq sq = seq_info(s, b);
  kt = end_aligned(kt, a.n_kvtiles, sq.skv, BKV);
  if (kt < 0) return;
  const int k0 = kt * BKV;
  if (k0 >= sq.skv) return;
  const int kw0 = k0 + pr * KW;
  const int delta = s.mask == 2 ? sq.skv - sq.sq : 0;
  const int q_lo = s.mask != 0 ? max(0, k0 - delta) : 0;
  const int qt0 = q_lo / BQ;
  const int q_hi = s.wl >= 0 ? k0 + BKV - 1 - delta + s.wl : sq.sq - 1;
  const int nq = q_hi < 0 ? 0 : max(0, min((sq.sq + BQ - 1) / BQ, q_hi / BQ + 1) - qt0);
  const int n_it = nq * s.group;
  const int64_t rowbase = packed ? sq.tq0 : (int64_t)b * s.sq;

  const us* kg = (const us*)a.k + seq_off(a.ak, packed, b, sq.tk0) + (int64_t)g * a.ak.head;
  const us* vg = (const us*)a.v + seq_off(a.av, packed, b, sq.tk0) + (int64_t)g * a.av.head;
  // role 0 keeps K, role 1 keeps V (B operands of S / dP: key kw0 + 16kb + l16, d = 32kk + 8G + t)
  v8s kvf[2][D / 32];
  {
    const us* src = role == 0 ? kg : vg;
    const int64_t srow = role == 0 ? a.ak.row : a.av.row;
    const int sd = role == 0 ? s.dqk : s.dv;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int64_t r = min(kw0 + 16 * kb + l16, sq.skv - 1);
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) kvf[kb][kk] = ld_chunk<PAD>(src + r * srow + 32 * kk + 8 * G, 32 * kk + 8 * G, sd);
    }
  }
  // K columns for the dQ product (B operand, lane = column d, 8 keys per lane): d block db0 + j, key
  // chunk kc: slot t < 4 holds key k0 + 32kc + 4G + t, slot t >= 4 key k0 + 32kc + 16 + 4G + t - 4 (the
  // key order of the transpose reads of dS)
  const int dqh = w >> 2, db0 = (w & 3) * DBW;
  v8s kq[DBW][4];
#pragma unroll
  for (int j = 0; j < DBW; ++j) {
    const int d = 16 * (db0 + j) + l16;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int key = k0 + 32 * kc + (t < 4 ? 4 * G + t : 16 + 4 * G + t - 4);
        const int64_t r = min(key, sq.skv - 1);
        kq[j][kc][t] = (PAD && d >= s.dqk) ? (short)0 : (short)kg[r * a.ak.row + d];
      }
  }
  v4f acc[2][NDB];  // role 0: dV, role 1: dK; key kw0 + 16kb + 4G + i, column 16dt + l16
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int dt = 0; dt < NDB; ++dt) acc[kb][dt] = v4f{};

  const TileDma<D, BQ, NDMA, true, PAD> dma(w, lane, a.aq.row, a.ao.row, s.dqk, s.dv);
  QueryWalk<BQ> ld(a, packed, b, sq, g * s.group, qt0, nq);
  const int qt_end = qt0 + nq;
  auto issue = [&](int stage) {
    const int qs0 = ld.qt * BQ;
    us* qs = smem + stage * STAGE;
    us* dos = qs + QTILE;
    float* l2s = reinterpret_cast<float*>(dos + QTILE);
    float* rss = l2s + 64;
    dma.copy(ld.qp, ld.op, sq.sq - 1 - qs0, qs, dos);
    const int r = min(qs0 + lane, sq.sq - 1);
    if (w == 0) dma4(ld.l2, 4u * r, l2s);
    if (w == 1) dma4(ld.rs, 4u * r, rss);
    ld.next();
  };

  // LDS offsets as in attn_bwd_dkdv_kernel: row reads rows 16m + l16, chunk 4kk + G; transpose reads rows
  // 4G + rr (+16) of a 32-row half, chunk 2dt + cc/2
  const int rrow = l16 * D, rkey = (sw_key<D>(l16) ^ G) << 3;
  const int trow = (4 * G + rr) * D + 4 * (cc & 1), tkey = (sw_key<D>(4 * G + rr) ^ (cc >> 1)) << 3;
  float* pb = pbuf + pr * 8 * 64 * 4;
  const float scale_log2 = s.scale_log2;
  const int64_t hqd = (int64_t)s.hq * s.dqk;

  // dQ(prev) += dS(prev) K over this workgroup's keys: rows 32*dqh + 16*m2 + 4G + i of the query tile at
  // prev_qs0 of q-head prev_h, columns 16*(db0 + j) + l16
  auto dq_step = [&](int buf, int prev_qs0, int prev_h) {
    const us* dsb = dsbuf + buf * BKV * BQ;
    v4f dqa[2][DBW];
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
      for (int j = 0; j < DBW; ++j) dqa[m2][j] = v4f{};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2) {
        const int row = 32 * kc + 4 * G + rr, chunk = 8 * dqh + 4 * m2 + cc;
        const int o = ds_chunk_off(row, chunk);  // row + 16 has the same swizzle
        const v8s dsa = cat44(lds_read_tr(dsb, o), lds_read_tr(dsb, o + 16 * 64));
#pragma unroll
        for (int j = 0; j < DBW; ++j) dqa[m2][j] = Elem<T>::mma16(Elem<T>::cast(dsa), Elem<T>::cast(kq[j][kc]), dqa[m2][j]);
      }
    float* base = a.dq_acc + (rowbase + prev_qs0) * hqd + (int64_t)prev_h * s.dqk;
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = 32 * dqh + 16 * m2 + 4 * G + i;
        if (prev_qs0 + q < sq.sq) {
#pragma unroll
          for (int j = 0; j < DBW; ++j) {
            const int d = 16 * (db0 + j) + l16;
            if (!PAD || d < s.dqk) atomic_add_f32(base + (int64_t)q * hqd + d, dqa[m2][j][i]);
          }
        }
      }
  };

  int qt_c = qt0, h_c = g * s.group;  // query tile and q-head of the iteration
  int prev_qs0 = 0, prev_h = 0;
  if constexpr (PAD) {
    zero_lds<2 * STAGE>(smem);
    __syncthreads();
  }
  if (n_it > 0) issue(0);
  for (int it = 0; it < n_it; ++it) {
    wait_vmem();
    __syncthreads();  // stage it is in LDS; dS of the previous tile is complete; P buffer is free
    if (it + 1 < n_it) issue((it + 1) & 1);
    const int sb = (it & 1) * STAGE;
    const int qs0 = qt_c * BQ, hcur = h_c;
    if (++qt_c == qt_end) {
      qt_c = qt0;
      ++h_c;
    }
    const bool active = kw0 < sq.skv && (s.mask == 0 || qs0 + BQ - 1 + delta >= kw0) &&
                        (s.wl < 0 || qs0 + delta - s.wl <= kw0 + KW - 1);
    const bool need_mask = (qs0 + BQ > sq.sq) || (kw0 + KW > sq.skv) || (s.mask != 0 && qs0 + delta < kw0 + KW - 1) ||
                           (s.wl >= 0 && qs0 + BQ - 1 + delta - s.wl > kw0);
    const float* l2s = reinterpret_cast<const float*>(smem + sb + 2 * QTILE);
    const float* rss = l2s + 64;
    const int rb = opaque(2 * (rrow + rkey)) + 2 * sb;
    v4f sv[4][2];  // role 0: S then P; role 1: dP then dS. Row 16m + 4G + i, key kw0 + 16kb + l16
    // ---- phase A: S (role 0) or dP (role 1), and for role 1 the dQ product of the previous tile
    if (active) {
      const int src = rb + (role == 0 ? 0 : 2 * QTILE);
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sv[m][kb] = v4f{};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const v8s x = lds_read16_at(smem, (src ^ (64 * kk)) + 32 * m * D);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            sv[m][kb] = Elem<T>::mma16(Elem<T>::cast(x), Elem<T>::cast(kvf[kb][kk]), sv[m][kb]);
        }
      if (role == 0) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const v4f l2 = *reinterpret_cast<const v4f*>(l2s + 16 * m + 4 * G);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[m][kb][i] = fast_exp2(sv[m][kb][i] * scale_log2 - l2[i]);
        }
        if (need_mask) {  // one branch per tile
          const int ql = opaque(qs0 + 4 * G), kl = opaque(kw0 + l16);
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int q = ql + 16 * m + i, key = kl + 16 * kb;
                const bool ok = q < sq.sq && key < sq.skv && (s.mask == 0 || key <= q + delta) &&
                                (s.wl < 0 || key >= q + delta - s.wl);
                sv[m][kb][i] = ok ? sv[m][kb][i] : 0.f;
              }
        }
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) *reinterpret_cast<v4f*>(pb + ((m * 2 + kb) * 64 + lane) * 4) = sv[m][kb];
      }
    }
    if (role == 1 && it > 0) dq_step((it - 1) & 1, prev_qs0, prev_h);
    __syncthreads();  // P of this tile is in LDS
    // ---- phase B: dQ product of the previous tile and dV (role 0), or dS and dK (role 1)
    if (role == 0 && it > 0) dq_step((it - 1) & 1, prev_qs0, prev_h);
    us* dsw = dsbuf + (it & 1) * BKV * BQ;
    if (role == 1) {
      if (active) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const v4f dr = *reinterpret_cast<const v4f*>(rss + 16 * m + 4 * G);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const v4f pv = *reinterpret_cast<const v4f*>(pb + ((m * 2 + kb) * 64 + lane) * 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[m][kb][i] = pv[i] * (sv[m][kb][i] - dr[i]);
          }
        }
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) sv[m][kb] = v4f{};
      }
      // dS rounded to T, [key][row]: key pr*32 + 16kb + l16, rows 16m + 4G .. +3 (one 8-byte chunk)
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          typename Elem<T>::op4 d4;
#pragma unroll
          for (int i = 0; i < 4; ++i) d4[i] = Elem<T>::cvt(sv[m][kb][i]);
          *reinterpret_cast<typename Elem<T>::op4*>(dsw + ds_chunk_off(pr * KW + 16 * kb + l16, 4 * m + G)) = d4;
        }
    }
    if (active) {
      // dV += P^T dO (role 0) / dK += dS^T Q (role 1), one 32-row half at a time: A = the accumulators of
      // rows 32h .. +31 (k slots: 4G + t, then 16 + 4G + t), B = dO^T / Q^T by transpose reads
      const int bsrc = (role == 0 ? 2 * QTILE : 0) + 2 * sb;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        typename Elem<T>::op8 pa[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          pa[kb] = pack8<T>(sv[2 * h][kb][0], sv[2 * h][kb][1], sv[2 * h][kb][2], sv[2 * h][kb][3], sv[2 * h + 1][kb][0],
                            sv[2 * h + 1][kb][1], sv[2 * h + 1][kb][2], sv[2 * h + 1][kb][3]);
        const int tb = opaque(2 * (trow + tkey)) + bsrc + 64 * D * h;
#pragma unroll
        for (int dt = 0; dt < NDB; ++dt) {
          const int o1 = tb ^ (32 * dt);
          const v8s bt = cat44(lds_read_tr_at(smem, o1), lds_read_tr_at(smem, o1 + 32 * D));
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) acc[kb][dt] = Elem<T>::mma16(pa[kb], Elem<T>::cast(bt), acc[kb][dt]);
        }
      }
    }
    prev_qs0 = qs0;
    prev_h = hcur;
  }
  if (n_it > 0) {
    __syncthreads();  // dS of the last tile is complete
    dq_step((n_it - 1) & 1, prev_qs0, prev_h);
  }

  T* outp = role == 0 ? (T*)a.dv + seq_off(a.av, packed, b, sq.tk0) + (int64_t)g * a.av.head
                      : (T*)a.dk + seq_off(a.ak, packed, b, sq.tk0) + (int64_t)g * a.ak.head;
  const int64_t orow = role == 0 ? a.av.row : a.ak.row;
  const float oscale = role == 0 ? 1.f : s.scale;
  const int od = role == 0 ? s.dv : s.dqk;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kw0 + 16 * kb + 4 * G + i;
      if (key < sq.skv) {
#pragma unroll
        for (int dt = 0; dt < NDB; ++dt)
          if (!PAD || 16 * dt + l16 < od) outp[(int64_t)key * orow + 16 * dt + l16] = Elem<T>::cvt(acc[kb][dt][i] * oscale);
      }
    }
}

// Preprocess of the single-pass backward: attn_bwd_pre_kernel's D and LSE * log2(e), plus the zeroing of
// this (row, head)'s D_qk floats of dq_acc ([rows][Hq][D_qk], fp32). HBM-bound.
template <int D, typename T>
__global__ void __launch_bounds__(256) attn_bwd_pre_zero_kernel(BwdArgs a) {
  const AttnShape& s = a.s;
  const bool packed = s.cu_q != nullptr;
  if (packed && *s.err) return;
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int64_t total = a.nrows * s.hq;
  const int64_t R = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.f;
  int64_t t = 0, lofs = 0;
  int h = 0;
  if (R < total) {
    t = R / s.hq;
    h = (int)(R % s.hq);
    int64_t oofs;
    if (packed) {
      oofs = t * a.ao.row + (int64_t)h * a.ao.head;
      lofs = t * a.alse.row + (int64_t)h * a.alse.head;
    } else {
      const int64_t bb = t / s.sq, si = t % s.sq;
      oofs = bb * a.ao.batch + si * a.ao.row + (int64_t)h * a.ao.head;
      lofs = bb * a.alse.batch + si * a.alse.row + (int64_t)h * a.alse.head;
    }
    if (8 * c < s.dv) {
      const v8s o8 = *reinterpret_cast<const v8s*>((const us*)a.o + oofs + 8 * c);
      const v8s d8 = *reinterpret_cast<const v8s*>((const us*)a.d_o + oofs + 8 * c);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += to_f32<T>(o8[i]) * to_f32<T>(d8[i]);
    }
    if (8 * c < s.dqk) {  // R = t * hq + h: the dq_acc row of (t, h) starts at R * dqk
      v4f* z = reinterpret_cast<v4f*>(a.dq_acc + R * s.dqk + 8 * c);
      z[0] = v4f{};
      z[1] = v4f{};
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (R < total && c == 0) {
    a.rowsum[(int64_t)h * a.nrows + t] = acc;
    const float l = a.lse[lofs];
    a.lse2[(int64_t)h * a.nrows + t] = l == -__builtin_inff() ? __builtin_inff() : l * kLog2e;
  }
}

// Last step of the single-pass backward: dQ = T(scale * dq_acc) in Q's layout. HBM-bound: reads 4 * D_qk,
// writes 2 * D_qk bytes per (row, head). Rows no key reached keep the zeros of the preprocess.
template <int D, typename T>
__global__ void __launch_bounds__(256) attn_bwd_dq_convert_kernel(BwdArgs a) {
  const AttnShape& s = a.s;
  const bool packed = s.cu_q != nullptr;
  if (packed && *s.err) {
    fill_nan_rows<T>(a.dq, a.aq, s.total_q, s.hq, s.dqk);
    return;
  }
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int64_t R = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  if (R >= a.nrows * s.hq || 8 * c >= s.dqk) return;  // no barrier in this kernel
  const int64_t t = R / s.hq;
  const int h = (int)(R % s.hq);
  int64_t qofs;
  if (packed) {
    qofs = t * a.aq.row + (int64_t)h * a.aq.head;
  } else {
    const int64_t bb = t / s.sq, si = t % s.sq;
    qofs = bb * a.aq.batch + si * a.aq.row + (int64_t)h * a.aq.head;
  }
  const v4f* src = reinterpret_cast<const v4f*>(a.dq_acc + R * s.dqk + 8 * c);
  const v4f x0 = src[0], x1 = src[1];
  typename Elem<T>::op8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = Elem<T>::cvt(x0[i] * s.scale);
    r[4 + i] = Elem<T>::cvt(x1[i] * s.scale);
  }
  *reinterpret_cast<typename Elem<T>::op8*>((T*)a.dq + qofs + 8 * c) = r;
}

// ------------------------------------------------------------------------------------------
// Launchers
// ------------------------------------------------------------------------------------------
constexpr int kFwdBM = 128;
// ------------------------------------------------------------------------------------------
// Merge of per-chunk results over disjoint key sets (the p2p ring step of pull request 3527, section
// Scope): LSE = log sum_k exp(LSE_k), O = sum_k exp(LSE_k - LSE) O_k, empty parts (LSE_k = -inf)
// neutral. HBM-bound: D/8 lanes per (row, head), 16 bytes per lane and part. Every lane reads all of
// its inputs before writing, so o / lse may be one of the parts (in-place accumulation).
// ------------------------------------------------------------------------------------------
template <int D, typename T>
__global__ void __launch_bounds__(256) attn_merge_kernel(MergeArgs a) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int64_t R = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  if (R >= a.nrows) return;  // no barrier in this kernel
  // rows are (token, head): neighbouring rows are neighbouring 2D-byte pieces of O (contiguous for the
  // usual layouts), which matters more than the 4-byte Stats (two parts on the dense D=128 query side,
  // same run: 38.5 us against 44.5 us for a (batch, head, position) order with contiguous Stats)
  const int64_t t = R / a.hq;
  const int h = (int)(R % a.hq);
  int64_t oofs, lofs;
  if (a.packed) {
    oofs = t * a.ao.row + (int64_t)h * a.ao.head;
    lofs = t * a.alse.row + (int64_t)h * a.alse.head;
  } else {
    const int64_t b = t / a.sq, si = t % a.sq;
    oofs = b * a.ao.batch + si * a.ao.row + (int64_t)h * a.ao.head;
    lofs = b * a.alse.batch + si * a.alse.row + (int64_t)h * a.alse.head;
  }
  float l[kMergeMaxParts];
  float m = -__builtin_inff();
#pragma unroll
  for (int k = 0; k < kMergeMaxParts; ++k) {
    l[k] = k < a.n_parts ? a.lse_parts[k][lofs] : -__builtin_inff();
    m = fmaxf(m, l[k]);
  }
  const bool col_live = 8 * c < a.dv;  // lanes past a narrower head's width read and write nothing
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (m != -__builtin_inff()) {
#pragma unroll
    for (int k = 0; k < kMergeMaxParts; ++k) {
      if (k < a.n_parts) {
        const float wk = fast_exp2((l[k] - m) * kLog2e);  // 0 for an empty part
        tot += wk;
        if (col_live) {
          const v8s x = *reinterpret_cast<const v8s*>((const us*)a.o_parts[k] + oofs + 8 * c);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wk, to_f32<T>(x[i]), acc[i]);
        }
      }
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  typename Elem<T>::op8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = Elem<T>::cvt(acc[i] * inv);
  if (col_live) *reinterpret_cast<typename Elem<T>::op8*>((T*)a.o + oofs + 8 * c) = r;
  if (c == 0) a.lse[lofs] = tot > 0.f ? m + __builtin_log2f(tot) * kLn2 : -__builtin_inff();
}

template <int D> constexpr int fwd_bn() { return D <= 128 ? 64 : 32; }
template <int D> constexpr int dkdv_kb() { return D <= 128 ? 2 : 1; }
template <int D> constexpr int dq_qb() { return D <= 128 ? 2 : 1; }
template <int D> constexpr int bwd_minw() { return D <= 256 ? 2 : 1; }

int instance_head_dim(int dqk, int dv) {
  const int m = dqk > dv ? dqk : dv;
  return m <= 64 ? 64 : m <= 128 ? 128 : m <= 256 ? 256 : m <= 512 ? 512 : 0;
}

int fwd_query_tile(int) { return kFwdBM; }
int bwd_key_tile(int head_dim) { return 64 * (head_dim <= 128 ? 2 : 1); }  // 64 for the D = 512 pair kernel too;
                                                                             // 128 for the single-pass kernel
int bwd_query_tile(int head_dim) { return 64 * (head_dim <= 128 ? 2 : 1); }

int launch_validate_cu(const AttnShape& s, void* stream) {
  hipLaunchKernelGGL(validate_cu_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, s);
  return (int)hipGetLastError();
}

template <int D> constexpr int fwd_minw() { return D <= 256 ? 2 : 1; }

template <int D, typename T, bool PAD>
static int fwd_t(const FwdArgs& a, hipStream_t st) {
  const dim3 grid(a.s.batch * a.s.hq * a.s.n_qtiles);
  // D = 256: 32 rows of Q (64 registers) and their O accumulator (128) fit one wave at two waves per SIMD with
  // 32-key tiles (253 registers, no spills); measured 35 % faster than the split kernel's wave pairs
  // (cp_share_d256 1.45 -> 0.94 ms, window_d256 0.295 -> 0.191 ms, asym_d192 1.43 -> 0.93 ms)
  if constexpr (D <= 256) {
    if (a.exp_split)
      hipLaunchKernelGGL((attn_fwd_kernel<D, fwd_bn<D>(), fwd_minw<D>(), T, PAD, true>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((attn_fwd_kernel<D, fwd_bn<D>(), fwd_minw<D>(), T, PAD>), grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((attn_fwd_split_kernel<D, T, PAD>), grid, dim3(512), 0, st, a);
  }
  return (int)hipGetLastError();
}

// Single-pass backward (a.atomic_dq; D <= 128, checked by the host): preprocess with zeroing, the fused
// kernel, the conversion, each launched when its bit is set.
template <int D, typename T, bool PAD>
static int bwd_atomic_t(const BwdArgs& a, int passes, hipStream_t st) {
  if constexpr (D > 128) {
    return (int)hipErrorInvalidValue;
  } else {
    constexpr int RPB = 256 / (D / 8);
    const int64_t rows = a.nrows * a.s.hq;
    const dim3 row_grid((unsigned)((rows + RPB - 1) / RPB));
    hipError_t e = hipSuccess;
    if ((passes & kPassPre) && rows > 0) {
      hipLaunchKernelGGL((attn_bwd_pre_zero_kernel<D, T>), row_grid, dim3(256), 0, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return (int)e;
    }
    if ((passes & kPassDkdv) && a.n_kvtiles > 0) {
      const dim3 grid(a.s.batch * a.s.hkv * a.n_kvtiles);
      hipLaunchKernelGGL((attn_bwd_fused_kernel<D, T, PAD>), grid, dim3(512), 0, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return (int)e;
    }
    if ((passes & kPassDq) && rows > 0) {
      hipLaunchKernelGGL((attn_bwd_dq_convert_kernel<D, T>), row_grid, dim3(256), 0, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return (int)e;
    }
    return (int)e;
  }
}

template <int D, typename T, bool PAD>
static int bwd_t(const BwdArgs& a, int passes, hipStream_t st) {
  if (a.atomic_dq) return bwd_atomic_t<D, T, PAD>(a, passes, st);
  // Launches with an empty grid are skipped (e.g. no query rows: only dK = dV = 0 remain to write).
  // With D <= 256, a request for both the preprocess and the dQ pass (attn_bwd, or the fused pass on
  // its own) runs the dQ pass with the preprocess folded in, before the dK/dV pass that reads its
  // D and LSE * log2(e): two launches instead of three. D = 512 keeps the three passes.
  constexpr int RPB = 256 / (D / 8);
  const int64_t rows = a.nrows * a.s.hq;
  hipError_t e = hipSuccess;
  if (passes & kPassDqPre) passes |= kPassPre | kPassDq;
  const bool fuse = D <= 256 && (passes & kPassPre) && (passes & kPassDq);
  auto run_dq = [&](bool pre) {
    if (a.s.n_qtiles == 0) return;
    const dim3 grid(a.s.batch * a.s.hq * a.s.n_qtiles);
    if constexpr (D <= 256) {
      if (pre)
        hipLaunchKernelGGL((attn_bwd_dq_kernel<D, dq_qb<D>(), bwd_minw<D>(), T, PAD, true>), grid, dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((attn_bwd_dq_kernel<D, dq_qb<D>(), bwd_minw<D>(), T, PAD>), grid, dim3(256), 0, st, a);
    } else if (a.ds != nullptr) {
      if (a.n_dsqtiles == 0) return;
      hipLaunchKernelGGL((attn_bwd_dq_ds_kernel<T, PAD>), dim3(a.s.batch * a.s.hq * a.n_dsqtiles), dim3(256), 0, st, a);
    } else {
      hipLaunchKernelGGL((attn_bwd_dq_pair_kernel<D, T, PAD>), grid, dim3(512), 0, st, a);
    }
    e = hipGetLastError();
  };
  if (fuse) {
    run_dq(true);
    if (e != hipSuccess) return (int)e;
  } else if ((passes & kPassPre) && rows > 0) {
    hipLaunchKernelGGL((attn_bwd_pre_kernel<D, T>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  }
  if ((passes & kPassDkdv) && a.n_kvtiles > 0) {
    const dim3 grid(a.s.batch * a.s.hkv * a.n_kvtiles);
    if constexpr (D <= 256) {
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, dkdv_kb<D>(), bwd_minw<D>(), T, PAD>), grid, dim3(256), 0, st, a);
    } else if (a.ds != nullptr) {
      hipLaunchKernelGGL((attn_bwd_dkdv_pair_kernel<D, T, PAD, true>), grid, dim3(512), 0, st, a);
    } else {
      hipLaunchKernelGGL((attn_bwd_dkdv_pair_kernel<D, T, PAD>), grid, dim3(512), 0, st, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  }
  if (!fuse && (passes & kPassDq)) run_dq(false);
  return (int)e;
}

// PAD instances serve heads narrower than D (either head dim below it); full-width heads keep the
// unpadded code.
template <int D>
static int fwd_d(bool bf, const FwdArgs& a, hipStream_t st) {
  const bool pad = a.s.dqk != D || a.s.dv != D;
  if (bf) return pad ? fwd_t<D, __bf16, true>(a, st) : fwd_t<D, __bf16, false>(a, st);
  return pad ? fwd_t<D, _Float16, true>(a, st) : fwd_t<D, _Float16, false>(a, st);
}

int launch_fwd(int dtype, int head_dim, const FwdArgs& a, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const bool bf = dtype == 0;
  switch (head_dim) {
    case 64: return fwd_d<64>(bf, a, st);
    case 128: return fwd_d<128>(bf, a, st);
    case 256: return fwd_d<256>(bf, a, st);
    case 512: return fwd_d<512>(bf, a, st);
  }
  return (int)hipErrorInvalidValue;
}

int launch_merge(int dtype, int head_dim, const MergeArgs& a, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const bool bf = dtype == 0;
  const int rpb = 256 / (head_dim / 8);
  const dim3 grid((unsigned)((a.nrows + rpb - 1) / rpb));
  switch (head_dim) {
#define SDPA_MERGE_CASE(DD)                                                                          \
  case DD:                                                                                          \
    if (bf) hipLaunchKernelGGL((attn_merge_kernel<DD, __bf16>), grid, dim3(256), 0, st, a);          \
    else hipLaunchKernelGGL((attn_merge_kernel<DD, _Float16>), grid, dim3(256), 0, st, a);           \
    return (int)hipGetLastError();
    SDPA_MERGE_CASE(64)
    SDPA_MERGE_CASE(128)
    SDPA_MERGE_CASE(256)
    SDPA_MERGE_CASE(512)
#undef SDPA_MERGE_CASE
  }
  return (int)hipErrorInvalidValue;
}

template <int D>
static int bwd_d(bool bf, const BwdArgs& a, int passes, hipStream_t st) {
  const bool pad = a.s.dqk != D || a.s.dv != D;
  if (bf) return pad ? bwd_t<D, __bf16, true>(a, passes, st) : bwd_t<D, __bf16, false>(a, passes, st);
  return pad ? bwd_t<D, _Float16, true>(a, passes, st) : bwd_t<D, _Float16, false>(a, passes, st);
}

int launch_bwd(int dtype, int head_dim, const BwdArgs& a, int passes, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const bool bf = dtype == 0;
  switch (head_dim) {
    case 64: return bwd_d<64>(bf, a, passes, st);
    case 128: return bwd_d<128>(bf, a, passes, st);
    case 256: return bwd_d<256>(bf, a, passes, st);
    case 512: return bwd_d<512>(bf, a, passes, st);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace sdpa
