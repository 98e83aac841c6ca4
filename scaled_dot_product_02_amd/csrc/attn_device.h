// attn_device.h - gfx950 (CDNA4) device primitives used by the attention kernels.
//
// MFMA lane layouts (wave64), checked on the hardware against a host matmul:
//   v_mfma_f32_32x32x16_{bf16,f16}: A[row][k]: lane l holds row l%32, k = 8*(l/32) + t (t = 0..7);
//     B[k][col]: lane l holds col l%32, k = 8*(l/32) + t; C[row][col] (16 fp32 per lane):
//     lane l holds col l%32, rows 8*(j/4) + 4*(l/32) + (j%4) for register j = 0..15.
//   v_mfma_f32_16x16x32_{bf16,f16}: A: lane l holds row l%16, k = 8*(l/16) + t;
//     B: lane l holds col l%16, k = 8*(l/16) + t; C (4 fp32 per lane): col l%16, rows 4*(l/16) + i.
// Because the contraction sums over k, any bijection between k slots and the true reduction index
// may be used as long as A and B agree on it; the kernels use this to feed an accumulator layout
// directly back in as the next product's operand.
//
// ds_read_b64_tr_b16 (LDS transpose read), as measured: within each group of 16 lanes, output
// lane i, element r is element (i % 4) of the 8 bytes addressed by lane 4*r + i/4. So if lanes
// 4r..4r+3 address row r of a 4 x 16 block of 16-bit values (4 consecutive elements each), lane i
// receives column i of that block: one transposed operand fragment per instruction.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"

namespace sdpa {

typedef short v8s __attribute__((__vector_size__(8 * sizeof(short))));
typedef short v4s __attribute__((__vector_size__(4 * sizeof(short))));
typedef __bf16 v8bf __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 v8h __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef __bf16 v4bf __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef _Float16 v4h __attribute__((__vector_size__(4 * sizeof(_Float16))));
typedef float v16f __attribute__((__vector_size__(16 * sizeof(float))));
typedef float v4f __attribute__((__vector_size__(4 * sizeof(float))));
typedef unsigned v4u __attribute__((__vector_size__(4 * sizeof(unsigned))));
typedef unsigned v2u __attribute__((__vector_size__(2 * sizeof(unsigned))));

typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element-type traits: 8-element MFMA operand, conversion from fp32 and the two MFMA shapes.
template <typename T> struct Elem;

template <> struct Elem<__bf16> {
  typedef v8bf op8;
  typedef v4bf op4;
  static __device__ __forceinline__ op8 cast(v8s x) { return __builtin_bit_cast(op8, x); }
  static __device__ __forceinline__ __bf16 cvt(float f) { return (__bf16)f; }
  static __device__ __forceinline__ v16f mma32(op8 a, op8 b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ v4f mma16(op8 a, op8 b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Elem<_Float16> {
  typedef v8h op8;
  typedef v4h op4;
  static __device__ __forceinline__ op8 cast(v8s x) { return __builtin_bit_cast(op8, x); }
  static __device__ __forceinline__ _Float16 cvt(float f) { return (_Float16)f; }
  static __device__ __forceinline__ v16f mma32(op8 a, op8 b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ v4f mma16(op8 a, op8 b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// 8 fp32 values -> one 8-element operand (round to nearest even).
template <typename T>
__device__ __forceinline__ typename Elem<T>::op8 pack8(float f0, float f1, float f2, float f3, float f4, float f5,
                                                       float f6, float f7) {
  typename Elem<T>::op8 r;
  r[0] = Elem<T>::cvt(f0); r[1] = Elem<T>::cvt(f1); r[2] = Elem<T>::cvt(f2); r[3] = Elem<T>::cvt(f3);
  r[4] = Elem<T>::cvt(f4); r[5] = Elem<T>::cvt(f5); r[6] = Elem<T>::cvt(f6); r[7] = Elem<T>::cvt(f7);
  return r;
}

// 16 bytes from LDS (element offset, 16-bit elements).
__device__ __forceinline__ v8s lds_read16(const unsigned short* base, int elem) {
  return *reinterpret_cast<const v8s*>(base + elem);
}

// Transposed 8-byte LDS read (see the header comment for the lane mapping).
__device__ __forceinline__ v4s lds_read_tr(const unsigned short* base, int elem) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(base + elem));
}
// Same two reads at a byte offset from base (lets a caller keep its offsets in bytes).
__device__ __forceinline__ v8s lds_read16_at(const void* base, int byte_off) {
  return *reinterpret_cast<const v8s*>(static_cast<const char*>(base) + byte_off);
}
__device__ __forceinline__ v4s lds_read8_at(const void* base, int byte_off) {
  return *reinterpret_cast<const v4s*>(static_cast<const char*>(base) + byte_off);
}
__device__ __forceinline__ v4s lds_read_tr_at(const void* base, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(static_cast<const char*>(base) + byte_off));
}

__device__ __forceinline__ v8s cat44(v4s a, v4s b) {
  v8s r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// Direct HBM -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4, scalar-base form): lane l
// reads base + off (base wave-uniform, off a 32-bit per-lane byte offset) and its 16 bytes land at
// lds_wave_base + 16*l (wave-uniform, passed in M0).
//
// Issued through inline asm on purpose. The compiler's wait-count pass models this instruction as
// a flat access to both global memory and LDS; while one is outstanding it turns every later LDS
// dependency into a full drain (s_waitcnt lgkmcnt(0), and vmcnt(0) before transpose reads), so the
// K-fragment reads of a tile could not run ahead of their MFMAs and each tile's P*V waited for the
// next tile's copy to land. The kernels order the copies themselves: every wave waits for its own
// copies (wait_vmem) before the barrier that hands a stage to the readers, and a stage is
// overwritten only after the barrier that ends its reads. vmcnt completes in issue order, so the
// compiler's own waits for other loads stay correct (copies it does not know about only make them
// more conservative).
__device__ __forceinline__ void dma16(const void* base, unsigned off, void* lds_wave_base) {
  const unsigned m0 = (unsigned)(uintptr_t)(lds_void*)lds_wave_base;
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(m0));
}
// Same with 4 bytes per lane (lane l's dword lands at lds_wave_base + 4*l).
__device__ __forceinline__ void dma4(const void* base, unsigned off, void* lds_wave_base) {
  const unsigned m0 = (unsigned)(uintptr_t)(lds_void*)lds_wave_base;
  asm volatile("global_load_lds_dword %0, %1" ::"v"(off), "s"(base), "{m0}"(m0));
}

// Wait until this wave's outstanding vector-memory loads (including LDS DMA) have landed: s_waitcnt
// with vmcnt = 0 and expcnt / lgkmcnt at their maxima (no wait on those). A real s_waitcnt, not inline
// asm, so that the compiler's wait-count tracking sees it (loads issued before it need no further
// wait after it).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// The same but leaving this wave's most recent vector-memory load in flight (vmcnt = 1; loads complete
// in issue order).
__device__ __forceinline__ void wait_vmem_but1() { __builtin_amdgcn_s_waitcnt(0x0F71); }

// LDS tile rows are stored with their 16-byte chunks permuted: physical chunk = logical chunk ^
// sw_key(row), the key a function of the row's low 4 bits (the readers see rows 16m + r).
//
// gfx950 LDS as measured with SQ_LDS_BANK_CONFLICT on single-wave probes (pairs of active lanes, then
// whole-wave patterns): 64 banks of 4 bytes, bank = (byte address / 4) % 64 with no hashing of higher
// bits. ds_read_b128 is served in 4 passes of 16 lanes: lane bit 5 and the parity of lane bits 2..4
// pick the pass (lanes 0-3, 12-15, 20-23, 24-27 form one), so two lanes conflict when they share that
// pass and a bank; every extra address on a bank costs one cycle. 8-byte reads, the transpose read
// ds_read_b64_tr_b16 included, are served in 2 passes of 32 consecutive lanes.
//
// The patterns the kernels read with (c = the read's logical chunk, constant over the wave):
//   16x16x32 operand rows: lane (G = lane/16, r = lane%16) reads row r, chunk 4c' + G. In one pass
//     lane bit 4 (G's low bit) is the parity of r's bits 2,3, so the 16 chunk positions are
//     key(r) ^ parity(r2, r3) (in bit 0) ^ const: that map has to be a permutation of r.
//   32x32x16 operand rows: lane reads row lane%32, chunk 2c' + lane/32: any permutation key works.
//   transpose reads: lanes 0-31 read rows 0-7 at chunks 2c', 2c'+1 (both 8-byte halves), lanes 32-63
//     rows 8-15: key(r) / 2 has to take 8 distinct values on rows 0-7 and on rows 8-15.
// D >= 128 (16+ chunks per row, rows a multiple of 256 bytes): key bits (3 2 1 0) = (r1, r0, r2^r3, r3)
// meets all three (the earlier key (r1, r0, r2, r3) failed the first: every 16x16x32 row read took two
// cycles per pass, 4 extra cycles per instruction, and the backward passes' LDS command queue filled).
// D = 64 (8 chunks per row, two rows per 256-byte bank row: chunk position 8(r & 1) + (c ^ key(r))):
// key (r1, r2^r3, r2) keeps all four patterns free of conflicts; the row-XOR key r & 7 left the
// forward's operand-row reads and transpose reads with 4 and 2 extra cycles per instruction.
template <int D>
__device__ __forceinline__ int sw_key(int r) {
  if constexpr (D >= 128) return ((r & 3) << 2) | ((((r >> 2) ^ (r >> 3)) & 1) << 1) | ((r >> 3) & 1);
  else return (((r >> 1) & 1) << 2) | ((((r >> 2) ^ (r >> 3)) & 1) << 1) | ((r >> 2) & 1);
}
// Element offset of logical chunk c of row r.
template <int D>
__device__ __forceinline__ int swz(int r, int c) { return r * D + ((c ^ sw_key<D>(r)) << 3); }
// The XOR of a read's compile-time chunk with the lane's key is left inside the loop: an opaque
// per-iteration copy of the key stops the compiler from hoisting one address register per unrolled
// read out of the loop (which spills at 256 registers); each read then costs one XOR-add.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^x on the VALU (the forward's optional exp split): Cody-Waite reduction specialised to base 2, which is
// exact in fp32 (n = rint(x), f = x - n in [-1/2, 1/2]), a degree-5 polynomial for 2^f, then v_ldexp_f32.
// The coefficients are the float32-rounded least-squares fit of the relative error made by
// scaled_dot_product_02_amd/exp2_poly.py (max relative error 2.0e-7 for x in [-30, 8]; a CPU test holds
// these literals to that fit). x is clamped at -127: 2^-127 is far below anything a row sum can see.
__device__ __forceinline__ float exp2_poly(float x) {
  x = fmaxf(x, -127.f);
  const float n = __builtin_rintf(x);
  const float f = x - n;
  float p = 1.326697064e-03f;
  p = __builtin_fmaf(p, f, 9.675459936e-03f);
  p = __builtin_fmaf(p, f, 5.550742522e-02f);
  p = __builtin_fmaf(p, f, 2.402212173e-01f);
  p = __builtin_fmaf(p, f, 6.931469440e-01f);
  p = __builtin_fmaf(p, f, 1.000000119e+00f);
  return __builtin_amdgcn_ldexpf(p, (int)n);
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Reductions over the lane pair (l, l ^ 32) with v_permlane32_swap (no LDS round trip): the swap
// of x with itself leaves x[l % 32] in the first and x[32 + l % 32] in the second result.
__device__ __forceinline__ float pair32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// True on every lane if the predicate holds on any lane of the wave (wave-uniform branch).
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Workgroup order. The hardware hands workgroup i of a 1-D grid to XCD i % 8 (each XCD has its own
// L2). Tile-major order: workgroup i runs tile i / units of unit i % units, tiles in the given
// direction (longest first for causal masks), so every wave of dispatch covers all units and each
// XCD gets the same mix of long and short work even when units (packed sequences) differ in
// length; when units is a multiple of 8, every tile of a unit runs on one XCD.
// Within an XCD the workgroups are dealt out in turn to its shader engines (workgroup i to engine
// (i / 8) % 4), so without care a unit count that is a multiple of 32 pins every tile of a unit to
// one engine; with packed sequences of unequal length one engine then gets several times the
// average work (measured: the packed Hkv8 dK/dV pass ran at half the dense rate). Each tile row is
// therefore rotated by 8 units: a unit keeps its XCD and its tiles cycle through the engines.
// The other orders (kOrderQuery: the forward and the dQ pass; kOrderGrouped: the dK/dV passes of dense
// batches) apply when units is a multiple of 8, so that a unit keeps one XCD and its tiles run close
// together in time there, sharing their K/V (Q/dO) through that XCD's L2:
//  - kOrderQuery, few tiles per unit (short sequences): unit-major inside each XCD. Workgroup i still runs on XCD
//    i % 8, and that XCD's consecutive workgroups take the tiles of one unit; tile-major order would
//    start a unit's second tile only after every unit's first, long after its K/V left the L2.
//    Measured on B128 H16 S256 D128: forward -9 %, dQ pass -7 %.
//  - both, more than kUnitsInFlight units per XCD: the XCD's units are taken kUnitsInFlight at a time, and
//    each such group runs tile-major (longest tile first, each tile row rotated by one unit across
//    the shader engines). Plain tile-major order spreads every round over all of the XCD's units, so
//    their K/V no longer fits the caches once an XCD holds many units; plain unit-major order runs
//    all of one unit's tiles at once, which measured slower on few long units (dense B2 H16 S8192:
//    forward +7 %). Measured against tile-major everywhere (same-run A/B, bit-identical results):
//    B8 H32 S4096 D128 forward -27 %, dQ pass -19 %, dK/dV pass -14 %; the packed batch of 16 sequences
//    U{256..4096}, H32/8 forward -7 %; B4 H32/8 S8192 dQ pass -4.5 %; groups of 2 or 8 units measured
//    within 2 % of 4. With at most kUnitsInFlight units per XCD the order is tile-major as before.
// The dK/dV pass (Q/dO shared by a unit's key tiles) ran 2.6 % slower unit-major on short sequences, and
// grouped, the packed batch of 16 sequences ran 11 % slower (also with the units sorted by sequence
// length first, so not for want of its longest-first rounds): packed dK/dV passes keep tile-major order
// (kOrderTileMajor).
constexpr int kFewTiles = 4;
constexpr int kUnitsInFlight = 4;
// Key-tile passes (dK/dV): round t of tile_order's order takes, for a unit whose sequence has ceil(len /
// tile_len) key tiles, its tile t - (n_tiles - that count); negative = nothing to do in this round. Units are
// thereby aligned at the ends of their sequences, so each round holds tiles at the same distance from their
// sequence's last key, which under every mask means about the same work, and the rounds run longest work first
// (start-aligned, a round would mix a long sequence's first tiles with a short one's last; measured on the
// packed batch of 16 sequences U{256..4096}: dK/dV pass -10.6 %, the same order as before on dense batches).
__device__ __forceinline__ int end_aligned(int t, int n_tiles, int len, int tile_len) {
  return t - (n_tiles - (len + tile_len - 1) / tile_len);
}
// The (unit, tile) of workgroup i (0 <= i < units * tiles; a bijection onto units x tiles). Host and device:
// the library's attn_tile_order_probe evaluates the same function on the host.
__host__ __device__ __forceinline__ void tile_map(int i, int units, int tiles, bool reverse, int order, int& unit,
                                                  int& tile) {
  if (order == kOrderQuery && units % 8 == 0 && tiles <= kFewTiles) {
    const int k = i / 8;
    unit = (k / tiles) * 8 + i % 8;
    tile = k % tiles;
  } else if (order != kOrderTileMajor && units % 8 == 0 && units / 8 > kUnitsInFlight) {
    const int k = i / 8;                               // position in XCD i % 8's sequence
    const int c = k / (kUnitsInFlight * tiles);        // group of units
    const int left = units / 8 - kUnitsInFlight * c;   // units of this XCD from group c on
    const int cu = left < kUnitsInFlight ? left : kUnitsInFlight;
    const int r = k - c * kUnitsInFlight * tiles;      // position in the group, tile-major
    tile = r / cu;
    unit = (kUnitsInFlight * c + (r + tile) % cu) * 8 + i % 8;
  } else {
    tile = i / units;
    unit = (i % units + 8 * (tile % units)) % units;
  }
  if (reverse) tile = tiles - 1 - tile;
}
__device__ __forceinline__ void tile_order(int units, int tiles, bool reverse, int& unit, int& tile, int order) {
  tile_map(blockIdx.x, units, tiles, reverse, order, unit, tile);
}
// Query-side units (forward, dQ pass) are q-heads in (sequence, q-head) order, so consecutive
// q-heads, including the heads of one GQA group, run on different XCDs. Measured on the packed
// Hq32/Hkv8 workload: keeping a group's heads on one XCD (sharing K/V in its L2) made the forward
// and the dQ pass about 1.8x slower than spreading them.
__device__ __forceinline__ void q_unit(int u, int batch, int hkv, int group, int& b, int& h) {
  b = u / (hkv * group);
  h = u % (hkv * group);
}

}  // namespace sdpa
