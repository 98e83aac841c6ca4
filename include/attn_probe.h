/*
 * attn_probe.h - measurement probes of the MI355X (gfx950) attention library (libsdpa02.so).
 *
 * Measurement aids, not part of the attention computation.
 *  - attn_mfma_probe: the attention entry points (attn.h) run their QK^T and PV contractions and the
 *    backward's products on the matrix cores, and their throughput is reported as a fraction of the
 *    chip's published dense bf16 peak. This probe measures, on the same device and in the same
 *    process, the rate the matrix cores sustain from registers alone and the engine clock they run at,
 *    as a ceiling to read those fractions against.
 *  - attn_lds_probe: the kernels stage K/V (forward, dQ pass) and Q/dO (dK/dV pass) tiles in LDS and
 *    read them back as matrix-core operands; how the LDS serves a read (its banks, and which lanes share
 *    a cycle) decides the tile swizzle. This probe issues one wave's reads at caller-chosen per-lane
 *    addresses, to be run under the SQ_LDS_BANK_CONFLICT counter.
 *  - attn_tile_order_probe: the workgroup -> (unit, tile) order every kernel launch follows, evaluated
 *    on the host, so that its coverage of every (unit, tile) pair can be checked without a GPU.
 */
#ifndef SDPA02_ATTN_PROBE_H
#define SDPA02_ATTN_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Launches `blocks` workgroups of 256 threads on `stream`; every wave runs `iters` rounds of four
 * independent 32x32x16 bf16 MFMAs (32768 FLOP each) on register operands, with no memory traffic in
 * the loop, so one call executes blocks * 4 * iters * 4 * 32768 FLOP. Lane l of every wave uses the
 * operands A[t] = bf16(x + y * (l + 8t)) and B[t] = bf16(x - y * (l + 8t)), t = 0..7.
 *   out    device float[blocks * 256] (out_bytes at least that): thread i of workgroup w writes the sum
 *          of its 64 accumulator values to out[256 w + i]; with y = 0 that sum is
 *          1024 * bf16(x)^2 * iters (a check that every MFMA ran).
 *   ticks  device uint64[2 * blocks] (ticks_bytes at least that): ticks[2w] = shader-clock ticks and
 *          ticks[2w + 1] = 100 MHz reference ticks that wave 0 of workgroup w spent in the loop, so
 *          100 MHz * ticks[2w] / ticks[2w + 1] is the engine clock it ran at.
 * blocks in [1, ATTN_PROBE_MAX_BLOCKS], iters in [1, ATTN_PROBE_MAX_ITERS], x and y finite, out 4-byte
 * and ticks 8-byte aligned, the two not overlapping; otherwise nothing is launched and the status says
 * why (ATTN_E_INVALID / ATTN_E_ALIGN / ATTN_E_WORKSPACE / ATTN_E_OVERLAP). Asynchronous on `stream`;
 * the caller owns both buffers. */
#define ATTN_PROBE_MAX_BLOCKS 65536
#define ATTN_PROBE_MAX_ITERS (1 << 24)
attn_status_t attn_mfma_probe(int32_t blocks, int32_t iters, float x, float y, float* out, size_t out_bytes,
                              uint64_t* ticks, size_t ticks_bytes, void* stream);

/* Launches one wave (a workgroup of 64 threads) on `stream`. The wave fills an LDS array of
 * ATTN_LDS_PROBE_BYTES bytes, then every lane l with lane_addr[l] >= 0 reads at byte address
 * lane_addr[l] of it, 8 * iters times (lanes with a negative entry stay inactive):
 *   kind ATTN_LDS_READ_B128 (0): ds_read_b128, 16 bytes; ATTN_LDS_READ_B64_TR_B16 (1): the transpose read
 *   ds_read_b64_tr_b16, 8 bytes; ATTN_LDS_READ_B64 (2): ds_read_b64, 8 bytes.
 * So the dispatch issues 8 * iters reads of that kind (plus the fill's ATTN_LDS_PROBE_BYTES / 1024
 * ds_write_b128), and SQ_LDS_BANK_CONFLICT / (8 * iters) is the extra cycles per read.
 *   lane_addr  host int32[64]: every non-negative entry a multiple of the read's width (16 or 8) with
 *              entry + width <= ATTN_LDS_PROBE_BYTES;
 *   out        device int32[64] (out_bytes at least 256): lane l writes the sum of what it read.
 * iters in [1, ATTN_LDS_PROBE_MAX_ITERS]. Otherwise nothing is launched and the status says why
 * (ATTN_E_INVALID / ATTN_E_ALIGN / ATTN_E_WORKSPACE). Asynchronous on `stream`; lane_addr is read
 * before the call returns. */
#define ATTN_LDS_PROBE_BYTES 32768
#define ATTN_LDS_PROBE_MAX_ITERS (1 << 20)
#define ATTN_LDS_READ_B128 0
#define ATTN_LDS_READ_B64_TR_B16 1
#define ATTN_LDS_READ_B64 2
attn_status_t attn_lds_probe(int32_t kind, const int32_t* lane_addr, int32_t iters, int32_t* out, size_t out_bytes,
                             void* stream);

/* Host only (no HIP call). Writes, for each workgroup index i in [0, units * tiles), the unit and the
 * tile that workgroup i of a launch over `units` units of `tiles` tiles each is given: unit_out[i] and
 * tile_out[i]. order selects the launch: ATTN_ORDER_QUERY the query-tile passes (forward, dQ pass; a unit
 * is a (sequence, q-head) pair), ATTN_ORDER_GROUPED the dK/dV passes of dense batches and
 * ATTN_ORDER_TILE_MAJOR those of packed batches (a unit is a (sequence, kv-head) pair; the tile is the
 * round before the end-aligned shift of each unit's key tiles); reverse = 1 numbers the tiles from the
 * last (the causal query-tile passes run their longest tiles first). Every (unit, tile) pair occurs
 * exactly once.
 * Arguments: units, tiles >= 1 with units * tiles <= ATTN_TILE_ORDER_PROBE_MAX; reverse 0 or 1; order one
 * of the three values; unit_out, tile_out caller-owned host arrays of n = units * tiles int32 each.
 * Otherwise nothing is written and the status says why (ATTN_E_INVALID). */
#define ATTN_ORDER_TILE_MAJOR 0
#define ATTN_ORDER_QUERY 1
#define ATTN_ORDER_GROUPED 2
#define ATTN_TILE_ORDER_PROBE_MAX (1 << 24)
attn_status_t attn_tile_order_probe(int32_t units, int32_t tiles, int32_t reverse, int32_t order, int32_t* unit_out,
                                    int32_t* tile_out, size_t n);

#ifdef __cplusplus
}
#endif

#endif /* SDPA02_ATTN_PROBE_H */
