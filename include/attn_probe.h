/*
 * attn_probe.h - matrix-core rate probe of the MI355X (gfx950) attention library (libsdpa02.so).
 *
 * A measurement aid, not part of the attention computation. The attention entry points (attn.h) run
 * their QK^T and PV contractions and the backward's products on the matrix cores; their throughput is
 * reported as a fraction of the chip's published dense bf16 peak. This probe measures, on the same
 * device and in the same process, the rate the matrix cores sustain from registers alone and the engine
 * clock they run at, as a ceiling to read those fractions against.
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

#ifdef __cplusplus
}
#endif

#endif /* SDPA02_ATTN_PROBE_H */
