/*
 * lily_trace.h: timelines of the one-launch expert FFN and of the
 * whole-step decode kernel (gfx950).
 *
 * The tracing build of the library (liblily_moe_trace.so: the same sources,
 * with gemm_w4.hip and decode.hip compiled with LILY_TRACE_ITEMS) records,
 * for every workgroup of each lily_moe_ffn launch (lily_moe_forward's
 * default path), when each of its work items started and ended and how long
 * it waited for its block's gate/up tiles, so that the launch's timeline
 * (occupancy, the end-of-launch tail, per-queue balance) can be read back;
 * and, for every workgroup and layer of each lily_moe_decode_stack launch,
 * when it passed the points between the layer's phases. Its outputs are the
 * product library's, bit for bit; the ordinary library (liblily_moe.so)
 * exports the same calls and returns LILY_ERR_UNSUPPORTED.
 *
 * Conventions as in lily_moe.h: 0 or a positive count on success, a
 * negative LILY_ERR_* code with lily_last_error() describing it.
 */
#ifndef LILY_TRACE_H
#define LILY_TRACE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Waits for `stream` (a hipStream_t as void*), then copies the trace of the
   last lily_moe_ffn launch on the current device into dst (host memory,
   caller-owned): uint64 [n][33][4], n = min(max_wgs, 1024) workgroups. Row
   i < 32 of workgroup w is its i-th item: {start, end, info, wait}, times in
   ticks of the 100 MHz wall clock (s_memrealtime); info = mia | down << 8 |
   n0 << 16 | schedule block << 32 (mia: 32-row sub-tiles holding rows;
   down: 1 for a down item; n0: first output column); wait: ticks spent
   waiting for the block's gate/up tiles. Row 32: {launch entry, exit, items
   run (rows past 32 not recorded), grid size}. Workgroups at or past the
   grid size hold stale rows. Returns n. Errors: LILY_ERR_INVALID_ARG (NULL
   dst, max_wgs < 1), LILY_ERR_UNSUPPORTED (not the tracing build),
   LILY_ERR_HIP. */
int lily_trace_ffn_items(unsigned long long* dst, int32_t max_wgs, void* stream);

/* Waits for `stream`, then copies the phase trace of the last
   lily_moe_decode_stack launch on the current device into dst (host memory,
   caller-owned): uint64 [n][64][8], n = min(max_wgs, 256) workgroups, layers
   0..63, ticks of the 100 MHz wall clock. Points per (workgroup, layer):
   0 layer start, 1 previous layer's output gathered and added to r, 2 x of
   the layer staged (norm done), 3 the workgroup's phase A part sums ready,
   4 its h words stored, 5 all h gathered by its compute wavefronts (points
   0-5 by the lead wavefront); 6 h gathered by compute wavefront 0, 7 the
   workgroup's phase B sums ready (compute wavefront 0; only workgroups with a
   phase B unit write it). Rows of layers past the launch's, and of
   workgroups past its grid, hold stale values. Returns n. Errors:
   LILY_ERR_INVALID_ARG, LILY_ERR_UNSUPPORTED (not the tracing build),
   LILY_ERR_HIP. */
int lily_trace_decode_stack(unsigned long long* dst, int32_t max_wgs, void* stream);

#ifdef __cplusplus
}
#endif

#endif
