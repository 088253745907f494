/*
 * lily_trace.h: the item trace of the one-launch expert FFN (gfx950).
 *
 * The tracing build of the library (liblily_moe_trace.so: the same sources,
 * with moe_w4_ffn compiled with LILY_TRACE_ITEMS) records, for every
 * workgroup of each lily_moe_ffn launch (lily_moe_forward's default path),
 * when each of its work items started and ended and how long it waited for
 * its block's gate/up tiles, so that the launch's timeline (occupancy, the
 * end-of-launch tail, per-queue balance) can be read back. Its outputs are
 * the product library's, bit for bit; the ordinary library
 * (liblily_moe.so) exports the same call and returns LILY_ERR_UNSUPPORTED.
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

#ifdef __cplusplus
}
#endif

#endif
