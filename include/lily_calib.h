/*
 * lily_calib.h: calibration kernels of the MoE library (gfx950).
 *
 * They measure what one MI355X achieves, so that the MoE kernels can be
 * reported against measured peaks as well as published ones: MFMA throughput
 * on changing operands with the shader clock it runs at, the rate of the
 * grouped GEMMs' int4 -> bf16 weight rebuild on the VALU, and streaming HBM
 * reads (plain vector loads, and the LDS DMA loads the grouped GEMMs use).
 * They compute nothing of the MoE layer.
 *
 * Conventions as in lily_moe.h: device pointers, caller-owned buffers,
 * asynchronous on `stream` (a hipStream_t as void*), 0 or a negative
 * LILY_ERR_* code with lily_last_error() describing it.
 */
#ifndef LILY_CALIB_H
#define LILY_CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* grid workgroups of waves_per_cu wavefronts (1..8; one workgroup per
   compute unit when grid = the CU count) each run `iters` (even) rounds of 8
   independent v_mfma_f32_32x32x16_bf16 (32768 flops each) on random bf16
   operands. sink: float [grid * waves_per_cu * 64] (written, meaningless);
   times: uint64 [grid * waves_per_cu][2], per wavefront the shader-clock
   cycles (s_memtime) and the 100 MHz wall ticks (s_memrealtime) of its loop.
   Errors: LILY_ERR_INVALID_ARG, LILY_ERR_HIP. */
int lily_calib_mfma(int32_t grid, int32_t waves_per_cu, int32_t iters, float* sink,
                    unsigned long long* times, void* stream);

/* The grouped GEMMs' rebuild of int4 weights as bf16(scale * q + bias) on
   the VALU, alone: grid workgroups of waves_per_cu wavefronts (1..16) each
   run `iters` rounds of 8 independent words per lane (64 weights per lane
   per round: per word one add, the 19-instruction rebuild of 8 weights and
   two 3-input sums). sink: uint32 [grid * waves_per_cu * 64] (written,
   meaningless); times: uint64 [grid * waves_per_cu][2], per wavefront the
   shader-clock cycles and 100 MHz wall ticks of its loop. Errors:
   LILY_ERR_INVALID_ARG, LILY_ERR_HIP. */
int lily_calib_dequant(int32_t grid, int32_t waves_per_cu, int32_t iters, uint32_t* sink,
                       unsigned long long* times, void* stream);

/* Reads `bytes` (a multiple of 1024) from src (16-byte aligned) with grid
   workgroups of 256 threads, grid-stride, each thread XOR-reducing what it
   read into sink: uint32 [grid * 256]. dma = 0: global_load_dwordx4 into
   registers; dma = 1: global_load_lds_dwordx4 (LDS DMA), 1 KB per load, four
   loads in flight per wavefront. Errors: LILY_ERR_INVALID_ARG, LILY_ERR_HIP. */
int lily_calib_read(const void* src, size_t bytes, int32_t grid, int32_t dma, uint32_t* sink,
                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LILY_CALIB_H */
