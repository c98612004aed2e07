/*
 * lynx_probe.h - test hooks of liblynx: one matrix instruction per wave on
 * raw per-lane register contents, so tests can pin the gfx950 operand layouts
 * (lane -> row/column/channel maps and the sparse-index bit order) that the
 * packed format in lynx.h and the GEMM kernels rely on.  The packed 2:4
 * operand the RT-Lynx page has the sparsifier emit (핵심 기여, third item)
 * must be exactly what the sparse matrix unit reads; these hooks let a test
 * check that on the device.
 *
 * Every pointer is a device pointer owned by the caller; each call launches
 * one workgroup of 64 lanes on `stream` and returns LYNX_OK or an error of
 * lynx_status (LYNX_ERR_NULL, LYNX_ERR_ALIGN, LYNX_ERR_SHAPE for an unknown
 * `which`/`abid`, LYNX_ERR_DEVICE, LYNX_ERR_UNSUPPORTED_DEVICE).
 * Per-lane buffers are lane-major: lane l's elements are contiguous.
 */
#ifndef LYNX_PROBE_H
#define LYNX_PROBE_H

#include "lynx.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * which = 0: v_smfmac_f32_16x16x64_bf16   a: 64x8 bf16, b: 64x16 bf16, idx: 64 u32, d: 64x4 f32
 * which = 1: v_smfmac_f32_32x32x32_bf16   a: 64x8 bf16, b: 64x16 bf16, idx: 64 u32, d: 64x16 f32
 * which = 2: v_mfma_f32_16x16x32_bf16     a: 64x8 bf16, b: 64x8 bf16,  idx unused,  d: 64x4 f32
 * which = 3: v_mfma_f32_32x32x16_bf16     a: 64x8 bf16, b: 64x8 bf16,  idx unused,  d: 64x16 f32
 * abid (0 or 1) is the sparse-index set selector of the smfmac forms (cbsz = 0).
 * The accumulator input is zero.
 */
lynx_status lynx_probe_mfma(int which, int abid, const uint16_t* a, const uint16_t* b,
                            const uint32_t* idx, float* d, lynx_stream_t stream);

/*
 * Matrix-instruction issue rate and clock: `grid` workgroups of 4 waves (one
 * wave per SIMD when grid = the compute-unit count); every wave issues
 * iters * 16 instructions `which` (numbered as above) over 4 independent
 * accumulators, stamping the shader-clock counter (s_memtime) and the 100 MHz
 * real-time counter (s_memrealtime) before and after.
 *   sink   [grid * 256] fp32 (written, keeps the work alive);
 *   stamps [grid * 4][2] uint64: per wave, shader cycles and real-time ticks
 *          spent in the loop.
 * Cycles per instruction = stamps[.][0] / (16 iters); the clock in MHz =
 * 100 * stamps[.][0] / stamps[.][1].  This measures the peak that the page's
 * sparse-unit speedups (주요 결과) rest on, on this device.
 */
lynx_status lynx_probe_mfma_rate(int which, int iters, int grid, float* sink, uint64_t* stamps,
                                 lynx_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LYNX_PROBE_H */
