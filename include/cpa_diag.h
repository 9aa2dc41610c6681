/*
 * cpa_diag.h - measurement helpers beside the Block-Union KV Selection library (gfx950).
 *
 * Not part of the attention path.  They give the reference points the prefill's fraction of
 * peak is read against: the rate the bf16 matrix cores reach on a loop of nothing but
 * independent MFMAs, the shader clock they run at while doing so, and the clocks the device
 * reports.  Same conventions as cpa.h: caller-owned device buffers, host-side checks before any
 * HIP call, work only enqueued on `stream`.
 */
#ifndef CPA_DIAG_H
#define CPA_DIAG_H

#include "cpa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * cpa_diag_mfma_loop - `blocks` workgroups of `threads` threads (a multiple of 64, at most
 * 512: one or two waves per SIMD) each run `iters` iterations of four independent
 * v_mfma_f32_32x32x16_bf16 per wave (32768 FLOP each), with no memory traffic in the loop.
 * One launch performs blocks * (threads / 64) * iters * 4 * 32768 FLOP.
 *
 *   sink  (out) device float [blocks * threads]: one value per thread, so the work is not
 *         optimised away; its contents have no meaning.
 *   clk   (out) device uint64 [2]: for workgroup 0, the shader-clock cycles (s_memtime) and the
 *         constant-rate wall-clock ticks (s_memrealtime) its loop took.  Their ratio times the
 *         wall-clock rate (cpa_diag_clock_rates) is the engine clock during the loop.
 * Errors: CPA_ERR_NULL, CPA_ERR_SHAPE (blocks < 1, threads not in {64, ..., 512} or not a
 * multiple of 64, iters outside [1, 10^7]), CPA_ERR_ALIGN (clk not 8-byte aligned),
 * CPA_ERR_LAUNCH.
 */
cpa_status cpa_diag_mfma_loop(int blocks, int threads, int iters, float* sink, unsigned long long* clk,
                              hipStream_t stream);

/*
 * cpa_diag_clock_rates - the device's peak engine clock and its constant wall-clock rate, in
 * kHz (host outputs), as the HIP runtime reports them (hipDeviceAttributeClockRate and
 * hipDeviceAttributeWallClockRate).  Errors: CPA_ERR_NULL, CPA_ERR_SHAPE (no such device).
 */
cpa_status cpa_diag_clock_rates(int device, int* engine_khz, int* wall_khz);

#ifdef __cplusplus
}
#endif
#endif /* CPA_DIAG_H */
