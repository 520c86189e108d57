/*
 * ss_probe.h -- C ABI of libssprobe.so, the ceiling probes that bound the scan kernels on the
 * MI355X (gfx950).  Measurement only: nothing here computes any part of the scan.  The pages
 * place the cost of the fused scan in memory traffic (omica.com.cn Mamba explainer, section 5;
 * bqwf.cn state-space survey, section 2.2, the hardware-aware scan kept in fast on-chip memory);
 * on this GPU the diagonal scan's exp per (step, state) also makes the plain ALUs a competing
 * bound, so the probes measure both ceilings.
 *
 * Every call is asynchronous on `stream` (a hipStream_t as void*, NULL = the default stream);
 * pointers are caller-owned device memory; the return value is a hipError_t (0 = success).
 */
#ifndef SS_PROBE_H
#define SS_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* VALU issue probe: `blocks` blocks of 256 threads; every wave runs `iters` rounds of 32
 * independent instructions of one kind: 0 f32 multiply, 1 f32 FMA, 2 f32 exp (v_exp_f32),
 * 3 DPP multiply, 4 exps and FMAs alternating, 5 one exp in four FMAs.  `out` receives
 * blocks * 256 floats (kept so that the work is not removed); `clk` two counts over the first
 * wave's loop: shader clocks (s_memtime) and ticks of the 100 MHz reference clock
 * (s_memrealtime), whose ratio is the clock the probe ran at.  Cycles per instruction per SIMD =
 * duration x clock / (instructions issued per SIMD). */
int ssp_valu(int kind, int blocks, int iters, float* out, uint64_t* clk, void* stream);

/* Streaming copy of n16 16-byte words from src to dst (disjoint), `blocks` blocks of 256 threads
 * (grid-stride); bytes moved = 32 n16. */
int ssp_copy(const void* src, void* dst, int64_t n16, int blocks, void* stream);

/* Streaming read of n16 16-byte words of src; `out` receives blocks * 256 words. */
int ssp_read(const void* src, uint32_t* out, int64_t n16, int blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SS_PROBE_H */
