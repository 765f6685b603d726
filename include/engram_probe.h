/*
 * engram_probe.h -- C ABI of libengram_probe.so: microbenchmarks that measure
 * the ceilings the Engram path's kernels are compared against on this GPU
 * (AMD Instinct MI355X, gfx950).  They compute nothing of the method; the
 * benchmark times them with HIP events on `stream` and reports every kernel's
 * fraction of the spec peak and of these measured ones.
 *
 * Conventions as include/engram.h: device pointers, caller-owned memory,
 * asynchronous on `stream`, host-side validation first, 0 = ok.
 */
#ifndef ENGRAM_PROBE_H
#define ENGRAM_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Matrix-core ceiling: `workgroups` workgroups of `waves` waves (1..8) each run
 * `iters` iterations of independent MFMAs on operands held in registers (no
 * memory traffic in the loop): 4 chains of 32 x 32 blocks or 8 of 16 x 16.
 *   kind 0: v_mfma_f32_32x32x16_bf16          (32,768 flop each, 4 per iteration)
 *   kind 1: v_mfma_f32_32x32x64_f8f6f4, E4M3   (131,072 flop each, 4 per iteration;
 *           issued through the scaled builtin with zero scale operands, which the
 *           compiler turns into the unscaled instruction)
 *   kind 2: v_mfma_f32_16x16x32_bf16           (16,384 flop each, 8 per iteration)
 *   kind 3: v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 with E8M0 scales from
 *           registers (131,072 flop each, 4 per iteration)
 *   kind 4: v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 with E8M0 scales from
 *           registers (65,536 flop each, 8 per iteration)
 * The operands are read once from `operands` (random bytes, at least 64 KiB),
 * so their bit patterns are those of real data; `out` receives one float per
 * wave (the accumulators' sum) so nothing is optimised away.
 * flops = workgroups * waves * iters * (MFMAs per iteration) * (flop per MFMA).
 * Returns 1 on invalid arguments (kind outside 0..4 among them).
 */
int engram_probe_mfma(int32_t kind, const void* operands, float* out, int32_t workgroups, int32_t waves,
                      int32_t iters, void* stream);

/* HBM read ceiling: every byte of src [bytes] read once with 16-byte loads
 * (bytes a multiple of 16, src 16-byte aligned); out [grid] floats. */
int engram_probe_read(const void* src, int64_t bytes, float* out, void* stream);

/* HBM copy ceiling: dst[0:bytes) = src[0:bytes) with 16-byte loads and stores. */
int engram_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* Workgroups engram_probe_read launches (the size of its `out`). */
int32_t engram_probe_read_grid(void);

#ifdef __cplusplus
}
#endif
#endif /* ENGRAM_PROBE_H */
