/* mla_peaks.h -- achievable-peak micro-benchmarks for one MI355X (gfx950).
 *
 * Measurement support, not part of the attention path: these calls let a benchmark state
 * a kernel's roofline fraction against what the chip measurably delivers as well as
 * against the published peaks (HBM3E 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s).  Built as a
 * library of its own (libmlapeaks.so) so the attention library exports only the path.
 *
 * Common rules: every pointer is a DEVICE pointer owned by the caller; every call is
 * asynchronous on `stream` (a hipStream_t; NULL is the default stream); the caller times
 * it (e.g. with events on that stream).  Return 0, -1 for invalid arguments (nothing is
 * launched), -4 when the launch fails.  Kernels use 256-thread workgroups.
 */
#ifndef MLA_PEAKS_H
#define MLA_PEAKS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (a positive multiple of 16, `buf` 16-byte aligned) once with 16-byte
 * non-temporal loads, eight in flight per thread, over `n_wg` workgroups.  sink[n_wg]
 * (u32) receives, per workgroup, the XOR of every 32-bit word that workgroup read, so the
 * XOR over all sinks equals the XOR of the whole buffer. */
int mla_peak_hbm_read(const void *buf, size_t bytes, unsigned *sink, int n_wg, void *stream);

/* Dense bf16 MFMA issue rate: each of the n_wg x 4 waves runs `iters` steps of eight
 * independent v_mfma_f32_16x16x32_bf16 (16,384 flops each) with A = 1.0 and B = b_val.
 * sink[n_wg * 256] (fp32) receives per thread the sum of its 32 accumulator values,
 * 1024 * b_val * iters when exact.  Flops = n_wg * 4 * iters * 8 * 16384. */
int mla_peak_mfma_bf16(int iters, float b_val, float *sink, int n_wg, void *stream);

/* LDS read rate: each of the n_wg x 4 waves runs `iters` steps that each read an 8 KiB
 * slot of a 64 KiB LDS array: eight ds_read_b128 (16 B per lane) when transpose = 0,
 * sixteen ds_read_b64_tr_b16 (8 B per lane) otherwise, all in flight before one wait.
 * Bytes read = n_wg * 4 * iters * 8192.  Word w of the array holds h | h << 16 with
 * h = (w * 40503) mod 65536; step `it` of wave v reads bytes 8192 s .. 8192 s + 8191,
 * s = 4 (it mod 2) + v.  sink[n_wg] (u32) receives each workgroup's XOR of the first
 * 32-bit word of every read (b128: words 4 l + 256 i of the slot for lane l, read i). */
int mla_peak_lds_read(int iters, int transpose, unsigned *sink, int n_wg, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PEAKS_H */
