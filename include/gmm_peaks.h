/*
 * gmm_peaks.h — peak-rate probes exported by libgmm_mi355x.so, beside the
 * E-step entry points of gmm.h.
 *
 * The E-step kernels are bound by the matrix cores (the score and statistics
 * contractions: "Turbo-GMM: FlashAttention-Inspired GPU-Accelerated Gaussian
 * Mixture Model", abstract, the dense scoring of N points against K
 * components) or by HBM reads of X (the small-K regime, where the whole
 * component axis stays on chip and X is streamed once). These probes measure
 * what this GPU actually sustains on each, so that the kernels' rates can be
 * quoted against a measured peak as well as the datasheet one. They compute
 * nothing useful.
 *
 * Conventions as in gmm.h: device pointers owned by the caller, asynchronous
 * on `stream` (a hipStream_t, NULL = default), time them with events on that
 * stream. Return 0, -1 for an invalid argument (nothing enqueued), -4 when the
 * launch fails.
 */
#ifndef GMM_MI355X_PEAKS_H
#define GMM_MI355X_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum gmm_peak_precision { GMM_PEAK_FP32 = 0, GMM_PEAK_FP64 = 1 };

/* Matrix-core issue loop: `blocks` blocks of four waves, each wave running
 * `trips` trips of eight independent MFMAs (32x32x2 fp32 or 16x16x4 fp64)
 * on four accumulator chains. out: device, blocks * 256 floats (written). */
int gmm_peak_mfma(int32_t precision, int64_t trips, int32_t blocks, float* out, void* stream);

/* Flops one gmm_peak_mfma launch executes (host-only arithmetic). */
double gmm_peak_mfma_flops(int32_t precision, int64_t trips, int32_t blocks);

/* HBM read stream: reads every 16-byte chunk of buf[0 .. bytes) once
 * (bytes rounded down to a multiple of 16; buf 16-byte aligned) with
 * `blocks` blocks of 256 threads; out (device, blocks * 256 uint32) is
 * written only in a case that does not arise in practice. */
int gmm_peak_hbm_read(const void* buf, size_t bytes, int32_t blocks, uint32_t* out, void* stream);

/* Co-issue probe: whether fp32 vector (VALU) work runs beside fp32
 * matrix-core (MFMA) work on one SIMD, which decides whether the E-step
 * kernels' row phases (max, exponentials, error bounds: VALU) can hide under
 * their contractions (MFMA). `blocks` blocks of 512 threads (eight waves;
 * with one block per CU, waves w and w + 4 share SIMD w % 4), each wave
 * running `trips` trips. Per trip a matrix wave issues eight independent
 * 32x32x2 fp32 MFMAs and a vector wave 128 independent fp32 FMAs. mode 0:
 * matrix only; 1: vector only; 2: both in every wave; 3: waves 0-3 matrix,
 * waves 4-7 vector. If the two kinds of work overlapped, modes 2 and 3
 * would take about max(t0, t1) and max(t0, t1) / 2; serialised, t0 + t1 and
 * (t0 + t1) / 2. out: device, blocks * 512 floats (written). */
int gmm_peak_coissue(int32_t mode, int64_t trips, int32_t blocks, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GMM_MI355X_PEAKS_H */
