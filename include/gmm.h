/*
 * gmm.h — C-ABI of libgmm_mi355x.so: the fused Gaussian-mixture EM E-step for
 * MI355X (gfx950), with its M-step, EM loop and top-2 assignment.
 *
 * The operation (pages: "Turbo-GMM: FlashAttention-Inspired GPU-Accelerated
 * Gaussian Mixture Model", abstract; "Flash-GMM: a memory-efficient kernel for
 * scalable soft clustering", abstract): EM for a Gaussian mixture scores N
 * points against K components, normalises each point's responsibilities with
 * a log-sum-exp, and accumulates the sufficient statistics, without writing
 * the N x K responsibility matrix to memory.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every array pointer is a DEVICE pointer owned by the caller. The library
 *   allocates no device memory of its own: scratch comes from `workspace`,
 *   which must hold at least gmm_workspace_bytes(N, d, K) bytes and be
 *   256-byte aligned (any hipMalloc / torch allocation is).
 * - Layouts are row-major and dense: X is N x d (x_dtype GMM_F32 = float,
 *   GMM_F16 = IEEE half, GMM_BF16 = bfloat16; half and bfloat16 values are
 *   widened exactly and all arithmetic is as for float X), mu and var are
 *   K x d float, logw is K float,
 *   Sx and Sxx are K x d float, Nk is K float.
 * - The mixture is diagonal: component k has mean mu[k], variance var[k]
 *   (per feature, > 0) and log mixing weight logw[k] (-inf allowed; at least
 *   one component must be finite).
 * - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *   enqueues work on it and never synchronises; outputs are valid once the
 *   stream has completed. Calls that share a workspace must be ordered on
 *   one stream.
 * - Return value: GMM_OK (0) or a negative GMM_E* code. Arguments are checked
 *   on the host before anything is enqueued: a rejected call enqueues nothing
 *   and touches no device memory. gmm_error_string() names each code.
 * - Limits: 1 <= d <= 128, 1 <= K <= 65536, 0 <= N < 2^40.
 * - Non-finite inputs (NaN X, var <= 0) are not checked on the device; they
 *   propagate into the outputs as NaN/Inf.
 */
#ifndef GMM_MI355X_H
#define GMM_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum gmm_status {
  GMM_OK = 0,
  GMM_EINVAL = -1,        /* null pointer, negative size, bad dtype or regime */
  GMM_EUNSUPPORTED = -2,  /* shape beyond the limits above, or regime not possible */
  GMM_EWORKSPACE = -3,    /* workspace NULL, too small or misaligned */
  GMM_EHIP = -4,          /* a HIP launch failed (see hipGetLastError) */
  GMM_ESCRATCH = -5       /* gmm_estep_stats_static: shape needs more than its static scratch */
};

enum gmm_dtype { GMM_F32 = 0, GMM_F16 = 1, GMM_BF16 = 2 };

/* Regime of the E-step (Turbo-GMM abstract: a single sweep over the component
 * axis kept on chip when it fits, a two-pass fallback otherwise).
 *   SINGLE  - single sweep, 32-component tiles, K <= 256
 *   TWOPASS - normalisers first, then statistics; any K. The first pass
 *             scores in fp32 on the matrix cores and keeps a few candidates
 *             per row and 256-component slab; a merge re-scores exactly
 *             (fp64) the entries a row's normaliser depends on, and the rare
 *             rows it cannot settle get an fp64 normaliser pass; the second
 *             pass then scores, per slab, only the rows that hold a
 *             responsibility above the statistics threshold there
 *   SMALLK  - single sweep with 16-component tiles, K <= 16 and d <= 64
 * AUTO takes SMALLK when it applies, else SINGLE for K <= 256, else TWOPASS. */
enum gmm_regime { GMM_REGIME_AUTO = 0, GMM_REGIME_SINGLE = 1, GMM_REGIME_TWOPASS = 2, GMM_REGIME_SMALLK = 3 };

/* Library version, major*10000 + minor*100 + patch. */
int gmm_version(void);

/* Static text for a status code. */
const char* gmm_error_string(int code);

/* Workspace bytes needed by every entry point below for this (N, d, K).
 * The fused kernels keep the responsibilities on chip (Flash-GMM abstract:
 * no N x K matrix in memory), so the scratch holds only the packed
 * parameters, per-row normalisers of the two-pass regime (Turbo-GMM
 * abstract: normalisers first, then a second score computation) and per-block
 * statistics partials: O(N + K d) bytes, never O(N K).
 * Returns 0 for arguments outside the limits. */
size_t gmm_workspace_bytes(int64_t N, int32_t d, int32_t K);
/* (In the two-pass regime the first pass also keeps 56 bytes per row and
 * 256-component slab, and the second pass's per-slab row lists 4 more, so the
 * workspace grows as N K / 256 there: about 4.8 GB in all at N = 4,194,304,
 * d = 128, K = 4096.) */

/* E-step with sufficient statistics (Turbo-GMM abstract: responsibility
 * normalisation and sufficient-statistic accumulation; Flash-GMM abstract:
 * no materialised responsibility matrix).
 *   s_nk = logw_k + log N(x_n | mu_k, diag var_k)
 *   l_n  = log sum_k exp(s_nk)          (per-point log-likelihood)
 *   r_nk = exp(s_nk - l_n)
 *   Nk[k] = sum_n r_nk,  Sx[k][j] = sum_n r_nk x_nj,  Sxx[k][j] = sum_n r_nk x_nj^2
 *   *loglik_total = sum_n l_n (device double)
 * loglik_point (nullable) receives l_n as N floats. N = 0 gives zero stats and
 * a zero log-likelihood. Outputs are fully overwritten. */
int gmm_estep_stats(const void* X, int32_t x_dtype, int64_t N, int32_t d,
                    const float* mu, const float* var, const float* logw, int32_t K,
                    float* Nk, float* Sx, float* Sxx,
                    double* loglik_total, float* loglik_point,
                    void* workspace, size_t ws_bytes, void* stream);

/* Allocation-free E-step, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): gmm_estep_stats (AUTO regime, same kernels, same results bit
 * for bit) without a workspace argument. It calls no hipMalloc, hipFree or
 * allocating library routine. Its scratch is a static device array of
 * GMM_STATIC_SCRATCH_MIB MiB that the library holds on every GPU it runs on
 * until the process ends (its address is looked up once per device, on the
 * first call there). Shapes whose workspace plan needs more than that
 * return GMM_ESCRATCH before anything is enqueued; for reference,
 * N = 1,048,576, d = 128, K = 256 needs about 68 MiB. Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (concurrent streams,
 * threads) race and give wrong results, so order them on one stream.
 * Arguments and outputs as in gmm_estep_stats. */
#define GMM_STATIC_SCRATCH_MIB 128
int gmm_estep_stats_static(const void* X, int32_t x_dtype, int64_t N, int32_t d,
                           const float* mu, const float* var, const float* logw, int32_t K,
                           float* Nk, float* Sx, float* Sxx,
                           double* loglik_total, float* loglik_point, void* stream);

/* gmm_estep_stats with the regime forced (GMM_REGIME_SINGLE needs K <= 256,
 * GMM_REGIME_SMALLK needs K <= 16 and d <= 64; otherwise GMM_EUNSUPPORTED). */
int gmm_estep_stats_regime(const void* X, int32_t x_dtype, int64_t N, int32_t d,
                           const float* mu, const float* var, const float* logw, int32_t K,
                           float* Nk, float* Sx, float* Sxx,
                           double* loglik_total, float* loglik_point,
                           void* workspace, size_t ws_bytes, int32_t regime, void* stream);

/* Testing aid: materialises R (N x K floats, row-major) through the same
 * scoring and normalisation code as gmm_estep_stats in the given regime, so
 * responsibilities can be checked element by element on small N. The
 * statistics are computed too and discarded; loglik_point is nullable. */
int gmm_estep_resp(const void* X, int32_t x_dtype, int64_t N, int32_t d,
                   const float* mu, const float* var, const float* logw, int32_t K,
                   float* R, float* loglik_point,
                   void* workspace, size_t ws_bytes, int32_t regime, void* stream);

/* M-step for diagonal covariance (the EM update the Turbo-GMM abstract
 * alternates with the E-step), in double precision:
 *   w_k = Nk/N,  mu_k = Sx_k/Nk,  var_k = max(Sxx_k/Nk - mu_k^2, var_floor)
 * mu, var, logw are in/out. A component with Nk < 1e-12*N keeps its mu and
 * var; its logw becomes log(max(Nk, 1e-300)/N). Needs N >= 1, var_floor >= 0. */
int gmm_mstep(const float* Nk, const float* Sx, const float* Sxx, int64_t N, int32_t d, int32_t K,
              float var_floor, float* mu, float* var, float* logw, void* stream);

/* EM iterations (Turbo-GMM abstract: EM alternates the fused E-step with the
 * parameter update; its fused kernels are equivalent to standard EM in real
 * arithmetic). `iters` iterations on the device: E-step (AUTO regime) then M-step, all
 * enqueued on `stream` with nothing read back. loglik_hist (device, `iters`
 * doubles) receives the log-likelihood of the parameters before each M-step.
 * mu, var, logw are in/out. Needs N >= 1, iters >= 0. */
int gmm_em_iterate(const void* X, int32_t x_dtype, int64_t N, int32_t d, int32_t K, int32_t iters,
                   float var_floor, float* mu, float* var, float* logw, double* loglik_hist,
                   void* workspace, size_t ws_bytes, void* stream);

/* Launch-shape query (host only, touches no device): the plan that
 * gmm_estep_stats_regime would use for (N, d, K, regime). info (host, 7
 * int64) receives {regime taken (1 single, 2 two-pass, 3 small-K), waves per
 * block, component slabs, rows per statistics chunk, number of chunks, 64-row
 * tiles, scratch bytes this plan uses}. A chunk is the row range whose statistics one block (one slab's
 * block in the two-pass regime) accumulates on chip across its tiles, so
 * rows per chunk / 64 is the number of tiles a block walks (Turbo-GMM
 * abstract: statistics accumulated on chip over the traversal). Returns the
 * codes of gmm_estep_stats_regime for the same arguments. */
int gmm_plan_info(int64_t N, int32_t d, int32_t K, int32_t regime, int64_t* info);

/* Measurement aid (one-shot, per host thread): the next E-step enqueued by
 * this thread through gmm_estep_stats, gmm_estep_stats_regime or
 * gmm_em_iterate records `start` (a hipEvent_t) on its stream immediately
 * before its fused E-step kernel(s) and `stop` immediately after them (before
 * the small reduction kernels), then forgets both. Passing NULLs cancels a
 * pending request. The events are the caller's; the library only records
 * them. Always returns GMM_OK. */
int gmm_set_timing_events(void* start, void* stop);

/* Precision of the statistics contraction (Nk, Sx, Sxx = sums of r * [1, x,
 * x^2]) of the fused E-step kernels. The pages measure their kernels with
 * half-precision data ("Flash-KMeans" article, test setup); these modes move
 * that contraction onto the bf16 or fp16 matrix cores where it pays:
 *   GMM_STATS_AUTO      - (default) as GMM_STATS_FP32, except that the second
 *                          pass of the two-pass regime takes exact fp16
 *                          splits when X is IEEE half: x is exact in fp16,
 *                          (16 x)^2 splits exactly into two fp16 values for
 *                          |x| >= 2^-6 (within 2^-25 below), and 2^10 r =
 *                          hi + lo + d with |d| <= max(2^-22 of it, 2^-25),
 *                          so each product is off by <= 2^-21 relative, plus
 *                          2^-35 |x| or 2^-35 x^2 + 2^-68 absolute, plus
 *                          2^-33 r on an Sxx term with |x| < 2^-6, before
 *                          the fp32 accumulation: close to fp32 products
 *                          except for the absolute floor on tiny features.
 *                          When some row has |x|^2 >= 225 (as the first pass
 *                          records it; then some |x_j| may reach 15 and
 *                          (16 x)^2 leave the fp16 range), the whole second
 *                          pass takes fp32 products instead;
 *   GMM_STATS_FP32      - fp32 MFMA products everywhere;
 *   GMM_STATS_SPLIT_BF16 - every fp32 operand v is split as v = hi + lo + d
 *                          with hi = bf16(v), lo = bf16(v - hi), |d| <=
 *                          2^-16 |v|, and a*b is taken as hi*hi + hi*lo +
 *                          lo*hi, exact products accumulated in fp32: each
 *                          product is off by <= 3.0001 * 2^-16 |a b| (4.6e-5
 *                          relative) before the accumulation's rounding,
 *                          inside the 1e-4 bar on the statistics. The
 *                          variance an M-step forms from them, Sxx/Nk - mu^2,
 *                          then carries up to 4.6e-5 (mu^2 + var) of absolute
 *                          error.
 * Scores, responsibilities, l_n and L are the same in every mode (fp32 MFMA
 * scores with the exact re-score). The setting is process-wide and read when
 * an E-step is enqueued (gmm_estep_stats*, gmm_estep_resp, gmm_em_iterate).
 * Returns GMM_OK, or GMM_EINVAL for an unknown mode (setting unchanged). Not
 * synchronised with calls enqueued concurrently from other threads. */
enum gmm_stats_precision { GMM_STATS_FP32 = 0, GMM_STATS_SPLIT_BF16 = 1, GMM_STATS_AUTO = 2 };
int gmm_set_stats_precision(int32_t mode);

/* Top-2 assignment for border-vector multi-assignment (Flash-GMM abstract:
 * responsibilities assign border vectors to several clusters). For each point:
 * idx[n][0], idx[n][1] = the two components with the largest s_nk (ties go to
 * the lower index) and resp[n][.] = their r_nk, normalised over all K. With
 * K = 1, idx[n][1] = -1 and resp[n][1] = 0. idx is N x 2 int32, resp N x 2 float. */
int gmm_assign_top2(const void* X, int32_t x_dtype, int64_t N, int32_t d,
                    const float* mu, const float* var, const float* logw, int32_t K,
                    int32_t* idx, float* resp, void* workspace, size_t ws_bytes, void* stream);

/* Row-chunked E-step for X that stays in HOST memory (Flash-GMM abstract:
 * datasets far larger than one GPU holds; the statistics are additive over
 * rows, so they are accumulated chunk by chunk). X_host is a host pointer
 * to the same row-major N x d layout; best pinned (hipHostMalloc or a pinned
 * torch tensor), since pageable memory cannot overlap its copies. Rows go
 * to the device chunk_rows at a time through two staging buffers in the
 * workspace: the copy of chunk i+1 runs on a library-owned copy stream
 * (one per device, created on first use, default priority) while chunk i is
 * scored on `stream`. Per chunk the E-step is the one of gmm_estep_stats
 * (AUTO regime); the chunks' statistics and log-likelihoods are summed in
 * fp64 in chunk order, so results are deterministic for a given chunk_rows
 * and agree with gmm_estep_stats to rounding. Outputs are device pointers as
 * in gmm_estep_stats; loglik_point (nullable) gets all N values.
 * The workspace must hold gmm_workspace_bytes_chunked(N, d, K, chunk_rows,
 * x_dtype) bytes. X_host must stay valid and unmodified until `stream` has
 * completed. Calls on one device are serialised by the library while they
 * enqueue; callers must not reuse a workspace on two streams at once.
 * chunk_rows >= 1 (values above N are treated as N). */
int gmm_estep_stats_chunked(const void* X_host, int32_t x_dtype, int64_t N, int32_t d,
                            const float* mu, const float* var, const float* logw, int32_t K,
                            float* Nk, float* Sx, float* Sxx,
                            double* loglik_total, float* loglik_point, int64_t chunk_rows,
                            void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes for gmm_estep_stats_chunked; 0 for arguments outside the
 * limits (or chunk_rows < 1, unknown x_dtype). */
size_t gmm_workspace_bytes_chunked(int64_t N, int32_t d, int32_t K, int64_t chunk_rows, int32_t x_dtype);

/* Inverted lists with border vectors from a top-2 assignment (Flash-GMM
 * abstract: a soft coarse quantizer assigns vectors near cluster borders to
 * several clusters). idx and resp are the N x 2 outputs of gmm_assign_top2
 * (device): point n is listed under idx[n][0] (which must lie in [0, K)) and,
 * when idx[n][1] >= 0 and resp[n][1] >= border_threshold, also under
 * idx[n][1]. Outputs (device): offsets, K + 1 int64 (list k is
 * members[offsets[k] .. offsets[k+1]), offsets[K] = number of entries) and
 * members, int32 point indices, increasing within each list. The result is
 * a pure function of the inputs (no atomics decide any order).
 * idx must be 8-byte aligned. members_capacity must be >= 2N; N < 2^31. The workspace must hold
 * gmm_border_lists_workspace_bytes(N, K) bytes, 256-byte aligned. */
int gmm_border_lists(const int32_t* idx, const float* resp, int64_t N, int32_t K, float border_threshold,
                     int64_t* offsets, int32_t* members, int64_t members_capacity,
                     void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes for gmm_border_lists; 0 for arguments outside the limits. */
size_t gmm_border_lists_workspace_bytes(int64_t N, int32_t K);

/* Lloyd's k-means on the same machinery (Flash-KMeans articles: a fused
 * assignment that never writes the N x K distance matrix, and a centroid
 * update that sorts points by cluster id and reduces contiguous segments
 * instead of scattering with atomics). C is K x d float (device), X as in
 * gmm_estep_stats; N < 2^31. The workspace must hold
 * gmm_kmeans_workspace_bytes(N, d, K) bytes, 256-byte aligned.
 *
 * gmm_kmeans_assign: assign[n] = argmin_k ||x_n - c_k||^2 (ties to the lower
 * index). fp32 matrix-core scores select, per row, every centre that the
 * fp32 rounding bound cannot rule out; those get exact fp64 distances
 * (difference form) and decide. dist2[n] (nullable) is the minimum squared
 * distance rounded to float; *inertia (nullable, device double) the fp64 sum
 * of the unrounded minima. */
int gmm_kmeans_assign(const void* X, int32_t x_dtype, int64_t N, int32_t d, const float* C, int32_t K,
                      int32_t* assign, float* dist2, double* inertia,
                      void* workspace, size_t ws_bytes, void* stream);

/* gmm_kmeans_update: C[k] (in/out) becomes the mean of the points with
 * assign[n] == k, summed in fp64 (each cluster's points in point order, cut
 * into fixed segments whose length depends on N and on how many blocks the
 * device holds at once, so results repeat exactly on one device model); a
 * centre with no points keeps its value. counts (nullable, K int64)
 * receives the cluster sizes. assign[n] must lie in [0, K). */
int gmm_kmeans_update(const void* X, int32_t x_dtype, int64_t N, int32_t d, const int32_t* assign, int32_t K,
                      float* C, int64_t* counts, void* workspace, size_t ws_bytes, void* stream);

/* `iters` Lloyd iterations on the device (assign, then update); inertia_hist
 * (device, iters doubles) receives the inertia of the centres before each
 * update. C is in/out. Needs N >= 1. */
int gmm_kmeans_iterate(const void* X, int32_t x_dtype, int64_t N, int32_t d, int32_t K, int32_t iters,
                       float* C, double* inertia_hist, void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes for the k-means entry points; 0 outside the limits. */
size_t gmm_kmeans_workspace_bytes(int64_t N, int32_t d, int32_t K);

#ifdef __cplusplus
}
#endif

#endif /* GMM_MI355X_H */
