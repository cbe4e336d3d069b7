// Internal declarations shared by the host API and the kernel translation unit.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gmm {

constexpr int kTileN = 64;           // points per tile (two 32-row MFMA blocks)
constexpr int kCompTile = 32;        // components per wave in the fp32 kernels
constexpr int kCompTile64 = 16;      // components per fp64 MFMA tile
constexpr int kMaxD = 128;
constexpr int kMaxK = 65536;
constexpr int kSlabWaves = 8;        // waves (x32 components) per two-pass slab
constexpr int kSingleMaxK = 256;     // largest K the single sweep keeps on chip
constexpr int kSmallMaxK = 16;       // small-K kernel: one 16-component tile
constexpr int kSmallMaxD = 64;
constexpr int kLseWaves = 4;         // waves per block in the fp64 normaliser pass
constexpr int kSmallWaves = 4;       // waves per block in the small-K kernel
constexpr int64_t kMaxChunkRows = 32768;  // rows per statistics partial, at most
constexpr int kCandT = 8;            // candidates kept per (row, slab) by the fp32 first pass
constexpr int kSlabSegs = 256;       // tile segments per slab in the build of the second pass's row lists
constexpr int kLlRows = 1024;        // rows per log-likelihood partial in the two-pass regime

// Device pointers into the caller's workspace, filled by gmm::plan().
struct Workspace {
  float* W32p;      // fp32 score operands, packed for the 32x32x2 MFMA B operand
  float* c32;       // [Kp32] expanded-form score constant (fp32), -inf for padding
  double* W64p;     // fp64 score operands, packed for the 16x16x4 f64 MFMA A operand
  double* c64e;     // [Kp16] expanded-form constant (fp64), -inf for padding
  double* iv64;     // [K][d] 1/var in fp64 (exact re-score)
  double* c64d;     // [K] difference-form constant (fp64)
  float* mup;       // [Kp][DP] means, zero padded (exact re-score of the fp32 kernels)
  double* ivp;      // [Kp][DP] 1/var in fp64, zero padded
  float* compmax;   // [K][4] per-component max|A|, max|B|, |c|, ||B||_2 (error bound inputs)
  float* errc;      // [4] a_max, b_max, c_max, b2_max
  float4* rowref;   // [N] per-row (m, lZ, theta, E) for the second pass (base 2)
  // fp32 first pass of the two-pass regime (Plan::pass1):
  float4* p1h;      // [kslabs][N] per (row, slab): z, slab max, capture threshold, candidate count
  float* p1v;       // [kslabs][N][kCandT] candidate scores (base 2, fp32)
  uint8_t* p1k;     // [kslabs][N][kCandT] their components within the slab
  float* rowE;      // [N] per-row fp32 score error bound E (natural units)
  double* lrow;     // [N] per-row l_n (natural), before the block sums
  int32_t* fblist;  // [N] rows whose normaliser needs the fp64 pass
  int32_t* fbcount; // [1] number of such rows
  int32_t* xflag;   // [1] (beside fbcount) set when some row's |x|^2 >= 225 (xrange_kernel)
  // row lists of the second pass (two-pass regime, Plan::pass1):
  float* rowSq;     // [N] |x|^2 of each row (fp32, from the first pass)
  int32_t* slist;   // [kslabs][N] per slab, in increasing order, the rows it keeps
  uint64_t* smask;  // [kslabs][tiles] per 64-row tile, the kept rows as a bit mask
  int32_t* soff;    // [kslabs][tiles] kept rows per tile
  int32_t* sseg;    // [kslabs][kSlabSegs] kept rows per tile segment, then their exclusive prefix
  int32_t* slen;    // [kslabs] length of each slab's list
  float* partials;  // [P][Kp][E] per-chunk statistics
  double* llpart;   // [max(P, tiles)] per-block log-likelihood sums
  float* stats;     // [K][1 + 2d] Nk | Sx | Sxx scratch for the EM loop
  double* redtmp;   // [G][K (1 + 2d)] segment sums of the two-stage statistics reduction (G > 1)
};

struct Plan {
  int64_t N;
  int d, K;
  int DT, DP;       // DP >= d: padded feature count (32*DT; 16-multiple for small-K)
  int regime;       // 1 single, 2 two-pass, 3 small-K
  int waves;        // waves per block in the statistics kernel
  int kslabs;       // component slabs (1 for the single sweep)
  int Kp;           // padded K of the statistics kernel = 32*waves*kslabs
  int Kp16;         // K rounded up to 16 (fp64 pass)
  int64_t P;        // row chunks of the statistics kernel
  int G;            // partial segments of the statistics reduction (1: one stage)
  int64_t rows_per_chunk;
  int64_t tiles;    // ceil(N / 64)
  int E;            // 1 + 2*DP floats per component in a partial
  int stats_split;  // statistics contraction as split-bf16 products on the bf16 MFMA
  int stats_f16;    // half-precision X: the second pass's statistics as exact fp16 splits
  int pass1;        // two-pass regime with the fp32 first pass (its record regions are laid out)
  float drop_rho;   // statistics skip threshold rho = 2^-20 / (rows of the whole E-step)
  size_t bytes;     // workspace bytes this plan uses
  Workspace ws;
};

// Fills `plan` (and the workspace pointers when base != nullptr). Returns a
// gmm_status code; does not touch the GPU.
int make_plan(int64_t N, int d, int K, int regime, void* base, Plan* plan);
// The same without the first-pass record regions of the two-pass regime
// (for the passes that only use the packed parameters: top-2, k-means).
int make_plan_params(int64_t N, int d, int K, int regime, void* base, Plan* plan);

// Kernel launchers (gmm_kernels.hip). All enqueue on `stream` and return a
// hipError_t from hipGetLastError().
hipError_t launch_precompute(const Plan& p, const float* mu, const float* var, const float* logw,
                             hipStream_t stream);
// One-shot timing events recorded around the fused E-step kernel(s) of the
// next launch_estep on this thread (see gmm_set_timing_events).
void set_timing_events(hipEvent_t start, hipEvent_t stop);

hipError_t launch_estep(const Plan& p, const void* X, int x_dtype, const float* mu,
                        float* Nk, float* Sx, float* Sxx, double* loglik_total,
                        float* loglik_point, float* R, hipStream_t stream);
// Row-chunked E-step: one chunk's statistics and log-likelihood are added to
// the fp64 accumulators acc[K * (1 + 2d) + 1] (set instead when `first`).
hipError_t launch_estep_accum(const Plan& p, const void* X, int x_dtype, const float* mu, double* acc, int first,
                              float* loglik_point, hipStream_t stream);
hipError_t launch_finalize_stats(const double* acc, int K, int d, float* Nk, float* Sx, float* Sxx,
                                 double* loglik_total, hipStream_t stream);
hipError_t launch_top2(const Plan& p, const void* X, int x_dtype, int32_t* idx, float* resp,
                       hipStream_t stream);
// Border-vector inverted lists (gmm_lists.hip): workspace layout and launcher.
struct ListsLayout {
  int64_t blocks_a, blocks_b;  // blocks of the pass over the points, and of the second pass (0: none)
  size_t o_H, o_O, o_total, o_S, o_keys, o_tmp_keys, o_tmp_vals, bytes;
};
ListsLayout lists_layout(int64_t N, int K);
hipError_t launch_border_lists(const int32_t* idx, const float* resp, int64_t N, int K, float thr,
                               int64_t* offsets, int32_t* members, void* workspace, hipStream_t stream);
// Lloyd's k-means: nearest-centre assignment on the fp32 score tile with an
// exact fp64 distance check of the centres the fp32 error bound cannot rule
// out (the plan's parameters packed from centres, unit variances, zero
// log-weights); dist2 and inertia (sum of the minima) are nullable.
hipError_t launch_kmeans_assign(const Plan& p, const void* X, int x_dtype, int32_t* assign, float* dist2,
                                double* inertia, hipStream_t stream);
hipError_t launch_fill(float* a, int64_t n, float v, hipStream_t stream);
// k-means update from the lists of a hard assignment (gmm_lists.hip).
int64_t kmeans_max_segments(int64_t N, int K);
hipError_t launch_kmeans_update(const void* X, int x_dtype, int64_t N, int d, int K, const int64_t* offsets,
                                const int32_t* members, int32_t* seg, int64_t* segoff, int64_t* scan_tmp,
                                double* part, int64_t max_segments, float* C, int64_t* counts,
                                hipStream_t stream);
hipError_t launch_mstep(const float* Nk, const float* Sx, const float* Sxx, int64_t N, int d, int K,
                        float var_floor, float* mu, float* var, float* logw, hipStream_t stream);
hipError_t launch_zero_outputs(float* Nk, float* Sx, float* Sxx, int d, int K,
                               double* loglik_total, hipStream_t stream);

}  // namespace gmm
