// HIP kernels for the fused Gaussian-mixture EM E-step on gfx950 (MI355X).
//
// What is computed (Turbo-GMM abstract; Flash-GMM abstract): for N points and
// K diagonal Gaussian components, the score s_nk = log w_k + log N(x_n|mu_k,
// var_k), the row normaliser l_n = logsumexp_k s_nk, the responsibilities
// r_nk = exp(s_nk - l_n) and the statistics Nk, Sx = sum r x, Sxx = sum r x^2,
// with r kept on chip (never written to HBM).
//
// Score contraction. With A_kj = -1/(2 var_kj), B_kj = mu_kj/var_kj and
// c_k = log w_k - 1/2 (d log 2pi + sum_j log var_kj + sum_j mu_kj^2/var_kj),
//     s_nk = sum_j (A_kj x_nj^2 + B_kj x_nj) + c_k,
// a dense (N x 2d) . (2d x K) product that runs on MFMA tiles. The 32x32
// fp32 tiles pair two features in an MFMA step (the x^2 steps of a feature
// block, then its x steps), so each lane squares only the x values it holds;
// the 16x16 tiles interleave x^2 and x of one feature per step.
//
// Precision. FP32 accumulation of the expanded form loses ~1e-4 absolute on
// scores of magnitude ~10^2, which is too coarse for responsibilities near
// 0.5. Each row therefore carries an a-priori bound E_n on the fp32 score
// error, and the entries whose responsibility that error could move by more
// than a small tau are re-scored exactly (fp64, difference form) before the
// normalisation: with l_n from the same fp32 scores (single sweep, small K)
// those with 2 E_n r (1 - r) > tau, widened to every component within 20 of
// the row maximum when the unrefined mass could still matter; with the
// first pass's l_n (two-pass regime) those its merge step chose. The
// fp32 operands are scaled by log2(e), so scores come out in base 2 and every
// exponential is one hardware exp2.
//
// Regimes (Turbo-GMM abstract): the single sweep keeps the whole component
// axis of a 64-point tile on chip (K <= 256) and does max, log-sum-exp and
// statistics in one traversal. The two-pass fallback computes l_n first: an
// fp32 pass per 256-component slab records each slab's maximum, sum of
// exponentials and a few candidate entries per row; a merge per row decides
// which entries must be exact for l_n (and for the second pass) and
// re-scores them in fp64; rows it cannot settle from the records get an
// fp64-MFMA normaliser pass. The second pass recomputes the same fp32 scores
// per slab, re-scores the same entries, and accumulates the statistics. A
// small-K kernel (K <= 16, d <= 64) gives each wave its own rows and keeps
// the whole mixture in registers.
//
// Lloyd's k-means assignment (Flash-KMeans articles) reuses the fp32 score
// tile: with unit variances the highest score is the nearest centre, and the
// fp32 error bound limits the exact fp64 distance check to the centres that
// rounding could have put first.
#include "gmm_device.hpp"
#include "gmm_internal.hpp"

#include <atomic>
#include <type_traits>
#include <algorithm>
#include <limits.h>
#include <math.h>

namespace gmm {

typedef float v32f __attribute__((ext_vector_type(32)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef double v4d __attribute__((ext_vector_type(4)));

constexpr double kLog2Pi = 1.83787706640934548356065947281;
constexpr double kLog2E = 1.44269504088896340735992468100;  // 1 / ln 2
constexpr double kLn2 = 0.693147180559945309417232121458;
// The window of the fallback rule: components with s >= max - 20, i.e.
// e = exp(s - max) >= exp(-20).
constexpr float kExpWindow = 2.0611536e-9f;
// tau: the largest change of a responsibility that the fp32 score error may
// cause in an entry left unrefined (20x below the 1e-5 bar).
constexpr float kGateTau = 5e-7f;
// Per-operation relative error assumed for fp32 arithmetic in the bound below:
// 2^-23, which also covers an accumulator that truncates rather than rounds.
constexpr float kUnitRound = 1.1920928955078125e-7f;
// The error bound's inputs (|x|^2 and |x|_1 of a row, summed in fp32 over at
// most 2 * 128 nonnegative terms) and its own fp32 evaluation are each off by
// less than 300 u relative; this factor (> 1 + 2000 u) keeps the computed
// bound an upper bound.
constexpr float kBoundSlack = 1.0005f;
constexpr int kRefCap = 128;       // re-score list entries per wave and pass
// Widest candidate window of the fp32 first pass (base-2 units below the
// slab maximum): wider than the 20-nat window (28.9 base-2 units) beyond
// which an entry's weight is below e^-20 of the row maximum's.
constexpr float kCapWin = 32.f;
// Candidate windows of the first pass, loosest first (base-2 units below the
// slab maximum); the last, 0, admits only the entries equal to the maximum.
constexpr int kCapLevels = 13;
__constant__ float kCapLadder[kCapLevels] = {kCapWin, 26.f, 22.f, 19.f, 17.f, 15.f, 13.f, 11.f, 9.f,
                                             7.f, 5.f, 3.f, 0.f};
// 2^-W for each level W of kCapLadder (compile-time constants).
constexpr float kCapQ[kCapLevels] = {0x1p-32f, 0x1p-26f, 0x1p-22f, 0x1p-19f, 0x1p-17f, 0x1p-15f, 0x1p-13f,
                                     0x1p-11f, 0x1p-9f,  0x1p-7f,  0x1p-5f,  0x1p-3f,  1.f};
// Word 3 of a raw buffer resource on CDNA (32-bit data format, no swizzle):
// loads at offsets past the record count return zero.
constexpr int kBufferRsrcWord3 = 0x00020000;

// v = hi + lo + d for eight fp32 values: hi and lo round to nearest bf16, so
// |lo| <= 2^-8 |v| and |d| <= 2^-16 |v|.
__device__ __forceinline__ void split_bf16(const float (&v)[8], v8bf& hi, v8bf& lo) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    hi[t] = (__bf16)v[t];
    lo[t] = (__bf16)(v[t] - (float)hi[t]);
  }
}

// The smallest float above a finite x.
__device__ __forceinline__ float next_up(float x) {
  if (x == 0.f) return __int_as_float(1);
  const int b = __float_as_int(x);
  return __int_as_float(x > 0.f ? b + 1 : b - 1);
}

// Row of the 32x32 MFMA accumulator held in slot j by lanes of half h:
// D[row][col] with col = lane % 32 and row = 8*(j/4) + 4*h + j%4.
__device__ __forceinline__ int acc_row(int h, int j) { return ((j >> 2) << 3) + (h << 2) + (j & 3); }

// Orders this wave's LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename XT>
__device__ __forceinline__ float load_x(const XT* X, int64_t i) { return (float)X[i]; }

// A double moved between lanes by a DPP lane permutation within each row of
// 16 lanes (two 32-bit moves).
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xffffffffll), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// DPP lane permutations within a row of 16 lanes: quad xor 1, quad xor 2, the
// mirror within each half row (i <-> 7 - i) and the mirror of the whole row
// (i <-> 15 - i). Applied in this order as add steps they leave every lane of
// an aligned group of 8 (16) with the group's sum (the quad sums, the half-row
// sums, then the two halves joined), bitwise identical on all of its lanes
// (the last step adds the same two values in either order).
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

// All-reduce over aligned groups of tpr consecutive lanes (tpr a power of two
// <= 16) with the DPP steps above; every lane of a group ends with the same
// value.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float group_max(float v, int tpr) {
  if (tpr > 1) v = fmaxf(v, dpp_f<kDppXor1>(v));
  if (tpr > 2) v = fmaxf(v, dpp_f<kDppXor2>(v));
  if (tpr > 4) v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  if (tpr > 8) v = fmaxf(v, dpp_f<kDppMirror>(v));
  return v;
}
__device__ __forceinline__ float group_sum(float v, int tpr) {
  if (tpr > 1) v += dpp_f<kDppXor1>(v);
  if (tpr > 2) v += dpp_f<kDppXor2>(v);
  if (tpr > 4) v += dpp_f<kDppHalfMirror>(v);
  if (tpr > 8) v += dpp_f<kDppMirror>(v);
  return v;
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t group_or(uint32_t v, int tpr) {
  if (tpr > 1) v |= dpp_u<kDppXor1>(v);
  if (tpr > 2) v |= dpp_u<kDppXor2>(v);
  if (tpr > 4) v |= dpp_u<kDppHalfMirror>(v);
  if (tpr > 8) v |= dpp_u<kDppMirror>(v);
  return v;
}
// Inclusive prefix sum over aligned groups of tpr consecutive lanes (tpr a
// power of two <= 16): DPP row shifts by 1, 2, 4, 8; a lane adds the shifted
// value only when its source lies in its own group.
__device__ __forceinline__ int group_incl_scan(int v, int sub, int tpr) {
  int t = __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  if (tpr > 1 && sub >= 1) v += t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  if (tpr > 2 && sub >= 2) v += t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  if (tpr > 4 && sub >= 4) v += t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  if (tpr > 8 && sub >= 8) v += t;
  return v;
}
__device__ __forceinline__ double group_sum_d(double v, int tpr) {
  if (tpr > 1) v += dpp_d<kDppXor1>(v);
  if (tpr > 2) v += dpp_d<kDppXor2>(v);
  if (tpr > 4) v += dpp_d<kDppHalfMirror>(v);
  if (tpr > 8) v += dpp_d<kDppMirror>(v);
  return v;
}

// Asynchronous fp32 tile load: rows [r0, r0 + 64) of X -> LDS tile [64][XS]
// with 16-byte global->LDS loads. One wave instruction fills 1 KB of LDS, i.e.
// 64 consecutive 16-byte chunks of the padded row-major tile, so the tile is
// XS/4 instructions spread over the waves. Chunks outside the data (the row
// padding, features d..DP-1, rows past `hi`) receive finite filler copied
// from a valid row: they only ever meet zero weights or r = 0.
// With `rows` (a row list), tile positions [r0, r0 + 64) name rows
// rows[r0 .. r0 + 63] instead (positions past `hi` take the last listed row).
template <int XS>
__device__ __forceinline__ void async_x_tile(float* xn, const float* X, int64_t r0, int64_t hi, int d,
                                             int wave, int waves, int lane, const int32_t* rows) {
  constexpr int CPR = XS / 4;  // 16-byte chunks per LDS row
  for (int j = wave; j < CPR; j += waves) {
    const int ch = 64 * j + lane;
    const int row = ch / CPR, slot = ch - row * CPR;
    const int64_t pos = r0 + row < hi ? r0 + row : hi - 1;
    const int64_t gr = rows ? (int64_t)rows[pos] : pos;
    const int q = 4 * slot < d ? slot : 0;
    __builtin_amdgcn_global_load_lds(X + gr * d + 4 * q,
                                     reinterpret_cast<__attribute__((address_space(3))) void*>(
                                         reinterpret_cast<uintptr_t>(xn + 256 * j)),
                                     16, 0, 0);
  }
}

// Rows [r0, r0 + 64) of X -> LDS tile [64][XS], zero padded to DP features
// and past `hi`. `vec`: 1 = 16-byte aligned float rows (d % 4 == 0), 2 =
// 16-byte aligned half-precision rows (d % 8 == 0).
// With `rows`, positions name listed rows as in async_x_tile.
template <int XS, typename XT>
__device__ __forceinline__ void load_x_tile(float* xs, const XT* X, int64_t r0, int64_t hi, int d, int DP,
                                            int tid, int nthr, int vec, const int32_t* rows = nullptr) {
  if (vec && sizeof(XT) == 4) {
    const float* Xf = reinterpret_cast<const float*>(X);
    for (int ch = tid; ch < 16 * DP; ch += nthr) {
      const int row = ch / (DP / 4), q = ch - row * (DP / 4);
      const int64_t pos = r0 + row;
      const int64_t gr = pos < hi && rows ? (int64_t)rows[pos] : pos;
      *reinterpret_cast<float4*>(xs + row * XS + 4 * q) =
          (pos < hi && 4 * q < d) ? *reinterpret_cast<const float4*>(Xf + gr * d + 4 * q)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  } else if (vec == 2 && sizeof(XT) == 2) {
    // half-precision rows of d % 8 == 0 values, 16-byte aligned: eight values
    // per load, widened into two float4
    for (int ch = tid; ch < 8 * DP; ch += nthr) {
      const int row = ch / (DP / 8), q = ch - row * (DP / 8);
      const int64_t pos = r0 + row;
      const int64_t gr = pos < hi && rows ? (int64_t)rows[pos] : pos;
      const uint4 raw = (pos < hi && 8 * q < d) ? *reinterpret_cast<const uint4*>(X + gr * d + 8 * q)
                                                 : make_uint4(0u, 0u, 0u, 0u);
      const XT* hv = reinterpret_cast<const XT*>(&raw);
      *reinterpret_cast<float4*>(xs + row * XS + 8 * q) =
          make_float4((float)hv[0], (float)hv[1], (float)hv[2], (float)hv[3]);
      *reinterpret_cast<float4*>(xs + row * XS + 8 * q + 4) =
          make_float4((float)hv[4], (float)hv[5], (float)hv[6], (float)hv[7]);
    }
  } else {
    for (int e = tid; e < 64 * DP; e += nthr) {
      const int row = e / DP, f = e - row * DP;
      const int64_t pos = r0 + row;
      const int64_t gr = pos < hi && rows ? (int64_t)rows[pos] : pos;
      xs[row * XS + f] = (pos < hi && f < d) ? load_x(X, gr * d + f) : 0.f;
    }
  }
}

// ---------------------------------------------------------------------------
// Parameter precompute (fp64 arithmetic)
// ---------------------------------------------------------------------------

// One wave per (padded) component: the score constants and the inputs of
// the fp32 error bound; lanes stride over the features and reduce in a fixed
// order.
__global__ void comp_consts_kernel(const float* __restrict__ mu, const float* __restrict__ var,
                                   const float* __restrict__ logw, int K, int d, int Kp, int Kp16,
                                   float* __restrict__ c32, double* __restrict__ c64e,
                                   double* __restrict__ c64d, float* __restrict__ compmax) {
  const int k = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (k >= Kp) return;
  if (k >= K) {
    if (lane == 0) {
      c32[k] = -INFINITY;
      if (k < Kp16) c64e[k] = -INFINITY;
    }
    return;
  }
  double slv = 0.0, sm2 = 0.0, amax = 0.0, bmax = 0.0, b2 = 0.0;
  for (int j = lane; j < d; j += 64) {
    const double v = var[(size_t)k * d + j], m = mu[(size_t)k * d + j];
    const double iv = 1.0 / v;
    slv += log(v);
    sm2 += m * m * iv;
    amax = fmax(amax, 0.5 * iv);
    bmax = fmax(bmax, fabs(m * iv));
    b2 += (m * iv) * (m * iv);
  }
  for (int o = 32; o > 0; o >>= 1) {
    slv += __shfl_xor(slv, o, 64);
    sm2 += __shfl_xor(sm2, o, 64);
    b2 += __shfl_xor(b2, o, 64);
    amax = fmax(amax, __shfl_xor(amax, o, 64));
    bmax = fmax(bmax, __shfl_xor(bmax, o, 64));
  }
  if (lane == 0) {
    const double cd = (double)logw[k] - 0.5 * ((double)d * kLog2Pi + slv);
    const double ce = cd - 0.5 * sm2;
    c64d[k] = cd;
    c64e[k] = ce;
    c32[k] = (float)(ce * kLog2E);  // base 2: the fp32 pass evaluates 2^(s / ln 2)
    compmax[4 * k + 0] = (float)amax;
    compmax[4 * k + 1] = (float)bmax;
    compmax[4 * k + 2] = isfinite(ce) ? (float)fabs(ce) : 0.0f;
    compmax[4 * k + 3] = (float)sqrt(b2);
  }
}

// One thread per (component, feature) over Kp x DP: packed MFMA operands.
//  W32p: float4 index (kt*Q + q)*64 + lane, lane = 32*h + c, holds features
//        4q..4q+3 of component 32*kt + c; h = 0 -> A, h = 1 -> B.
//  W64p: double index ((kt*S + s)*4 + g)*16 + c holds feature 2s + g/2 of
//        component 16*kt + c; g even -> A, g odd -> B.
//  mup, ivp: [Kp][DP] mean and 1/var, zero past d and K (aligned rows for the
//        exact re-score of the fp32 kernels).
__global__ void pack_kernel(const float* __restrict__ mu, const float* __restrict__ var, int K, int d,
                            int Kp, int Kp16, int DP, float* __restrict__ W32p,
                            double* __restrict__ W64p, double* __restrict__ iv64,
                            float* __restrict__ mup, double* __restrict__ ivp) {
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t >= (int64_t)Kp * DP) return;
  const int k = (int)(t / DP), f = (int)(t - (int64_t)k * DP);
  double A = 0.0, B = 0.0, iv = 0.0;
  float m = 0.f;
  if (k < K && f < d) {
    const float v = var[(size_t)k * d + f];
    iv = 1.0 / (double)v;
    m = mu[(size_t)k * d + f];
    A = -0.5 * iv;
    B = (double)m * iv;
    iv64[(size_t)k * d + f] = iv;
  }
  mup[t] = m;
  ivp[t] = iv;
  {
    // fp32 score operands, base-2 scaled like c32: lane (h, c) of feature
    // block q (features 4q..4q+3) holds A of features 4q + 2h + {0, 1} in
    // slots 0-1 (the x^2 steps) and their B in slots 2-3 (the x steps)
    const int kt = k >> 5, c = k & 31, q = f >> 2, h = (f >> 1) & 1, u = f & 1, Q = DP >> 2;
    const size_t base = (((size_t)kt * Q + q) * 64 + 32 * h + c) * 4 + u;
    W32p[base] = (float)(A * kLog2E);
    W32p[base + 2] = (float)(B * kLog2E);
  }
  if (k < Kp16) {
    // 16x16x4 f64 MFMA A operand of 16-component tile kt: lane (g, c) of step
    // 2j holds A of feature 4j + g of component c (the x^2 step), of step
    // 2j + 1 its B (the x step)
    const int kt = k >> 4, c = k & 15, j = f >> 2, g = f & 3, S = DP >> 1;
    const size_t base = (((size_t)kt * S + 2 * j) * 4 + g) * 16 + c;
    W64p[base] = A;
    W64p[base + 64] = B;
  }
}

// One block: global maxima of the per-component error-bound inputs
// errc = {max |A_kj|, max |B_kj|, max |c_k|, max_k ||B_k||_2}.
__global__ void errc_kernel(const float* __restrict__ compmax, int K, float* __restrict__ errc) {
  __shared__ float s[4][256];
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k = threadIdx.x; k < K; k += blockDim.x)
    for (int i = 0; i < 4; ++i) v[i] = fmaxf(v[i], compmax[4 * k + i]);
  for (int i = 0; i < 4; ++i) s[i][threadIdx.x] = v[i];
  __syncthreads();
  for (int o = blockDim.x / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o)
      for (int i = 0; i < 4; ++i) s[i][threadIdx.x] = fmaxf(s[i][threadIdx.x], s[i][threadIdx.x + o]);
    __syncthreads();
  }
  if (threadIdx.x < 4) errc[threadIdx.x] = s[threadIdx.x][0];
}

// Score tile of one wave: s_k(x) - c_k = sum_j (A_kj x_j^2 + B_kj x_j) for the
// 64 rows of the LDS tile `xs` and the wave's 32 components (operands W from
// the buffer resource `wrs`), on two 32x32x2 fp32 MFMA accumulators (rows
// 0-31 in acc0, 32-63 in acc1; score_store adds c_k and writes them to the
// wave's 32 columns of an LDS score tile); with NORMS wave 0 also writes
// |x|^2 and |x|_1 of each row to `xq` (inputs of the error bound), from the
// squares the MFMAs consume.
template <int DT, bool NORMS>
__device__ __forceinline__ void score_acc(const float* xs, float* xq, __amdgpu_buffer_rsrc_t wrs, int wave,
                                          int lane, v16f& acc0, v16f& acc1) {
  constexpr int DP = 32 * DT, Q = DP / 4, XS = DP + 4;
  const int h = lane >> 5, c = lane & 31;
  auto wload = [&](int q) { return __builtin_amdgcn_raw_buffer_load_b128(wrs, (q * 64 + lane) * 16, 0, 0); };
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    acc0[j] = 0.f;
    acc1[j] = 0.f;
  }
  // Score operands (L2-resident) are prefetched two steps ahead in two
  // register pairs that swap roles every two steps, so the loop needs no
  // register rotation (which would wait for the loads in flight).
  // Feature block q takes four MFMAs per row half: the two k slots of the
  // 32x32x2 MFMA are features 4q + 2h + u of lanes h = 0 and h = 1, first as
  // x^2 (u = 0, 1), then as x; each lane squares only its own two features.
  float sq0 = 0.f, sq1 = 0.f, ab0 = 0.f, ab1 = 0.f;  // error-bound inputs over this lane's features
  auto xld = [&](int q, float2& x0, float2& x1) {
    x0 = *reinterpret_cast<const float2*>(xs + c * XS + 4 * q + 2 * h);
    x1 = *reinterpret_cast<const float2*>(xs + (c + 32) * XS + 4 * q + 2 * h);
  };
  auto step = [&](const float2& x0, const float2& x1, v4f w) {
    const float s00 = x0.x * x0.x, s01 = x0.y * x0.y, s10 = x1.x * x1.x, s11 = x1.y * x1.y;
    acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(s00, w[0], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(s10, w[0], acc1, 0, 0, 0);
    acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(s01, w[1], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(s11, w[1], acc1, 0, 0, 0);
    acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(x0.x, w[2], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(x1.x, w[2], acc1, 0, 0, 0);
    acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(x0.y, w[3], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(x1.y, w[3], acc1, 0, 0, 0);
    if constexpr (NORMS) {
      sq0 += s00 + s01;  // rows c and c + 32
      sq1 += s10 + s11;
      ab0 += fabsf(x0.x) + fabsf(x0.y);
      ab1 += fabsf(x1.x) + fabsf(x1.y);
    }
  };
  // The X operands of the next step are read from LDS before this step's
  // MFMAs issue; the scheduling barriers keep every load where it is.
  static_assert(Q % 4 == 0, "the score loop takes four steps at a time");
  v4f wa = wload(0), wb = wload(1);
  float2 pa0, pa1, pb0, pb1;
  xld(0, pa0, pa1);
#pragma unroll 1
  for (int q = 0; q < Q; q += 4) {
    const v4f wc = wload(q + 2), wd = wload(q + 3);
    xld(q + 1, pb0, pb1);
    __builtin_amdgcn_sched_barrier(0);
    step(pa0, pa1, wa);
    __builtin_amdgcn_sched_barrier(0);
    xld(q + 2, pa0, pa1);
    __builtin_amdgcn_sched_barrier(0);
    step(pb0, pb1, wb);
    __builtin_amdgcn_sched_barrier(0);
    wa = wload(q + 4 < Q ? q + 4 : 0);
    wb = wload(q + 5 < Q ? q + 5 : 1);
    xld(q + 3, pb0, pb1);
    __builtin_amdgcn_sched_barrier(0);
    step(pa0, pa1, wc);
    __builtin_amdgcn_sched_barrier(0);
    xld(q + 4 < Q ? q + 4 : 0, pa0, pa1);
    __builtin_amdgcn_sched_barrier(0);
    step(pb0, pb1, wd);
  }
  if (NORMS && wave == 0) {
    // the two halves of the wave hold the two halves of each row's features
    sq0 += __shfl_xor(sq0, 32, 64);
    sq1 += __shfl_xor(sq1, 32, 64);
    ab0 += __shfl_xor(ab0, 32, 64);
    ab1 += __shfl_xor(ab1, 32, 64);
    if (h == 0) {
      xq[2 * c] = sq0;
      xq[2 * c + 1] = ab0;
      xq[2 * (c + 32)] = sq1;
      xq[2 * (c + 32) + 1] = ab1;
    }
  }
}

// One 32-row accumulator of score_acc, plus the component constants, to
// rows row0 .. row0 + 31 of the LDS score tile (row stride SCS).
__device__ __forceinline__ void score_store(float* sc, const v16f& acc, int row0, float ck, int wave, int lane,
                                            int SCS) {
  const int h = lane >> 5, c = lane & 31;
  // The store base goes through an empty asm so that the 16 store
  // addresses are formed here, per tile, instead of being hoisted out of
  // the tile loop and held (or spilled) across it.
  int scb = (4 * h + row0) * SCS + wave * 32 + c;
  asm volatile("" : "+v"(scb));
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = ((j >> 2) << 3) + (j & 3);  // acc_row(h, j) - 4 h
    sc[scb + r * SCS] = acc[j] + ck;
  }
}

// Scores of a 64-row X tile against the wave's 32 components into the LDS
// score tile [64][SCS] (see score_acc), with NORMS |x|^2 and |x|_1 of the
// rows into xq.
template <int DT, bool NORMS>
__device__ __forceinline__ void score_tile(const float* xs, float* sc, float* xq, __amdgpu_buffer_rsrc_t wrs,
                                           float ck, int wave, int lane, int SCS) {
  v16f acc0, acc1;
  score_acc<DT, NORMS>(xs, xq, wrs, wave, lane, acc0, acc1);
  score_store(sc, acc0, 0, ck, wave, lane, SCS);
  score_store(sc, acc1, 32, ck, wave, lane, SCS);
}

// |x|^2 and |x|_1 of row `row` of an LDS X tile (row stride XS, features past
// d not read), summed by the g consecutive lanes of the row's group: lane
// `sub` takes the 16-byte chunks sub, sub + g, ...; every lane of the group
// ends with both sums. (A chunk that straddles d is read whole: the element
// loads of such rows leave zeros past d.)
template <int DP, int XS>
__device__ __forceinline__ void row_norms(const float* xs, int row, int sub, int g, int d, float& sq, float& ab) {
  sq = 0.f;
  ab = 0.f;
  for (int q = sub; q < DP / 4 && 4 * q < d; q += g) {
    const float4 v = *reinterpret_cast<const float4*>(xs + row * XS + 4 * q);
    sq += (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
    ab += (fabsf(v.x) + fabsf(v.y)) + (fabsf(v.z) + fabsf(v.w));
  }
  sq = group_sum(sq, g);
  ab = group_sum(ab, g);
}

// ---------------------------------------------------------------------------
// Fused score kernel: the single sweep (MODE 0), and the first (MODE 2) and
// second (MODE 1) passes of the two-pass regime
// ---------------------------------------------------------------------------
//
// Block = `waves` waves; wave w owns components kw = k0 + 32w .. kw + 31 of
// its slab. The block walks the 64-point tiles of its row chunk (MODE 1: of
// its slab's row list):
//   1. X tile -> LDS (padded to DP features and 64 rows)
//   2. scores: two 32x32 fp32 MFMA accumulators per wave -> LDS score tile
//   3. row phase (`waves` threads per row): max, log-sum-exp (MODE 0) or the
//      row references (m, lZ, theta) of the merge (MODE 1), gated exact
//      re-score; the tile then holds e = exp(s - m) and a per-row 1/z
//      (MODE 0) or r itself (MODE 1). MODE 2 instead writes per (row, slab)
//      the slab's maximum, normaliser and candidates (p1_rows), a half tile
//      at a time, and stops there.
//   4. statistics: r of the wave's 32 components is the A operand, x and
//      x^2 the B operands of MFMAs that accumulate Sx and Sxx in registers:
//      in the single sweep one point per two-block 32x32x1 MFMA, skipping a
//      point whose 32 responsibilities are all at or below
//      rho / max(1, |x|^2); in the second pass every point of the listed
//      rows, two per 32x32x2 MFMA.
// At the end each block writes its statistics partial; a separate kernel
// sums the partials in a fixed order (no atomics anywhere).
// Outputs of the fp32 first pass (MODE 2), per (row, slab): see Pass1Out.
struct Pass1Out {
  float4* h;      // [kslabs][N] (z, slab max m, capture threshold th, candidate count)
  float* v;       // [kslabs][N][kCandT] candidate scores
  uint8_t* k;     // [kslabs][N][kCandT] candidate components within the slab
  float* rowE;    // [N] the row's fp32 score error bound (written by slab 0)
  float* rowSq;   // [N] the row's |x|^2 in fp32 (written by slab 0)
};

// The first pass (MODE 2) keeps one X tile and half a score tile in LDS and
// fits in 128 registers, so that two blocks share a CU and one block's row
// phase overlaps the other's score MFMAs.
// WV: the block's wave count when fixed at compile time (8, for slabs of 256
// components), 0 when it comes from `waves_rt`. With it fixed, the row
// phase's cross-lane reductions over a row's threads compile to straight DPP
// sequences instead of branches on the thread count.
template <int DT, int MODE, typename XT, int SPLIT, int WV>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(MODE == 2 ? 4 : 1)))
estep_stats_kernel(const XT* __restrict__ X, int64_t N, int d, int K, int Kp, int waves_rt, int kslabs,
                   int64_t rows_per_chunk, const float4* __restrict__ W32p, const float* __restrict__ c32,
                   const float* __restrict__ mup, const double* __restrict__ ivp,
                   const double* __restrict__ c64d, const float* __restrict__ errc,
                   const float4* __restrict__ rowref, float* __restrict__ partials,
                   double* __restrict__ llpart, float* __restrict__ ll_point, float* __restrict__ R,
                   Pass1Out p1, float rho, const int32_t* __restrict__ slab_rows,
                   const int32_t* __restrict__ slab_len, const int32_t* __restrict__ xflag, int vec) {
  constexpr int DP = 32 * DT, Q = DP / 4, XS = DP + 4, E = 1 + 2 * DP;
  // The fp16-split second pass (SPLIT 2) and its fp32 twin are launched
  // together; *xflag (xrange_kernel) decides which one does the work.
  if (xflag && ((SPLIT == 2) == (*xflag != 0))) return;
  extern __shared__ __align__(16) float smem[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, c = lane & 31;
  const int waves = WV ? WV : waves_rt;
  const int nthr = WV ? WV * 64 : (int)blockDim.x;
  const int KS = waves * 32, SCS = KS + 8;
  // (chunk, slab) of this block, slab fastest. Blocks are dealt to the 8 XCDs
  // in turn, so with a slab count that is a multiple of 8 (or divides 8) each
  // XCD serves a fixed subset of the slabs: the score operands its waves
  // re-read every tile (256 KB per slab at d = 128) then stay in its L2.
  const int64_t chunk = blockIdx.x / kslabs;
  const int slab = blockIdx.x - (int)(chunk * kslabs);
  const int k0 = slab * KS;
  const int kw = k0 + wave * 32;
  // The first pass has no rv, lls, reflist or nzrow, one X tile and a score
  // tile of 32 rows.
  constexpr int kXT = MODE == 2 ? 1 : 2, kSR = MODE == 2 ? 32 : 64;
  float* xsb = smem;               // [kXT][64][XS]: current (and next) X tile
  float* sc = xsb + kXT * 64 * XS; // [kSR][SCS]
  float* rv = sc + kSR * SCS;      // [64][4] per-row references (m, lZ or 1/z, theta)
  double* lls = reinterpret_cast<double*>(rv + (MODE == 2 ? 0 : 256));  // [nthr]
  uint32_t* reflist = reinterpret_cast<uint32_t*>(lls + nthr);  // [waves][kRefCap]
  uint32_t* nzrow = reflist + waves * kRefCap;  // [64]: bit w = row has a nonzero r for wave w

  const int tpr = waves;  // threads per row in the row phase
  const int prow = tid / tpr, psub = tid - prow * tpr;
  const float a_max = errc[0], b_max = errc[1], c_max = errc[2], b2_max = errc[3];
  // fp32 score error: the MFMA sums 2*DP products of rounded operands from
  // zero, then c is added once, so
  //   |s32 - s| <= (2*DP + 4) u sum_i |F_i W_i| + 2 u |c|,
  //   sum_i |F_i W_i| <= a_max |x|^2 + min(b_max |x|_1, b2_max |x|_2).
  const float gam = (float)(2 * DP + 4) * kUnitRound * kBoundSlack;

  // Statistics accumulators, feature block t: Sx and Sxx of component
  // kw + acc_row(h, j), feature DT c + t at element j. The fp32 path keeps
  // both in one two-block accumulator (Sx in elements 0-15, Sxx in 16-31).
  v16f SX[DT], SXX[DT];
  v32f S2[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      SX[t][j] = 0.f;
      SXX[t][j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) S2[t][j] = 0.f;
  }
  float nk = 0.f;
  double ll_acc = 0.0;

  // Row positions [lo, hi) of this block: rows lo..hi-1, or (second pass
  // with row lists) positions in the slab's list of the rows that hold a
  // responsibility above the statistics threshold, the list cut into as many
  // equal chunks (multiples of 64) as the grid has per slab.
  const int32_t* rows = MODE == 1 && slab_rows ? slab_rows + (size_t)slab * N : nullptr;
  int64_t lo, hi;
  if (rows) {
    const int64_t len = slab_len[slab], nch = gridDim.x / kslabs;
    const int64_t rpc = ((len + nch - 1) / nch + 63) / 64 * 64;
    lo = min(len, chunk * rpc);
    hi = min(len, lo + rpc);
  } else {
    lo = chunk * rows_per_chunk;
    hi = min(N, lo + rows_per_chunk);
  }
  auto row_at = [&](int64_t pos) { return rows ? (int64_t)rows[pos] : pos; };
  // The score operands are read through a buffer resource over this wave's
  // slab: the loads are then opaque to the IR optimiser, which would otherwise
  // fold the rotating prefetch registers below into one load per use.
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float4*>(W32p) + (size_t)(__builtin_amdgcn_readfirstlane(kw) >> 5) * Q * 64, (short)0,
      Q * 64 * 16, kBufferRsrcWord3);
  const float ck = c32[kw + c];

  // The next tile's X streams straight into the other LDS buffer (16-byte
  // global->LDS loads) while the statistics MFMAs run.
  const bool async_x = vec && sizeof(XT) == 4;
  // Half-precision rows of at most 96 values (vec == 2: d % 8 == 0, 16-byte
  // aligned): the next tile is fetched as 16-byte chunks of eight values
  // (chunk tid + nthr i, at most two per thread) into registers while the
  // statistics run, and widened into the other buffer at the end of the tile.
  constexpr bool kHalfPre = sizeof(XT) == 2 && DT <= 3;
  const bool hpref = kHalfPre && vec == 2 && 8 * DP <= 2 * nthr;
  uint4 hpre[2];
  // The first pass has no statistics phase to hide the next tile's load
  // under: there the next tile is fetched into registers (16-byte chunks,
  // fp32 rows with d % 4 == 0 or half-precision rows with d % 8 == 0) when the
  // row phase starts, and written over the (single) X tile when it ends.
  // (Not at DT = 4, where those registers would spill at the first pass's
  // 128-register budget; the other block on the CU covers that load.)
  constexpr int kP1Chunks = sizeof(XT) == 4 ? DT : (DT + 1) / 2;  // per thread, at 512 threads
  const bool p1pre = MODE == 2 && DT <= 3 && vec != 0 && nthr * kP1Chunks * (sizeof(XT) == 4 ? 4 : 8) >= 64 * DP;
  uint4 p1x[kP1Chunks];
  if (lo < hi) load_x_tile<XS>(xsb, X, lo, hi, d, DP, tid, nthr, vec, rows);
  // First-pass row phase over 32 rows of the tile (rows rb .. rb + 31, rows
  // xrow0 .. of the X tile): T2 = 2 * waves threads per row, four
  // 16-byte chunks of the 32 * waves-entry score row each (entries
  // 4 (psub + T2 i) + u).
  auto p1_rows = [&](int64_t rb, int xrow0) {
    constexpr int NC = 4;
    const int T2 = 2 * waves;
    // First pass (fp32 normalisers), per (row, slab): the slab maximum m,
    // z = sum 2^(s - m) over the slab, and the candidates: every entry with
    // s >= th, th the loosest of m - W (W on the ladder kCapLadder, ending
    // with m itself) that admits at most kCandT entries; if even m admits
    // more, th is the next float above m and nothing is recorded. So every
    // entry of the slab at or above th is recorded and none below it is;
    // the merge step relies on exactly that.
    const int row = tid / T2, psub = tid - row * T2;
    const int64_t grow = rb + row;
    const bool valid = grow < hi;
    float sq = 0.f, ab = 0.f;  // |x|^2, |x|_1 (slab 0 records the row's bound)
    if (slab == 0) row_norms<DP, XS>(xsb, xrow0 + row, psub, T2, d, sq, ab);
    const float4* srow4 = reinterpret_cast<const float4*>(sc + row * SCS);
    float4 ev[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) ev[i] = srow4[psub + T2 * i];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NC; ++i) mx = fmaxf(mx, fmaxf(fmaxf(ev[i].x, ev[i].y), fmaxf(ev[i].z, ev[i].w)));
    const float m = group_max(mx, T2);
    const float ms = m == -INFINITY ? 0.f : m;  // a slab whose entries are all -inf has z = 0
    double z = 0.0;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const float4 v = ev[i];
      // fp32 sums of four e <= 1, gathered in fp64: |dz| <= 2 u z
      z += (double)((__builtin_amdgcn_exp2f(v.x - ms) + __builtin_amdgcn_exp2f(v.y - ms)) +
                    (__builtin_amdgcn_exp2f(v.z - ms) + __builtin_amdgcn_exp2f(v.w - ms)));
    }
    z = group_sum_d(z, T2);
    auto count_ge = [&](float th) {
      int c = 0;
      if (mx >= th)
#pragma unroll
        for (int i = 0; i < NC; ++i)
          c += (int)(ev[i].x >= th) + (int)(ev[i].y >= th) + (int)(ev[i].z >= th) + (int)(ev[i].w >= th);
      return c;
    };
    float th = -INFINITY;
    int mine = 0, cnt = 0;
    if (m != -INFINITY) {
      // The loosest level that admits at most kCandT entries. Counts only
      // fall along the ladder, so: level 0, then a bisection of the levels
      // [lo, kCapLevels), kCapLevels standing for none. Levels that z alone
      // shows to admit more are not counted: an entry below a level's
      // threshold has e < q = 2^-W (times qm, a margin for the fp32 rounding
      // of m - W) and an entry at or above it e <= 1, so
      // z < count + (KS - count) q, i.e. count > (z - KS q) / (1 - q); z is
      // taken 1e-6 low for its own rounding and the test (in fp32) carries
      // 1e-3 of slack. A level proven to admit more implies as much of every
      // looser one, so lo = 1 + the tightest proven level. Dense slabs thus
      // go straight to the tight levels.
      const float zl = (float)z * (1.f - 1e-6f);
      const float qm = __builtin_amdgcn_exp2f((fabsf(m) + kCapWin) * 2.4e-7f);
      int lo = 0;
      if (zl > (float)kCandT)  // (no level can be proven otherwise)
#pragma unroll
        for (int i = 0; i < kCapLevels - 1; ++i) {
          const float q = kCapQ[i] * qm;
          lo = zl - (float)KS * q > (float)kCandT * (1.f - q) + 1e-3f ? i + 1 : lo;
        }
      int hi = kCapLevels, mine_hi = 0, cnt_hi = 0;  // the last level found to admit <= kCandT
      if (lo == 0) {
        const int c0 = count_ge(m - kCapLadder[0]);
        const int g0 = (int)group_sum((float)c0, T2);
        if (g0 <= kCandT) {
          hi = 0;
          mine_hi = c0;
          cnt_hi = g0;
        } else {
          lo = 1;
        }
      }
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const int cm = count_ge(m - kCapLadder[mid]);
        const int gm = (int)group_sum((float)cm, T2);
        if (gm <= kCandT) {
          hi = mid;
          mine_hi = cm;
          cnt_hi = gm;
        } else {
          lo = mid + 1;
        }
      }
      if (hi < kCapLevels) {
        th = m - kCapLadder[hi];
        mine = mine_hi;
        cnt = cnt_hi;
      } else {
        th = next_up(m);
      }
    }
    // this thread's first slot: exclusive prefix of the counts over the row's lanes
    const int incl = group_incl_scan(mine, psub, T2);
    // The candidates are staged in the row's own score-tile row (its scores
    // are in registers by now; the row's threads are lanes of one wave):
    // candidate j's score at float j, its component at word 8 + j. The
    // record is then written by consecutive lanes: the scores as floats, the
    // components packed four to a word (slots past the count hold stale
    // words, masked to a byte; the merge reads only the first `count`).
    float* stg = sc + row * SCS;
    if (mine) {
      int slot = incl - mine;
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const float vv[4] = {ev[i].x, ev[i].y, ev[i].z, ev[i].w};
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (vv[u] >= th) {
            stg[slot] = vv[u];
            reinterpret_cast<uint32_t*>(stg)[8 + slot] = (uint32_t)(4 * (psub + T2 * i) + u);
            ++slot;
          }
      }
    }
    wave_lds_sync();
    if (valid) {
      const size_t rec = (size_t)slab * N + grow;
      if (psub == 0) p1.h[rec] = make_float4((float)z, m, th, (float)cnt);
      if (slab == 0 && psub == 0) {
        p1.rowE[grow] = gam * (a_max * sq + fminf(b_max * ab, b2_max * sqrtf(sq))) + 2.f * kUnitRound * c_max;
        p1.rowSq[grow] = sq;
      }
      for (int j = psub; j < cnt; j += T2) p1.v[rec * kCandT + j] = stg[j];
      for (int j = psub; 4 * j < cnt; j += T2) {
        const uint32_t* kk = reinterpret_cast<const uint32_t*>(stg) + 8 + 4 * j;
        *reinterpret_cast<uint32_t*>(p1.k + rec * kCandT + 4 * j) =
            (kk[0] & 0xffu) | ((kk[1] & 0xffu) << 8) | ((kk[2] & 0xffu) << 16) | ((kk[3] & 0xffu) << 24);
      }
    }
  };
  int cur = 0;
  for (int64_t r0 = lo; r0 < hi; r0 += 64) {
    float* xs = xsb + cur * 64 * XS;
    __syncthreads();
    if (MODE == 1 && tid < 64) {
      const int64_t pos = r0 + tid;
      const int64_t gr = pos < hi ? row_at(pos) : 0;
      const float4 mr = pos < hi ? rowref[gr] : make_float4(0.f, 0.f, INFINITY, 0.f);
      rv[4 * tid] = mr.x;
      rv[4 * tid + 1] = mr.y;
      rv[4 * tid + 2] = mr.z;
    }

    // 2. scores (the first pass stores them a half tile at a time)
    v16f acc1;
    if constexpr (MODE == 2) {
      v16f acc0;
      score_acc<DT, false>(xs, nullptr, wrs, wave, lane, acc0, acc1);
      score_store(sc, acc0, 0, ck, wave, lane, SCS);
    } else {
      score_tile<DT, false>(xs, sc, nullptr, wrs, ck, wave, lane, SCS);
    }
    __syncthreads();

    // 3. row phase. The score tile holds s / ln 2 (operands and constants are
    //    base-2 scaled, so one hardware exp2 per entry); it is rewritten in
    //    place to e = exp(s - m) with 1/z beside each row (MODE 0) or
    //    directly to r (MODE 1). m, lZ and the LDS row references are in base 2;
    //    the error bound E stays in natural units (scaling by log2(e) and
    //    back cancels in the bound).
    if constexpr (MODE == 2) {
      if (p1pre && r0 + 64 < hi) {
        constexpr int VPC = sizeof(XT) == 4 ? 4 : 8;  // values per 16-byte chunk
#pragma unroll
        for (int i = 0; i < kP1Chunks; ++i) {
          const int ch = tid + nthr * i, row = ch / (DP / VPC), q = ch - row * (DP / VPC);
          const int64_t gr = r0 + 64 + row;
          p1x[i] = (ch < 64 * DP / VPC && gr < hi && VPC * q < d)
                       ? *reinterpret_cast<const uint4*>(X + gr * d + VPC * q)
                       : make_uint4(0u, 0u, 0u, 0u);
        }
      }
      p1_rows(r0, 0);
      __syncthreads();
      score_store(sc, acc1, 0, ck, wave, lane, SCS);
      __syncthreads();
      p1_rows(r0 + 32, 32);
    } else {
      const int row = prow;
      const int64_t grow = r0 + row;
      const bool valid = grow < hi;
      float* srow = sc + row * SCS;
      // |x|^2 and |x|_1 for the bound and the skip threshold (the second pass
      // needs neither)
      float sq = 0.f, ab = 0.f;
      if (MODE == 0) row_norms<DP, XS>(xs, row, psub, tpr, d, sq, ab);
      const float Ebound = gam * (a_max * sq + fminf(b_max * ab, b2_max * sqrtf(sq))) + 2.f * kUnitRound * c_max;

      // Each thread owns the 16-byte chunks psub + tpr*i (i < 8) of its row,
      // i.e. components 4*(psub + tpr*i) + u, u < 4; bit 4i+u of `mask`.
      float4* srow4 = reinterpret_cast<float4*>(srow);
      float m, lZ = 0.f;
      double z = 0.0;
      uint32_t mask1 = 0;  // MODE 1: the entries the first pass re-scored
      // The thread's 32 entries stay in registers from one LDS read (all
      // eight loads in flight) through the max, exp and flag passes.
      float4 ev[8];
      if (MODE == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) ev[i] = srow4[psub + tpr * i];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fmaxf(fmaxf(ev[i].x, ev[i].y), fmaxf(ev[i].z, ev[i].w)));
        m = group_max(mx, tpr);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float4& v = ev[i];
          v.x = __builtin_amdgcn_exp2f(v.x - m);
          v.y = __builtin_amdgcn_exp2f(v.y - m);
          v.z = __builtin_amdgcn_exp2f(v.z - m);
          v.w = __builtin_amdgcn_exp2f(v.w - m);
          srow4[psub + tpr * i] = v;
          // fp32 sums of four e <= 1, gathered in fp64: |dz| <= 2 u z
          z += (double)((v.x + v.y) + (v.z + v.w));
        }
        z = group_sum_d(z, tpr);
      } else {
        // the first pass's row reference: the row's maximal fp32 score m, lZ =
        // l - m, and theta: the entries with s - m >= theta are the ones the
        // first pass re-scored exactly (the same fp32 scores, bit for bit)
        m = rv[4 * row];
        lZ = rv[4 * row + 1];
        const float theta = valid ? rv[4 * row + 2] : INFINITY;
#pragma unroll
        for (int i = 0; i < 8; ++i) ev[i] = srow4[psub + tpr * i];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float4& v = ev[i];
          const float dx = v.x - m, dy = v.y - m, dz = v.z - m, dw = v.w - m;
          mask1 |= ((dx >= theta ? 1u : 0u) | (dy >= theta ? 2u : 0u) | (dz >= theta ? 4u : 0u) |
                    (dw >= theta ? 8u : 0u)) << (4 * i);
          v.x = __builtin_amdgcn_exp2f(dx - lZ);
          v.y = __builtin_amdgcn_exp2f(dy - lZ);
          v.z = __builtin_amdgcn_exp2f(dz - lZ);
          v.w = __builtin_amdgcn_exp2f(dw - lZ);
          srow4[psub + tpr * i] = v;
        }
      }
      // (Single sweep) Which waves' component slices hold a responsibility
      // above rho / max(1, |x|^2) in this row (r = e / z); a point whose
      // 32 responsibilities for a wave are all at or below that threshold is
      // left out of that wave's statistics. Over all N points this drops at
      // most N rho (1 + 2E) from any Nk, and, as |x_j| <= |x|^2 for |x|^2 >= 1,
      // at most as much from any Sx or Sxx element: rho = 2^-20 / N keeps every
      // statistic within about 1e-6 of its value. Entry chunk psub + tpr i
      // belongs to wave (i * waves) / 8. The bits are taken from the fp32
      // responsibilities, before the re-score (which moves an entry by a
      // factor within 1 +- 2E); rows past the end take none (their r is zero).
      if constexpr (SPLIT == 0 && MODE == 0) {
        uint32_t nzb = 0;
        const float wthr = rho / fmaxf(1.f, sq) * (float)z;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float4 v = ev[i];
          const bool nz = (v.x > wthr) | (v.y > wthr) | (v.z > wthr) | (v.w > wthr);
          nzb |= (nz ? 1u : 0u) << ((i * waves) >> 3);
        }
        nzb = group_or(nzb, tpr);
        if (psub == 0) nzrow[row] = valid ? nzb : 0u;
      }
      // Which entries need the exact re-score (E = Ebound, r_k = e_k / z)?
      //  MODE 0: l_n comes from the same fp32 scores, so an unrefined entry is
      //   off by r_k |ds_k - sum_j r_j ds_j| <= 2 E r_k (1 - r_k): entries with
      //   2 E r_k (1 - r_k) > tau are refined (a nearly one-hot row needs
      //   nothing). Refined entries are then off by at most E * U, U = the
      //   unrefined mass; if that could exceed tau the window widens to every
      //   entry within 20 of the row maximum (e >= kExpWindow).
      //  MODE 1: the first pass decided, per row, which entries to re-score
      //   (those with s - m >= theta) and took l_n from exactly those exact
      //   scores and the other fp32 ones, so that every entry meets tau; this
      //   pass re-scores the same entries.
      uint32_t mask = 0;
      if (MODE == 0) {
        const float zf = (float)z;
        const float thr2 = kGateTau * zf * zf * __builtin_amdgcn_rcpf(2.f * Ebound);  // on e (z - e)
        const float maxq = zf >= 2.f ? zf - 1.f : 0.25f * zf * zf;
        const bool refine = valid && maxq > thr2;
        float flagged = 0.f;
        if (refine)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float4 v = ev[i];
            const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const bool fl = vv[u] * (zf - vv[u]) > thr2;
              mask |= (fl ? 1u : 0u) << (4 * i + u);
              flagged += fl ? vv[u] : 0.f;
            }
          }
        // Upper bound on the unrefined mass z - (flagged mass): the fp32 sum of
        // at most K flagged e <= 1 is off by <= (32 + 3) u z, z itself by 2 u z.
        const double unref = fmax(0.0, z - (double)group_sum(flagged, tpr)) + 64.0 * (double)kUnitRound * z;
        const float anyflag = group_max(mask ? 1.f : 0.f, tpr);
        if (refine && anyflag > 0.f && (double)Ebound * unref / z > (double)kGateTau) {
          mask = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float4 v = ev[i];
            mask |= (v.x >= kExpWindow ? 1u : 0u) << (4 * i);
            mask |= (v.y >= kExpWindow ? 1u : 0u) << (4 * i + 1);
            mask |= (v.z >= kExpWindow ? 1u : 0u) << (4 * i + 2);
            mask |= (v.w >= kExpWindow ? 1u : 0u) << (4 * i + 3);
          }
        }
      } else {
        mask = mask1;
      }
      // Exact re-score of the window entries. Each wave pools the entries of
      // its rows into an LDS list and re-scores eight at a time, eight lanes
      // per entry splitting the features (fp64, difference form).
      if (MODE == 0 && psub == 0) rv[4 * row] = m;
      {
        const int cnt = __popc(mask);
        const int incl = wave_incl_scan(cnt);
        const int total = __builtin_amdgcn_readlane(incl, 63);
        const int base = incl - cnt;
        uint32_t* wl = reflist + wave * kRefCap;
        for (int p0 = 0; p0 < total; p0 += kRefCap) {
          uint32_t m2 = mask;
          int pos = base;
          while (m2) {
            const int i = __ffs(m2) - 1;
            m2 &= m2 - 1u;
            if (pos >= p0 && pos < p0 + kRefCap)
              wl[pos - p0] = ((uint32_t)row << 16) | (uint32_t)(4 * (psub + tpr * (i >> 2)) + (i & 3));
            ++pos;
          }
          wave_lds_sync();
          const int n = min(total - p0, kRefCap);
          // eight lanes per entry, 4*DT contiguous features each; every load
          // is issued before the arithmetic (inactive lanes read entry 0)
          constexpr int FPL = DP / 8;
          for (int e0 = 0; e0 < n; e0 += 8) {
            const int e = e0 + (lane >> 3), sl = lane & 7;
            const bool act = e < n;
            const uint32_t ent = act ? wl[e] : 0u;
            const int er = (int)(ent >> 16), ek = (int)(ent & 0xffffu), kg = k0 + ek;
            const float4* xr = reinterpret_cast<const float4*>(xs + er * XS + sl * FPL);
            const float4* mr = reinterpret_cast<const float4*>(mup + (size_t)kg * DP + sl * FPL);
            const double2* ir = reinterpret_cast<const double2*>(ivp + (size_t)kg * DP + sl * FPL);
            float4 mv[FPL / 4];
            double2 iv[FPL / 2];
#pragma unroll
            for (int i = 0; i < FPL / 4; ++i) mv[i] = mr[i];
#pragma unroll
            for (int i = 0; i < FPL / 2; ++i) iv[i] = ir[i];
            // the sum starts from -2 c_k (one lane), so that the constant's load
            // is in flight with the others
            double a0 = sl == 0 ? -2.0 * c64d[kg] : 0.0, a1 = 0.0;  // features past d carry 1/var = 0
            __builtin_amdgcn_sched_barrier(0);  // all global loads in flight before the arithmetic
#pragma unroll
            for (int i = 0; i < FPL / 4; ++i) {
              const float4 xv = xr[i];
              const double t0 = (double)xv.x - (double)mv[i].x, t1 = (double)xv.y - (double)mv[i].y;
              const double t2 = (double)xv.z - (double)mv[i].z, t3 = (double)xv.w - (double)mv[i].w;
              a0 = fma(t0 * t0, iv[2 * i].x, a0);
              a1 = fma(t1 * t1, iv[2 * i].y, a1);
              a0 = fma(t2 * t2, iv[2 * i + 1].x, a0);
              a1 = fma(t3 * t3, iv[2 * i + 1].y, a1);
            }
            double acc = a0 + a1;
            acc += dpp_d<kDppXor1>(acc);  // the eight lanes of an entry: half a DPP row
            acc += dpp_d<kDppXor2>(acc);
            acc += dpp_d<kDppHalfMirror>(acc);
            if (act && sl == 0) {
              // exact (s - m) / ln 2: acc = sum_j (x_j - mu_j)^2 / var_j - 2 c_k
              const double dl = (-0.5 * acc) * kLog2E - (double)rv[4 * er];
              sc[er * SCS + ek] = __builtin_amdgcn_exp2f(MODE == 0 ? (float)dl : (float)(dl - (double)rv[4 * er + 1]));
            }
          }
          wave_lds_sync();
        }
      }
      if (MODE == 0) {
        const bool redo = group_max(mask ? 1.f : 0.f, tpr) > 0.f;  // this row was re-scored
        double z2 = 0.0;
        if (redo)
#pragma unroll 4
          for (int i = 0; i < 8; ++i) {
            const float4 v = srow4[psub + tpr * i];
            z2 += (double)((v.x + v.y) + (v.z + v.w));
          }
        z2 = group_sum_d(z2, tpr);
        if (redo) z = z2;
        // z is in [1, K]: the fp32 hardware log2 is good to ~1e-7 absolute, far
        // inside the 1e-4 relative bar of l_n; r = e / z uses the hardware
        // reciprocal of z in fp32 (1 ulp: with z's own 2 u, r is within
        // 4e-7 relative).
        const double lZd = (double)__builtin_amdgcn_logf((float)z);  // log2
        const float invz = valid ? __builtin_amdgcn_rcpf((float)z) : 0.f;
        if (valid && psub == 0) {
          const double l = ((double)m + lZd) * kLn2;
          ll_acc += l;
          if (ll_point) ll_point[grow] = (float)l;
        }
        // the tile keeps e; the statistics loop applies r = e / z as it reads it
        if (psub == 0) rv[4 * row + 1] = invz;
        if (R && valid)
#pragma unroll 1
          for (int i = 0; i < 32; ++i) {
            const int kl = 4 * (psub + tpr * (i >> 2)) + (i & 3);
            if (k0 + kl < K) R[grow * K + k0 + kl] = srow[kl] * invz;
          }
      } else if (!valid) {
#pragma unroll 1
        for (int i = 0; i < 8; ++i) srow4[psub + tpr * i] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      if (MODE == 1 && R && valid)
#pragma unroll 1
        for (int i = 0; i < 32; ++i) {
          const int kl = 4 * (psub + tpr * (i >> 2)) + (i & 3);
          if (k0 + kl < K) R[grow * K + k0 + kl] = srow[kl];
        }
    }
    __syncthreads();

    // 4. statistics, with the next X tile streaming into the other buffer
    const int64_t rn = r0 + 64;
    if (MODE != 2 && async_x && rn < hi) async_x_tile<XS>(xsb + (cur ^ 1) * 64 * XS, reinterpret_cast<const float*>(X),
                                             rn, hi, d, wave, waves, lane, rows);
    if constexpr (kHalfPre && MODE != 2)
      if (hpref && rn < hi)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ch = tid + nthr * i, row = ch / (DP / 8), q = ch - row * (DP / 8);
        const int64_t pos = rn + row;
        const bool in = ch < 8 * DP && pos < hi && 8 * q < d;
        hpre[i] = in ? *reinterpret_cast<const uint4*>(X + row_at(pos) * d + 8 * q) : make_uint4(0u, 0u, 0u, 0u);
      }
    if constexpr (MODE == 2) {
      // the first pass accumulates no statistics
    } else if constexpr (SPLIT == 1) {
      // Split-bf16 products on the 32x32x16 bf16 MFMA (see the small-K
      // kernel for the error of a product): block pb covers points
      // 16 pb + 8 h + t (t < 8) of lane (h, c), r of component c as the A
      // operand and x or x^2 of feature DT c + t2 of the same points as B, so
      // the accumulators keep the layout of the fp32 path.
#pragma unroll 1
      for (int pb = 0; pb < 4; ++pb) {
        float rr[8], xv[8][DT];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int row = 16 * pb + 8 * h + t;
          rr[t] = sc[row * SCS + wave * 32 + c];
          if (MODE == 0) rr[t] *= rv[4 * row + 1];  // e -> r = e / z (0 past the last row)
          nk += rr[t];
          const float* xr = xs + row * XS + DT * c;
#pragma unroll
          for (int t2 = 0; t2 < DT; ++t2) xv[t][t2] = xr[t2];
        }
        v8bf rh, rl;
        split_bf16(rr, rh, rl);
#pragma unroll
        for (int t2 = 0; t2 < DT; ++t2) {
          float xx[8], x2[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            xx[t] = xv[t][t2];
            x2[t] = xx[t] * xx[t];
          }
          v8bf xh, xl, qh, ql;
          split_bf16(xx, xh, xl);
          split_bf16(x2, qh, ql);
          SX[t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rh, xh, SX[t2], 0, 0, 0);
          SXX[t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rh, qh, SXX[t2], 0, 0, 0);
          SX[t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rh, xl, SX[t2], 0, 0, 0);
          SXX[t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rh, ql, SXX[t2], 0, 0, 0);
          SX[t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rl, xh, SX[t2], 0, 0, 0);
          SXX[t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rl, qh, SXX[t2], 0, 0, 0);
        }
      }
    } else if constexpr (SPLIT == 2) {
      // Half-precision X (second pass): exact fp16 splits on the 32x32x16 f16
      // MFMA (which keeps fp16 subnormal inputs), in the lane layout of the
      // bf16 path. x is exact in fp16; q = (16 x)^2 is exact in fp32 (22
      // significant bits) and equals q_hi + q_lo, two fp16 values, for |x| >=
      // 2^-6 (below, within 2^-25); r' = 2^10 r is r_hi + r_lo + d with |d|
      // <= max(2^-22 r', 2^-25). Sx takes r_hi x + r_lo x and Sxx r_hi q_hi +
      // r_hi q_lo + r_lo q_hi, products exact in fp32: per term Sx is off by
      // at most 2^-22 r|x| + 2^-35 |x| and Sxx by 2^-21 r x^2 + 2^-35 x^2 +
      // 2^-68, plus 2^-33 r where |x| < 2^-6, before the fp32 accumulation.
      // The partial is scaled back by 2^-10 and 2^-18 (exact). This variant runs only when every row has
      // |x|^2 < 225 (so every |x| < 15 and q stays in the fp16 range); the
      // plain fp32 second pass is launched beside it and runs otherwise
      // (`xflag`).
#pragma unroll 1
      for (int pb = 0; pb < 4; ++pb) {
        v8h rh, rl;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float e = sc[(16 * pb + 8 * h + t) * SCS + wave * 32 + c];
          nk += e;
          const float rs = e * 1024.f;
          rh[t] = (_Float16)rs;
          rl[t] = (_Float16)(rs - (float)rh[t]);
        }
#pragma unroll
        for (int t2 = 0; t2 < DT; ++t2) {
          v8h xh, qh, ql;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float x = xs[(16 * pb + 8 * h + t) * XS + DT * c + t2];
            const float q = (16.f * x) * (16.f * x);
            xh[t] = (_Float16)x;
            qh[t] = (_Float16)q;
            ql[t] = (_Float16)(q - (float)qh[t]);
          }
          SX[t2] = __builtin_amdgcn_mfma_f32_32x32x16_f16(rh, xh, SX[t2], 0, 0, 0);
          SXX[t2] = __builtin_amdgcn_mfma_f32_32x32x16_f16(rh, qh, SXX[t2], 0, 0, 0);
          SX[t2] = __builtin_amdgcn_mfma_f32_32x32x16_f16(rl, xh, SX[t2], 0, 0, 0);
          SXX[t2] = __builtin_amdgcn_mfma_f32_32x32x16_f16(rh, ql, SXX[t2], 0, 0, 0);
          SXX[t2] = __builtin_amdgcn_mfma_f32_32x32x16_f16(rl, qh, SXX[t2], 0, 0, 0);
        }
      }
    } else if constexpr (MODE == 1) {
      // Second pass: two points per step on the 32x32x2 MFMA, lanes h = 0 and
      // h = 1 holding r and x of points p0 and p0 + 1 (the A and B operands),
      // Sx and Sxx in separate instructions whose accumulators have the
      // layout of the two-block form's blocks. Every point is taken: the row
      // lists already left out the (row, slab) pairs without a responsibility
      // above the threshold, and on the pairs they keep this plain loop runs
      // faster than the one-point form with its per-point skip (ivf 71.6 ->
      // 67.4 ms; largek 68.0 -> 68.9 ms).
#pragma unroll 2
      for (int p0 = 0; p0 < 64; p0 += 2) {
        const int p = p0 + h;
        const float r = sc[p * SCS + wave * 32 + c];
        nk += r;
        const float* xr = xs + p * XS + DT * c;
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const float xv = xr[t];
          SX[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(r, xv, SX[t], 0, 0, 0);
          SXX[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(r, xv * xv, SXX[t], 0, 0, 0);
        }
      }
    } else {
      // One point per step on the two-block 32x32x1 MFMA: both halves of the
      // wave hold r of component c of point p (the A operand of either block),
      // lanes h = 0 hold x and lanes h = 1 hold x^2 of feature DT c + t (the B
      // operands), so one instruction adds r x to block 0 (Sx) and r x^2 to
      // block 1 (Sxx). Only the points with a nonzero r for this wave are
      // visited (a zero r adds exactly zero); the operands of the next such
      // point are read from LDS before this point's MFMAs issue.
      // A point's operands are prepared (r = e / z, x or x^2) before the next
      // point's LDS reads issue, so the wait for them never covers those.
      auto sload = [&](int p, float& e, float& iz, float(&xv)[DT]) {
        e = sc[p * SCS + wave * 32 + c];
        iz = MODE == 0 ? rv[4 * p + 1] : 1.f;
        const float* xr = xs + p * XS + DT * c;
#pragma unroll
        for (int t = 0; t < DT; ++t) xv[t] = xr[t];
      };
      float r, bv[DT];
      auto prep = [&](float e, float iz, const float(&xv)[DT]) {
        r = MODE == 0 ? e * iz : e;  // e -> r = e / z
        nk += r;
#pragma unroll
        for (int t = 0; t < DT; ++t) bv[t] = h ? xv[t] * xv[t] : xv[t];
      };
      auto smfma = [&]() {
#pragma unroll
        for (int t = 0; t < DT; ++t) S2[t] = __builtin_amdgcn_mfma_f32_32x32x1f32(r, bv[t], S2[t], 0, 0, 0);
      };
      // Active points in increasing order, two per iteration (no register
      // rotation). An odd count is padded with the lowest inactive point
      // (its responsibilities are at most the threshold, or zero past the
      // last row: taking it only adds what the skip would leave out); past
      // the end the loads read point 0, unused.
      uint64_t am = __builtin_amdgcn_ballot_w64((nzrow[lane] >> wave) & 1u);
      const int na = __builtin_popcountll(am);
      if (na & 1) am |= ~am & (am + 1);
      auto pop = [&]() {
        const int p = am ? __builtin_ctzll(am) : 0;
        am &= am - 1;
        return p;
      };
      if (na) {
        float ea, ia, xa[DT], eb, ib, xb[DT];
        sload(pop(), ea, ia, xa);
#pragma unroll 1
        for (int k = 0; k < na; k += 2) {
          prep(ea, ia, xa);
          __builtin_amdgcn_sched_barrier(0);
          sload(pop(), eb, ib, xb);
          __builtin_amdgcn_sched_barrier(0);
          smfma();
          __builtin_amdgcn_sched_barrier(0);
          prep(eb, ib, xb);
          __builtin_amdgcn_sched_barrier(0);
          sload(pop(), ea, ia, xa);
          __builtin_amdgcn_sched_barrier(0);
          smfma();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (MODE == 2) {
      // one X buffer: the scores of this tile are done with it
      if (rn < hi && p1pre) {
        float* xn = xsb;
        constexpr int VPC = sizeof(XT) == 4 ? 4 : 8;
#pragma unroll
        for (int i = 0; i < kP1Chunks; ++i) {
          const int ch = tid + nthr * i, row = ch / (DP / VPC), q = ch - row * (DP / VPC);
          if (ch < 64 * DP / VPC) {
            if constexpr (sizeof(XT) == 4) {
              *reinterpret_cast<uint4*>(xn + row * XS + 4 * q) = p1x[i];
            } else {
              const XT* hv = reinterpret_cast<const XT*>(&p1x[i]);
              *reinterpret_cast<float4*>(xn + row * XS + 8 * q) =
                  make_float4((float)hv[0], (float)hv[1], (float)hv[2], (float)hv[3]);
              *reinterpret_cast<float4*>(xn + row * XS + 8 * q + 4) =
                  make_float4((float)hv[4], (float)hv[5], (float)hv[6], (float)hv[7]);
            }
          }
        }
      } else if (rn < hi) {
        load_x_tile<XS>(xsb, X, rn, hi, d, DP, tid, nthr, vec, rows);
      }
    } else if constexpr (kHalfPre) {
      if (rn < hi && hpref) {
        float* xn = xsb + (cur ^ 1) * 64 * XS;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int ch = tid + nthr * i, row = ch / (DP / 8), q = ch - row * (DP / 8);
          if (ch < 8 * DP) {
            const XT* hv = reinterpret_cast<const XT*>(&hpre[i]);
            *reinterpret_cast<float4*>(xn + row * XS + 8 * q) =
                make_float4((float)hv[0], (float)hv[1], (float)hv[2], (float)hv[3]);
            *reinterpret_cast<float4*>(xn + row * XS + 8 * q + 4) =
                make_float4((float)hv[4], (float)hv[5], (float)hv[6], (float)hv[7]);
          }
        }
      } else if (rn < hi) {
        load_x_tile<XS>(xsb + (cur ^ 1) * 64 * XS, X, rn, hi, d, DP, tid, nthr, vec, rows);
      }
    } else if (rn < hi && !async_x) {
      load_x_tile<XS>(xsb + (cur ^ 1) * 64 * XS, X, rn, hi, d, DP, tid, nthr, vec, rows);
    }
    // This thread's async tile loads have landed. The wait is unconditional so
    // that no global->LDS load counts as in flight at the top of the loop:
    // the compiler would otherwise drain every global load before each LDS
    // read of the score loop.
    __builtin_amdgcn_s_waitcnt(0);
    if (MODE != 2) cur ^= 1;
  }

  if constexpr (MODE == 2) return;
  // statistics partial of this (chunk, slab)
  float* part = partials + (size_t)chunk * Kp * E;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int comp = kw + acc_row(h, j);
      const int f = DT * c + t;
      // (the fp16 split path accumulated 2^10 r x and 2^18 r x^2)
      part[(size_t)comp * E + 1 + f] =
          SPLIT == 2 ? SX[t][j] * 0x1p-10f : (SPLIT || MODE == 1) ? SX[t][j] : S2[t][j];
      part[(size_t)comp * E + 1 + DP + f] =
          SPLIT == 2 ? SXX[t][j] * 0x1p-18f : (SPLIT || MODE == 1) ? SXX[t][j] : S2[t][16 + j];
    }
  // the halves of the split path and of the second pass saw different points;
  // those of the single sweep's one-point form the same ones
  if (SPLIT || MODE == 1) nk += __shfl_xor(nk, 32, 64);
  if (h == 0) part[(size_t)(kw + c) * E] = nk;

  if (MODE == 0) {
    lls[tid] = ll_acc;
    __syncthreads();
    if (tid == 0) {
      double s = 0.0;
      for (int i = 0; i < nthr; ++i) s += lls[i];
      llpart[chunk] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Per-row normalisers from the fp32 first pass (two-pass regime)
// ---------------------------------------------------------------------------
//
// One wave per 64 consecutive rows, one lane per row, all in base-2 units.
// From the row's per-slab records: m = the largest fp32 score, z = sum_s z_s
// 2^(m_s - m), so that m + log2 z is the log-sum-exp of the fp32 scores.
// With E the row's bound on |s32 - s| (E2 = E log2 e in base 2), the second
// pass gets (m, lZ, theta) and re-scores exactly the entries with
// s32 - m >= theta, with r = 2^(s' - m - lZ) where s' is the exact score of
// those entries and the fp32 score of the others. With F the re-scored set
// and U the responsibility mass outside it, an entry is then off by at most
//   r E U (k in F),   r E (1 + U - 2 r) (k outside F).
//  (a) No re-score (theta = +inf, U = 1): every entry is off by at most
//      2 E r (1 - r), and over a row max_k r (1 - r) is the largest entry's
//      r_1 (1 - r_1) (the others sum to 1 - r_1), with r_1 = 1/z. Taken
//      when 2 E r_1 (1 - r_1) <= tau: one-hot rows and dense rows of small r.
//  (b) Otherwise a window theta = -W: outside it s32 - m < -W, so
//      r < 2^(-W + 2 E2) (the exact l is at least m - E2), and W >= Wb =
//      log2(2E / tau) + 2 E2 keeps every outside entry within tau. The
//      smallest W of a ladder from Wb up to what the records hold completely
//      (every slab recorded all its entries at or above its threshold th, so
//      the window must stay above the largest th) with E U <= tau, U bounded
//      by 2^(2 E2) (z - sum of the window's 2^(s32 - m)) / z, is taken; its
//      entries are re-scored here (fp64, difference form) and l is
//      m + log2(z + sum over the window of 2^(s - m) - 2^(s32 - m)).
//  (c) Neither (no window satisfies E U <= tau, or a slab had more than
//      kCandT entries near its maximum): the row goes on the fallback list
//      for the fp64 normaliser pass.
// l_n (natural log) goes to lrow; the fallback pass writes its rows' entries.
template <int DT, typename XT>
__global__ void __launch_bounds__(64)
lse_merge_kernel(const XT* __restrict__ X, int64_t N, int d, int kslabs, int KS,
                 const float4* __restrict__ p1h, const float* __restrict__ p1v, const uint8_t* __restrict__ p1k,
                 const float* __restrict__ rowE, const float* __restrict__ mup,
                 const double* __restrict__ ivp, const double* __restrict__ c64d, float4* __restrict__ rowref,
                 double* __restrict__ lrow, int32_t* __restrict__ fblist, int32_t* __restrict__ fbcount, int vec) {
  constexpr int DP = 32 * DT, FPL = DP / 8, kLevels = 8, kCap = 512;
  static_assert(kCandT == 8, "a record's candidates are read as two float4");
  __shared__ uint32_t elist[kCap];  // (lane << 16) | component
  __shared__ float ev32[kCap];      // its fp32 score
  __shared__ double ex[kCap];       // its exact score
  const int lane = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.x * 64, n = n0 + lane;
  const bool valid = n < N;
  // slab sl's header of this lane's row (read where needed: L2-resident)
  auto hdr = [&](int sl) { return p1h[(size_t)sl * N + n]; };
  auto cands = [&](int sl, float (&v)[kCandT]) {
    const float4* q = reinterpret_cast<const float4*>(p1v + ((size_t)sl * N + n) * kCandT);
    const float4 a = q[0], b = q[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  };

  // the row's largest fp32 score, and the largest capture threshold
  float m = -INFINITY, tc = -INFINITY;
  if (valid)
    for (int sl = 0; sl < kslabs; ++sl) {
      const float4 h = hdr(sl);
      m = fmaxf(m, h.y);
      tc = fmaxf(tc, h.z);
    }
  const float E = valid ? rowE[n] : 0.f;
  const double E2 = (double)E * kLog2E;
  // the window ladder of (b): from Wb to what the records hold completely,
  // each as the fp32 threshold the second pass compares s32 - m with (the
  // 1/64 keeps the rounding of s32 - m inside)
  const double Wb = log2(2.0 * (double)E / (double)kGateTau) + 2.0 * E2 + 1.0 / 64;
  const double Wmax = fmin((double)kCapWin, (double)m - (double)tc) - 1.0 / 64;
  // z (hardware exp2 of exact fp32 differences, each term within 2 ulp;
  // fp64 sums)
  double z = 0.0;
  if (valid)
    for (int sl = 0; sl < kslabs; ++sl) {
      const float4 h = hdr(sl);
      if (h.y != -INFINITY) z += (double)h.x * (double)__builtin_amdgcn_exp2f(h.y - m);
    }
  // the fp32 mass of the windows lev[0..kLevels) (thresholds on s32 - m,
  // loosest last)
  float lev[kLevels];
  double S[kLevels];
  auto window_mass = [&]() {
#pragma unroll
    for (int i = 0; i < kLevels; ++i) S[i] = 0.0;
    for (int sl = 0; sl < kslabs; ++sl) {
      const float4 h = hdr(sl);
      if (h.w > 0.f && h.y - m >= lev[kLevels - 1]) {
        float v[kCandT];
        cands(sl, v);
#pragma unroll
        for (int j = 0; j < kCandT; ++j) {
          const float dd = v[j] - m;
          if (j < (int)h.w && dd >= lev[kLevels - 1]) {
            const double e = (double)__builtin_amdgcn_exp2f(dd);
#pragma unroll
            for (int i = 0; i < kLevels; ++i)
              if (dd >= lev[i]) S[i] += e;
          }
        }
      }
    }
  };
  const double grow = exp2(2.0 * E2);
  // E U <= tau for the window lev[i]; 16 u covers the rounding of z and of
  // the window sums
  auto holds = [&](int i) {
    return (double)E * grow * ((z - S[i]) / z + 16.0 * (double)kUnitRound) <= (double)kGateTau;
  };
  const double r1 = 1.0 / z;
  float theta = INFINITY;
  bool fallback = false;
  if (valid && !(2.0 * (double)E * r1 * (1.0 - r1) <= (double)kGateTau)) {
    fallback = true;
    if (Wmax >= Wb) {
      // the smallest window in two rounds of kLevels levels: a coarse ladder
      // over [Wb, Wmax], then a fine one inside the bracket it found
      double wlo = Wb, whi = Wmax;
      for (int round = 0; round < 2 && fallback; ++round) {
#pragma unroll
        for (int i = 0; i < kLevels; ++i) lev[i] = (float)-(wlo + (whi - wlo) * i / (kLevels - 1));
        window_mass();
        int first = kLevels;
#pragma unroll
        for (int i = kLevels - 1; i >= 0; --i)
          if (holds(i)) first = i;
        if (first == kLevels) break;  // not even the widest window: fallback
        theta = lev[first];
        if (first == 0) fallback = false;
        else {
          whi = -(double)lev[first];
          wlo = -(double)lev[first - 1];
          if (round == 1) fallback = false;
        }
      }
      if (theta != INFINITY) fallback = false;
    }
  }
  // exact re-score of every window entry, pooled over the wave: lane l's
  // entries take list positions [base, base + cnt), eight lanes per entry
  int cnt = 0;
  if (valid && !fallback && theta != INFINITY)
    for (int sl = 0; sl < kslabs; ++sl) {
      const float4 h = hdr(sl);
      if (h.w <= 0.f || h.y - m < theta) continue;
      float v[kCandT];
      cands(sl, v);
#pragma unroll
      for (int j = 0; j < kCandT; ++j) cnt += (j < (int)h.w && v[j] - m >= theta) ? 1 : 0;
    }
  const int incl = wave_incl_scan(cnt);
  const int total = __builtin_amdgcn_readlane(incl, 63);
  const int base = incl - cnt;
  double corr = 0.0;
  for (int p0 = 0; p0 < total; p0 += kCap) {
    if (cnt) {
      int pos = base;
      for (int sl = 0; sl < kslabs; ++sl) {
        const float4 h = hdr(sl);
        if (h.w <= 0.f || h.y - m < theta) continue;
        float v[kCandT];
        cands(sl, v);
        const size_t rec = ((size_t)sl * N + n) * kCandT;
#pragma unroll
        for (int j = 0; j < kCandT; ++j)
          if (j < (int)h.w && v[j] - m >= theta) {
            if (pos >= p0 && pos < p0 + kCap) {
              elist[pos - p0] = ((uint32_t)lane << 16) | (uint32_t)(sl * KS + p1k[rec + j]);
              ev32[pos - p0] = v[j];
            }
            ++pos;
          }
      }
    }
    wave_lds_sync();
    const int nn = min(total - p0, kCap);
    for (int e0 = 0; e0 < nn; e0 += 8) {
      const int e = e0 + (lane >> 3), sl8 = lane & 7;
      const bool act = e < nn;
      const uint32_t ent = act ? elist[e] : 0u;
      const int er = (int)(ent >> 16), kg = (int)(ent & 0xffffu);
      const int64_t xr = (n0 + er) * (int64_t)d;
      const float4* mr = reinterpret_cast<const float4*>(mup + (size_t)kg * DP + sl8 * FPL);
      const double2* ir = reinterpret_cast<const double2*>(ivp + (size_t)kg * DP + sl8 * FPL);
      // every load before the arithmetic; features past d carry 1/var = 0.
      // vec: rows of d % 4 == 0 values, 16-byte (fp32) or 8-byte (half)
      // aligned, read four values per load.
      float xv[FPL];
      float4 mv[FPL / 4];
      double2 iv[FPL / 2];
#pragma unroll
      for (int j = 0; j < FPL / 4; ++j) {
        const int f = sl8 * FPL + 4 * j;
        if (vec) {
          float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
          if (f < d) {
            if constexpr (sizeof(XT) == 4) {
              q = *reinterpret_cast<const float4*>(X + xr + f);
            } else {
              const uint2 raw = *reinterpret_cast<const uint2*>(X + xr + f);
              const XT* hv = reinterpret_cast<const XT*>(&raw);
              q = make_float4((float)hv[0], (float)hv[1], (float)hv[2], (float)hv[3]);
            }
          }
          xv[4 * j] = q.x;
          xv[4 * j + 1] = q.y;
          xv[4 * j + 2] = q.z;
          xv[4 * j + 3] = q.w;
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) xv[4 * j + u] = f + u < d ? load_x(X, xr + f + u) : 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < FPL / 4; ++i) mv[i] = mr[i];
#pragma unroll
      for (int i = 0; i < FPL / 2; ++i) iv[i] = ir[i];
      const double cst = sl8 == 0 ? -2.0 * c64d[kg] : 0.0;
      __builtin_amdgcn_sched_barrier(0);
      double a0 = cst, a1 = 0.0;
#pragma unroll
      for (int i = 0; i < FPL / 4; ++i) {
        const double t0 = (double)xv[4 * i] - (double)mv[i].x, t1 = (double)xv[4 * i + 1] - (double)mv[i].y;
        const double t2 = (double)xv[4 * i + 2] - (double)mv[i].z, t3 = (double)xv[4 * i + 3] - (double)mv[i].w;
        a0 = fma(t0 * t0, iv[2 * i].x, a0);
        a1 = fma(t1 * t1, iv[2 * i].y, a1);
        a0 = fma(t2 * t2, iv[2 * i + 1].x, a0);
        a1 = fma(t3 * t3, iv[2 * i + 1].y, a1);
      }
      double acc = a0 + a1;
      acc += dpp_d<kDppXor1>(acc);
      acc += dpp_d<kDppXor2>(acc);
      acc += dpp_d<kDppHalfMirror>(acc);
      if (act && sl8 == 0) ex[e] = (-0.5 * acc) * kLog2E;  // exact s, base 2
    }
    wave_lds_sync();
    for (int pos = max(base, p0); pos < min(base + cnt, p0 + kCap); ++pos)
      corr += exp2(ex[pos - p0] - (double)m) - exp2((double)ev32[pos - p0] - (double)m);
    wave_lds_sync();
  }
  if (valid && !fallback) {
    const double l2 = (double)m + log2(z + corr);
    rowref[n] = make_float4(m, (float)(l2 - (double)m), theta, E);
    lrow[n] = l2 * kLn2;
  }
  if (valid && fallback) fblist[atomicAdd(fbcount, 1)] = (int32_t)n;
}

// Per kLlRows rows, 256 threads of four consecutive rows each: l_n (natural)
// to ll_point (nullable) and the block's sum, in a fixed order (each thread's
// rows in turn, then a pairwise tree over the threads), to llpart.
__global__ void __launch_bounds__(256) row_ll_sum_kernel(const double* __restrict__ lrow, int64_t N,
                                                         float* __restrict__ ll_point, double* __restrict__ llpart) {
  static_assert(kLlRows == 4 * 256, "four rows per thread");
  __shared__ double s[256];
  const int64_t r = (int64_t)blockIdx.x * kLlRows + 4 * threadIdx.x;
  double a = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (r + i < N) {
      const double l = lrow[r + i];
      if (ll_point) ll_point[r + i] = (float)l;
      a += l;
    }
  s[threadIdx.x] = a;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) s[threadIdx.x] += s[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) llpart[blockIdx.x] = s[0];
}

// ---------------------------------------------------------------------------
// Row lists of the second pass (two-pass regime)
// ---------------------------------------------------------------------------
//
// The statistics leave out a point's contribution to a slice of components
// when every responsibility it holds there is at most rho / max(1, |x|^2)
// (the threshold of the in-kernel skip). Whole slabs can be ruled out per row
// from the first pass alone: with the slab's largest fp32 score m_s and the
// row's (m, lZ, E) in base 2, every entry of the slab has
//   r <= 2^(m_s + E2 - m - lZ)
// (its exact score is within E2 of its fp32 one, and the second pass uses
// either), so a slab with m_s + E2 - m - lZ < log2(rho / max(1, |x|^2)) holds
// no responsibility the statistics would take. The check runs in fp64 with
// 1/64 of slack against the rounding of the fp32 inputs; rows it cannot decide
// (NaN) are kept. Each slab's list then holds, in increasing order, the rows
// it keeps, and the second pass walks only those.

// Per (64-row tile, slab): the kept rows as a bit mask and their count.
__global__ void __launch_bounds__(64) slab_keep_kernel(const float4* __restrict__ p1h,
                                                       const float4* __restrict__ rowref,
                                                       const float* __restrict__ rowSq, int64_t N, int64_t tiles,
                                                       float rho, uint64_t* __restrict__ smask,
                                                       int32_t* __restrict__ scnt) {
  const int slab = blockIdx.y;
  const int64_t t = blockIdx.x, n = t * 64 + threadIdx.x;
  bool keep = false;
  if (n < N) {
    const float ms = p1h[(size_t)slab * N + n].y;
    const float4 rr = rowref[n];
    const double lhs = (double)ms - (double)rr.x - (double)rr.y + (double)rr.w * kLog2E + 1.0 / 64;
    const double rhs = log2((double)rho) - log2(fmax(1.0, (double)rowSq[n]));
    keep = !(lhs < rhs);
  }
  const uint64_t m = __builtin_amdgcn_ballot_w64(keep);
  if (threadIdx.x == 0) {
    smask[(size_t)slab * tiles + t] = m;
    scnt[(size_t)slab * tiles + t] = __builtin_popcountll(m);
  }
}

// Per (segment, slab), one block of 256: the kept rows of the segment's
// tiles (kSlabSegs segments of equal tile count per slab, the last ones
// possibly empty), read with consecutive threads on consecutive tiles.
__global__ void __launch_bounds__(256) slab_seg_kernel(const int32_t* __restrict__ scnt, int64_t tiles,
                                                       int32_t* __restrict__ sseg) {
  __shared__ int32_t part[256];
  const int slab = blockIdx.y, g = blockIdx.x;
  const int64_t per = (tiles + kSlabSegs - 1) / kSlabSegs;
  const int64_t lo = min(tiles, g * per), hi = min(tiles, lo + per);
  const int32_t* c = scnt + (size_t)slab * tiles;
  int32_t a = 0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += 256) a += c[i];
  part[threadIdx.x] = a;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) part[threadIdx.x] += part[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) sseg[(size_t)slab * kSlabSegs + g] = part[0];
}

// One block of kSlabSegs per slab: the segment counts become their exclusive
// prefix (in place), the total the slab's list length.
__global__ void __launch_bounds__(kSlabSegs) slab_scan_kernel(int32_t* __restrict__ sseg, int32_t* __restrict__ slen) {
  __shared__ int32_t part[kSlabSegs];
  int32_t* c = sseg + (size_t)blockIdx.x * kSlabSegs;
  const int32_t a = c[threadIdx.x];
  part[threadIdx.x] = a;
  __syncthreads();
  for (int o = 1; o < kSlabSegs; o <<= 1) {  // inclusive scan
    const int32_t v = (int)threadIdx.x >= o ? part[threadIdx.x - o] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  c[threadIdx.x] = part[threadIdx.x] - a;
  if (threadIdx.x == kSlabSegs - 1) slen[blockIdx.x] = part[kSlabSegs - 1];
}

// Per (segment, slab), one wave: the segment's tiles in order, each kept row
// to its place in the slab's list (its tile's base plus its rank among the
// tile's kept rows).
__global__ void __launch_bounds__(64) slab_scatter_kernel(const uint64_t* __restrict__ smask,
                                                          const int32_t* __restrict__ sseg, int64_t N,
                                                          int64_t tiles, int32_t* __restrict__ slist) {
  const int slab = blockIdx.y, g = blockIdx.x, lane = threadIdx.x;
  const int64_t per = (tiles + kSlabSegs - 1) / kSlabSegs;
  const int64_t lo = min(tiles, g * per), hi = min(tiles, lo + per);
  int32_t* out = slist + (size_t)slab * N;
  int32_t off = sseg[(size_t)slab * kSlabSegs + g];
  const uint64_t below = (1ull << lane) - 1ull;
  for (int64_t t = lo; t < hi; ++t) {
    const uint64_t m = smask[(size_t)slab * tiles + t];
    if ((m >> lane) & 1u) out[off + __builtin_popcountll(m & below)] = (int32_t)(t * 64 + lane);
    off += __builtin_popcountll(m);
  }
}

__global__ void fill_int_kernel(int32_t* __restrict__ a, int64_t n, int32_t v) {
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t < n) a[t] = v;
}

// ---------------------------------------------------------------------------
// Nearest-centre assignment (Lloyd's k-means): fp32 scores, exact fp64 check
// ---------------------------------------------------------------------------
//
// With unit variances and zero log-weights the mixture score of centre k is
// s_k = -|x - c_k|^2 / 2 - (d/2) log 2 pi, so the nearest centre has the
// highest score. A block walks the 64-point tiles of its row chunk and, per
// tile, every slab of KS = 32 * waves centres (X stays in LDS across slabs):
//   1. scores of the slab on the fp32 matrix cores (score_tile);
//   2. per row (`waves` threads per row): every centre whose fp32 score is
//      within twice the score error bound of the slab's best fp32 score may be
//      the slab's nearest centre. Those candidates get |x - c_k|^2 exactly in
//      fp64 (difference form, 2 to 8 lanes per candidate by d) and the smallest
//      wins, ties to the lower index;
//   3. the slab's winner replaces the row's best so far only when strictly
//      nearer, so across slabs ties also go to the lower index.
// Outputs per row: the index and |x - c|^2 (rounded to fp32); per block the
// fp64 sum of the exact |x - c|^2 (the inertia partial).
template <int DT, typename XT>
__global__ void __launch_bounds__(512)
kmeans_assign_kernel(const XT* __restrict__ X, int64_t N, int d, int K, int waves, int kslabs,
                     int64_t rows_per_chunk, const float4* __restrict__ W32p, const float* __restrict__ c32,
                     const float* __restrict__ mup, const float* __restrict__ errc, int32_t* __restrict__ assign,
                     float* __restrict__ dist2, double* __restrict__ llpart, int vec) {
  constexpr int DP = 32 * DT, Q = DP / 4, XS = DP + 4;
  extern __shared__ __align__(16) float smem[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, c = lane & 31;
  const int nthr = blockDim.x;
  const int KS = waves * 32, SCS = KS + 8;
  const int64_t chunk = blockIdx.x;
  float* xs = smem;                                      // [64][XS] X tile
  float* sc = xs + 64 * XS;                              // [64][SCS] scores of one slab
  float* xq = sc + 64 * SCS;                             // [64][2] |x|^2 and |x|_1 of the tile's rows
  double* bestd = reinterpret_cast<double*>(xq + 128);   // [64] the row's nearest distance so far
  double* lls = bestd + 64;                              // [nthr]
  double* rd2 = lls + nthr;                              // [waves][kRefCap] exact candidate distances
  int* bestk = reinterpret_cast<int*>(rd2 + waves * kRefCap);        // [64] and its centre
  uint32_t* reflist = reinterpret_cast<uint32_t*>(bestk + 64);      // [waves][kRefCap]

  const int tpr = waves;
  const int prow = tid / tpr, psub = tid - prow * tpr;
  const float a_max = errc[0], b_max = errc[1], c_max = errc[2], b2_max = errc[3];
  // fp32 score error bound in natural units (as in the statistics kernel);
  // the base-2 scores are off by at most log2(e) times that
  const float gam = (float)(2 * DP + 4) * kUnitRound * kBoundSlack;
  double ll_acc = 0.0;

  const int64_t lo = chunk * rows_per_chunk;
  const int64_t hi = min(N, lo + rows_per_chunk);
  // fp32 rows (vec == 1) and half-precision rows (vec == 2): the next tile
  // is fetched into registers (16-byte chunks tid + nthr * i) while the rows
  // of this one are decided, and written to LDS once the tile is done (half
  // values widened there); other inputs load at the end of the tile.
  const int nch = 16 * DP / nthr;
  const bool pref = vec == 1 && sizeof(XT) == 4 && nch <= 8 && nch * nthr == 16 * DP;
  const int nhc = 8 * DP, nh = (nhc + nthr - 1) / nthr;  // half rows: chunks of eight values
  const bool hpref = vec == 2 && sizeof(XT) == 2 && nh <= 8;
  float4 xpre[8];
  auto chunk_at = [&](int i, int& row, int& q) {
    const int ch = tid + nthr * i;
    row = ch / Q;
    q = ch - row * Q;
  };
  load_x_tile<XS>(xs, X, lo, hi, d, DP, tid, nthr, vec);
  for (int64_t r0 = lo; r0 < hi; r0 += 64) {
    const int64_t rn = r0 + 64;
    for (int slab = 0; slab < kslabs; ++slab) {
      const int k0 = slab * KS, kw = k0 + wave * 32;
      __syncthreads();  // the tile's X is in LDS; the previous slab is done with the score tile
      const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float4*>(W32p) + (size_t)(__builtin_amdgcn_readfirstlane(kw) >> 5) * Q * 64, (short)0,
          Q * 64 * 16, kBufferRsrcWord3);
      score_tile<DT, true>(xs, sc, xq, wrs, c32[kw + c], wave, lane, SCS);
      __syncthreads();
      if (slab == 0 && pref && rn < hi) {
        const float* Xf = reinterpret_cast<const float*>(X);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (i < nch) {
            int row, q;
            chunk_at(i, row, q);
            const int64_t gr = rn + row;
            xpre[i] = (gr < hi && 4 * q < d) ? *reinterpret_cast<const float4*>(Xf + gr * d + 4 * q)
                                             : make_float4(0.f, 0.f, 0.f, 0.f);
          }
      }
      if (sizeof(XT) == 2 && slab == 0 && hpref && rn < hi) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int ch = tid + nthr * i, row = ch / (DP / 8), q = ch - row * (DP / 8);
          const int64_t gr = rn + row;
          if (i < nh)
            xpre[i] = (ch < nhc && gr < hi && 8 * q < d)
                          ? __builtin_bit_cast(float4, *reinterpret_cast<const uint4*>(X + gr * d + 8 * q))
                          : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }

      const int row = prow;
      const bool valid = r0 + row < hi;
      const float sq = xq[2 * row], ab = xq[2 * row + 1];
      const float Ebound = gam * (a_max * sq + fminf(b_max * ab, b2_max * sqrtf(sq))) + 2.f * kUnitRound * c_max;
      const float4* srow4 = reinterpret_cast<const float4*>(sc + row * SCS);
      float4 ev[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) ev[i] = srow4[psub + tpr * i];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fmaxf(fmaxf(ev[i].x, ev[i].y), fmaxf(ev[i].z, ev[i].w)));
      const float m = group_max(mx, tpr);
      // Two base-2 scores, each off by at most log2(e) E < 1.45 E, can swap
      // order only within 2.9 E; the subtraction's own rounding is covered by
      // the last term. Padding centres score -inf and never qualify.
      const float thr = m - (2.9f * Ebound + 4.f * kUnitRound * fabsf(m));
      uint32_t mask = 0;
      if (valid)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          mask |= (ev[i].x >= thr ? 1u : 0u) << (4 * i);
          mask |= (ev[i].y >= thr ? 1u : 0u) << (4 * i + 1);
          mask |= (ev[i].z >= thr ? 1u : 0u) << (4 * i + 2);
          mask |= (ev[i].w >= thr ? 1u : 0u) << (4 * i + 3);
        }
      double bd = INFINITY;
      int bk = INT_MAX;
      {
        const int cnt = __popc(mask);
        const int incl = wave_incl_scan(cnt);
        const int total = __builtin_amdgcn_readlane(incl, 63);
        const int base = incl - cnt;
        uint32_t* wl = reflist + wave * kRefCap;
        double* wd = rd2 + wave * kRefCap;
        for (int p0 = 0; p0 < total; p0 += kRefCap) {
          {
            uint32_t m2 = mask;
            int pos = base;
            while (m2) {
              const int i = __ffs(m2) - 1;
              m2 &= m2 - 1u;
              if (pos >= p0 && pos < p0 + kRefCap)
                wl[pos - p0] = ((uint32_t)row << 16) | (uint32_t)(4 * (psub + tpr * (i >> 2)) + (i & 3));
              ++pos;
            }
          }
          wave_lds_sync();
          const int n = min(total - p0, kRefCap);
          // LPE lanes per candidate (16 or 12 contiguous features each), so
          // that short rows take few passes; all loads are issued before the
          // arithmetic (inactive lanes read entry 0)
          constexpr int LPE = DT == 1 ? 2 : DT == 2 ? 4 : 8, FPL = DP / LPE, EPP = 64 / LPE;
          static_assert(FPL % 4 == 0, "float4 pieces");
          for (int e0 = 0; e0 < n; e0 += EPP) {
            const int e = e0 + lane / LPE, sl = lane % LPE;
            const bool act = e < n;
            const uint32_t ent = act ? wl[e] : 0u;
            const int er = (int)(ent >> 16), kg = k0 + (int)(ent & 0xffffu);
            const float4* xr = reinterpret_cast<const float4*>(xs + er * XS + sl * FPL);
            const float4* mr = reinterpret_cast<const float4*>(mup + (size_t)kg * DP + sl * FPL);
            float4 mv[FPL / 4];
#pragma unroll
            for (int i = 0; i < FPL / 4; ++i) mv[i] = mr[i];
            __builtin_amdgcn_sched_barrier(0);
            // features past d are skipped
            double a0 = 0.0, a1 = 0.0;
#pragma unroll
            for (int i = 0; i < FPL / 4; ++i) {
              const float4 xv = xr[i];
              const int f = sl * FPL + 4 * i;
              const double t0 = f < d ? (double)xv.x - (double)mv[i].x : 0.0;
              const double t1 = f + 1 < d ? (double)xv.y - (double)mv[i].y : 0.0;
              const double t2 = f + 2 < d ? (double)xv.z - (double)mv[i].z : 0.0;
              const double t3 = f + 3 < d ? (double)xv.w - (double)mv[i].w : 0.0;
              a0 = fma(t0, t0, a0);
              a1 = fma(t1, t1, a1);
              a0 = fma(t2, t2, a0);
              a1 = fma(t3, t3, a1);
            }
            double acc = a0 + a1;
            acc += dpp_d<kDppXor1>(acc);
            if (LPE >= 4) acc += dpp_d<kDppXor2>(acc);
            if (LPE >= 8) acc += dpp_d<kDppHalfMirror>(acc);
            if (act && sl == 0) wd[e] = acc;
          }
          wave_lds_sync();
          // each thread takes the distances of its own candidates of this pass,
          // in increasing centre order (a strict < keeps the lower index)
          {
            uint32_t m2 = mask;
            int pos = base;
            while (m2) {
              const int i = __ffs(m2) - 1;
              m2 &= m2 - 1u;
              if (pos >= p0 && pos < p0 + kRefCap) {
                const double dd = wd[pos - p0];
                if (dd < bd) {
                  bd = dd;
                  bk = k0 + 4 * (psub + tpr * (i >> 2)) + (i & 3);
                }
              }
              ++pos;
            }
          }
          wave_lds_sync();
        }
      }
      // the row's threads are `tpr` consecutive lanes of one wave
      for (int o = 1; o < tpr; o <<= 1) {
        const double od = __shfl_xor(bd, o, 64);
        const int ok = __shfl_xor(bk, o, 64);
        if (od < bd || (od == bd && ok < bk)) {
          bd = od;
          bk = ok;
        }
      }
      if (psub == 0 && (slab == 0 || bd < bestd[row])) {
        bestd[row] = bd;
        bestk[row] = bk;
      }
    }
    __syncthreads();
    if (tid < 64 && r0 + tid < hi) {
      const double b = bestd[tid];
      const int k = bestk[tid];
      assign[r0 + tid] = k < K ? k : -1;  // -1 only for a row with a NaN score
      if (dist2) dist2[r0 + tid] = (float)b;  // optional output
      ll_acc += b;
    }
    if (rn < hi) {
      if (pref) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (i < nch) {
            int row, q;
            chunk_at(i, row, q);
            *reinterpret_cast<float4*>(xs + row * XS + 4 * q) = xpre[i];
          }
      } else if (sizeof(XT) == 2 && hpref) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int ch = tid + nthr * i, row = ch / (DP / 8), q = ch - row * (DP / 8);
          if (i < nh && ch < nhc) {
            const uint4 raw = __builtin_bit_cast(uint4, xpre[i]);
            const XT* hv = reinterpret_cast<const XT*>(&raw);
            *reinterpret_cast<float4*>(xs + row * XS + 8 * q) =
                make_float4((float)hv[0], (float)hv[1], (float)hv[2], (float)hv[3]);
            *reinterpret_cast<float4*>(xs + row * XS + 8 * q + 4) =
                make_float4((float)hv[4], (float)hv[5], (float)hv[6], (float)hv[7]);
          }
        }
      } else {
        load_x_tile<XS>(xs, X, rn, hi, d, DP, tid, nthr, vec);
      }
    }
  }
  lls[tid] = ll_acc;
  __syncthreads();
  if (tid == 0) {
    double s = 0.0;
    for (int i = 0; i < nthr; ++i) s += lls[i];
    llpart[chunk] = s;
  }
}


// ---------------------------------------------------------------------------
// Small-K single sweep (K <= 16, d <= 64): 16x16x4 f32 MFMA tiles
// ---------------------------------------------------------------------------
//
// Every wave owns all (at most 16) components and works alone on the 64-point
// tiles of its own row range; waves only meet at the start (parameters into
// LDS) and at the end (statistics partial of the block). Per tile:
//  1. the X tile goes to the wave's LDS tile (prefetched in registers one
//     tile ahead for fp32 rows of at most 32 features);
//  2. scores: four 16x16x4 MFMA chains, one per 16-point group, with the
//     score operands (16 components x 2d, base-2 scaled) in registers; the
//     accumulators go to the wave's LDS score tile [64][SS];
//  3. row phase with one lane per point: max, e = 2^(s - m), z, the fp32
//     error bound and the re-score flags, all in registers; flagged entries
//     are re-scored exactly (fp64 difference form, one lane per entry);
//     r = e / z goes back to the score tile;
//  4. statistics: 16x16x4 MFMAs with r (component c, point slot g) as the A
//     operand and x or x^2 of those points as B.

// exp(x) for x <= ~0 through the hardware exp2 (1 ulp): the relative error is
// ~|x| * 2^-24 * log2(e) from rounding x*log2(e), i.e. an absolute error in
// exp(x) of at most ~3e-8 over x <= 0.
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }

// Per wave: a 64-point tile of X [64][XS] and a score/responsibility tile
// [64][SS] in LDS. Scores come from four 16x16x4 blocks; the row phase then
// runs one point per lane (in-lane max / sum over the <= 16 components), and
// the statistics MFMAs read r back in the accumulator layout.
template <int DS>
struct SmallTile {
  static constexpr int DP = 16 * DS, XS = DP + 4, SS = 20;
  static constexpr int XF = 64 * XS, SF = 64 * SS;  // floats per wave
  static constexpr int PF = DS <= 2 ? DP / 4 : 0;   // float4 per lane prefetched in registers
  // exact re-score: lanes per entry and features per lane
  static constexpr int LPE = DS == 1 ? 1 : (DS == 2 ? 2 : 4), FPL = DP / LPE;
};

// Two blocks per CU (two waves per SIMD): at most 256 registers per lane.
template <int DS, typename XT, bool SPLIT>
__global__ void __launch_bounds__(256, 2)
estep_small_kernel(const XT* __restrict__ X, int64_t N, int d, int K, int64_t wave_rows,
                   const double* __restrict__ W64p, const double* __restrict__ c64e,
                   const float* __restrict__ mu, const double* __restrict__ iv64,
                   const double* __restrict__ c64d, const float* __restrict__ errc,
                   float* __restrict__ partials, double* __restrict__ llpart,
                   float* __restrict__ ll_point, float* __restrict__ R, int vec) {
  using T = SmallTile<DS>;
  constexpr int DP = T::DP, S = DP / 2, XS = T::XS, SS = T::SS, E = 1 + 2 * DP;
  // Row stride (doubles) of the re-score parameters, padded so that one lane
  // per entry reading 16-byte pieces of different components' rows spreads
  // over the banks.
  constexpr int MS = DP + 2;
  __shared__ __align__(16) float tiles[kSmallWaves][T::XF + T::SF];
  __shared__ __align__(16) double mus[16 * MS];
  __shared__ __align__(16) double ivs[16 * MS];
  __shared__ double cds[16];
  __shared__ double lls[kSmallWaves];
  __shared__ float rowm[kSmallWaves][64];
  __shared__ uint32_t elist[kSmallWaves][64];
  static_assert(16 * E <= T::XF + T::SF, "the block partial is staged in the tile space");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;

  for (int i = tid; i < 16 * DP; i += blockDim.x) {
    const int k = i / DP, f = i - k * DP;
    const bool in = k < K && f < d;
    mus[k * MS + f] = in ? (double)mu[(size_t)k * d + f] : 0.0;
    ivs[k * MS + f] = in ? iv64[(size_t)k * d + f] : 0.0;
  }
  if (tid < 16) cds[tid] = tid < K ? c64d[tid] : 0.0;
  __syncthreads();

  // Score operands in registers. Step s pairs lane (g, c) with feature
  // g*(DP/4) + s/2, as x^2 on even steps and x on odd steps: each lane reads
  // its point's features contiguously and squares each once. W64p holds
  // feature f, part t (A, B) of component c at ((2*(f/4) + t)*4 + f%4)*16 + c.
  // Operands and constants are scaled by log2(e) before rounding to fp32, so
  // the scores come out in base-2 units and e = 2^(s - m) needs no multiply.
  // Every fp32 operand is still the correctly rounded value of an exact one,
  // so the error bound below holds for the scaled scores with each maximum
  // scaled alike; it is applied in natural units, where it is unchanged.
  float w[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int f = g * (DP / 4) + (s >> 1);
    w[s] = (float)(W64p[((2 * (f >> 2) + (s & 1)) * 4 + (f & 3)) * 16 + c] * kLog2E);
  }
  float cks[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) cks[k] = (float)(c64e[k] * kLog2E);
  const float a_max = errc[0], c_max = errc[2], b2_max = errc[3];
  const float gam = (float)(2 * DP + 4) * kUnitRound * kBoundSlack;

  v4f SX[DS], SXX[DS];
#pragma unroll
  for (int t = 0; t < DS; ++t) SX[t] = SXX[t] = (v4f){0.f, 0.f, 0.f, 0.f};
  float nk = 0.f;
  double ll = 0.0;

  float* xs = &tiles[wave][0];
  float* sc = &tiles[wave][T::XF];
  const int64_t wid = (int64_t)blockIdx.x * kSmallWaves + wave;
  const int64_t lo = wid * wave_rows;
  const int64_t hi = min(N, lo + wave_rows);
  const bool pf = vec && sizeof(XT) == 4 && T::PF > 0;
  const float* Xf = reinterpret_cast<const float*>(X);

  // register prefetch of a 64-row tile: float4 chunk ch = 64 i + lane is row
  // ch / (DP/4), features 4 (ch % (DP/4)); rows past hi and features past d
  // read as zero.
  float4 pre[T::PF > 0 ? T::PF : 1];
  auto fetch = [&](int64_t r) {
    if (d == DP && r + 64 <= hi) {  // a whole tile of unpadded rows: 64 * DP contiguous floats
      const float4* src = reinterpret_cast<const float4*>(Xf + r * DP) + lane;
#pragma unroll
      for (int i = 0; i < T::PF; ++i) pre[i] = src[64 * i];
      return;
    }
#pragma unroll
    for (int i = 0; i < T::PF; ++i) {
      const int ch = 64 * i + lane;
      const int row = ch / (DP / 4), q = ch - row * (DP / 4);
      const int64_t gr = r + row;
      pre[i] = (gr < hi && 4 * q < d) ? *reinterpret_cast<const float4*>(Xf + gr * d + 4 * q)
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  if (pf && lo < hi) fetch(lo);

  for (int64_t r0 = lo; r0 < hi; r0 += 64) {
    // 1. X tile -> LDS (prefetched registers, or direct loads), next tile requested
    if (pf) {
#pragma unroll
      for (int i = 0; i < T::PF; ++i) {
        const int ch = 64 * i + lane;
        const int row = ch / (DP / 4), q = ch - row * (DP / 4);
        *reinterpret_cast<float4*>(xs + row * XS + 4 * q) = pre[i];
      }
      if (r0 + 64 < hi) fetch(r0 + 64);
    } else {
      for (int e = lane; e < 64 * DP; e += 64) {
        const int row = e / DP, f = e - row * DP;
        const int64_t gr = r0 + row;
        xs[row * XS + f] = (gr < hi && f < d) ? load_x(X, gr * d + f) : 0.f;
      }
    }
    wave_lds_sync();

    // The MFMA phases run at raised wave priority, so that a wave issuing
    // MFMAs is preferred while the other wave of the SIMD does VALU work.
    __builtin_amdgcn_s_setprio(1);
    // 2. scores, 16-point block b: lane (g, c) supplies point 16b + c,
    //    feature g*(DP/4) + s/2; accumulator slot j = point 16b+4g+j. The
    //    squares the MFMAs consume are also summed: after the sum over the
    //    four lanes g of a point, lane (g = b, c) keeps |x|^2 of point
    //    16b + c, the point it takes in the row phase.
    float sq = 0.f;
    {
      // the four blocks' operands first (one LDS round trip), then their four
      // MFMA chains interleaved
      float xa[4][DP / 4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int q = 0; q < DP / 16; ++q) {
          const float4 v = *reinterpret_cast<const float4*>(xs + (16 * b + c) * XS + g * (DP / 4) + 4 * q);
          xa[b][4 * q] = v.x;
          xa[b][4 * q + 1] = v.y;
          xa[b][4 * q + 2] = v.z;
          xa[b][4 * q + 3] = v.w;
        }
      __builtin_amdgcn_sched_barrier(0);
      v4f acc[4];
      float sqb[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        acc[b] = (v4f){0.f, 0.f, 0.f, 0.f};
        sqb[b] = 0.f;
      }
#pragma unroll
      for (int u = 0; u < DP / 4; ++u) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float x2 = xa[b][u] * xa[b][u];
          sqb[b] += x2;
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(x2, w[2 * u], acc[b], 0, 0, 0);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[b][u], w[2 * u + 1], acc[b], 0, 0, 0);
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        float v = sqb[b];
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        if (g == b) sq = v;
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[(16 * b + 4 * g + j) * SS + c] = acc[b][j];
      }
    }
    __builtin_amdgcn_s_setprio(0);
    wave_lds_sync();

    // 3. row phase: lane = point
    {
      const int p = lane;
      const int64_t gr = r0 + p;
      const bool valid = gr < hi;
      float e[16];
      float m = -INFINITY;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(sc + p * SS + 4 * q);
        e[4 * q] = v.x + cks[4 * q];
        e[4 * q + 1] = v.y + cks[4 * q + 1];
        e[4 * q + 2] = v.z + cks[4 * q + 2];
        e[4 * q + 3] = v.w + cks[4 * q + 3];
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) m = fmaxf(m, e[k]);
      float z = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        e[k] = __builtin_amdgcn_exp2f(e[k] - m);
        z += e[k];
      }
      // sq = |x|^2 of point p, from the score loop (its fp32 sum order differs
      // from a row-wise sum by rounding only, which the bound's factor covers)
      // re-score rule of the single sweep (see the main kernel): refine entries
      // with 2 E r (1 - r) > tau; widen to the e >= kExpWindow window if the unrefined
      // mass could still move the refined ones by more than tau.
      const float Eb = gam * (a_max * sq + b2_max * __builtin_sqrtf(sq)) + 2.f * kUnitRound * c_max;
      const float thr2 = kGateTau * z * z * __builtin_amdgcn_rcpf(2.f * Eb);  // on e (z - e)
      uint32_t mask = 0;
      float unref = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const bool fl = valid && e[k] * (z - e[k]) > thr2;
        mask |= (fl ? 1u : 0u) << k;
        unref += fl ? 0.f : e[k];
      }
      if (mask && Eb * unref > kGateTau * z) {
        mask = 0;
#pragma unroll
        for (int k = 0; k < 16; ++k) mask |= (valid && e[k] >= kExpWindow ? 1u : 0u) << k;
      }
      // Exact re-score (fp64 difference form) of the wave's flagged entries:
      // e goes to the score tile, the entries to an LDS list, and LPE lanes
      // re-score one entry (FPL features each, partial sums combined by DPP).
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(sc + p * SS + 4 * q) = make_float4(e[4 * q], e[4 * q + 1], e[4 * q + 2], e[4 * q + 3]);
      rowm[wave][p] = m;
      if (__ballot(mask != 0)) {
        const int cnt = __popc(mask);
        const int incl = wave_incl_scan(cnt);
        const int total = __builtin_amdgcn_readlane(incl, 63);
        const int base = incl - cnt;
        for (int p0 = 0; p0 < total; p0 += 64) {
          uint32_t m2 = mask;
          int pos = base;
          while (m2) {
            const int k = __ffs(m2) - 1;
            m2 &= m2 - 1u;
            if (pos >= p0 && pos < p0 + 64) elist[wave][pos - p0] = ((uint32_t)p << 4) | (uint32_t)k;
            ++pos;
          }
          wave_lds_sync();
          constexpr int LPE = T::LPE, FPL = T::FPL, EPR = 64 / LPE;
          const int n = min(total - p0, 64), part = lane % LPE;
          for (int e0 = 0; e0 < n; e0 += EPR) {
            const int ei = e0 + lane / LPE;
            const uint32_t ent = ei < n ? elist[wave][ei] : 0u;
            const int ep = (int)(ent >> 4), ek = (int)(ent & 15u);
            const float* xr = xs + ep * XS + part * FPL;
            const double* mr = mus + ek * MS + part * FPL;
            const double* ir = ivs + ek * MS + part * FPL;
            double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;  // features >= d carry 1/var = 0
#pragma unroll 2
            for (int q = 0; q < FPL / 4; ++q) {
              const float4 xv = *reinterpret_cast<const float4*>(xr + 4 * q);
              const double2 m01 = *reinterpret_cast<const double2*>(mr + 4 * q);
              const double2 m23 = *reinterpret_cast<const double2*>(mr + 4 * q + 2);
              const double2 i01 = *reinterpret_cast<const double2*>(ir + 4 * q);
              const double2 i23 = *reinterpret_cast<const double2*>(ir + 4 * q + 2);
              const double t0 = (double)xv.x - m01.x, t1 = (double)xv.y - m01.y;
              const double t2 = (double)xv.z - m23.x, t3 = (double)xv.w - m23.y;
              a0 = fma(t0 * t0, i01.x, a0);
              a1 = fma(t1 * t1, i01.y, a1);
              a2 = fma(t2 * t2, i23.x, a2);
              a3 = fma(t3 * t3, i23.y, a3);
            }
            double a = (a0 + a1) + (a2 + a3);
            if (LPE >= 2) a += dpp_d<kDppXor1>(a);
            if (LPE >= 4) a += dpp_d<kDppXor2>(a);
            if (ei < n && part == 0)
              sc[ep * SS + ek] = __builtin_amdgcn_exp2f((float)((cds[ek] - 0.5 * a) * kLog2E - (double)rowm[wave][ep]));
          }
          wave_lds_sync();
        }
        if (mask) {
          z = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 v = *reinterpret_cast<const float4*>(sc + p * SS + 4 * q);
            z += (v.x + v.y) + (v.z + v.w);
          }
        }
      }
      // r = e / z in place (e is read back from the tile, so it need not stay
      // in registers across the re-score)
      const float inv = valid ? __builtin_amdgcn_rcpf(z) : 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4 v = *reinterpret_cast<float4*>(sc + p * SS + 4 * q);
        v.x *= inv;
        v.y *= inv;
        v.z *= inv;
        v.w *= inv;
        *reinterpret_cast<float4*>(sc + p * SS + 4 * q) = v;
      }
      if (valid) {
        const double l = ((double)m + (double)__builtin_amdgcn_logf(z)) * kLn2;  // logf is log2
        ll += l;
        if (ll_point) ll_point[gr] = (float)l;
        if (R)
          for (int k = 0; k < K; ++k) R[gr * K + k] = sc[p * SS + k];
      }
    }
    wave_lds_sync();

    __builtin_amdgcn_s_setprio(1);
    if constexpr (!SPLIT) {
      // 4. statistics: step j of block b uses r of point 16b + 4g + j (component c)
      // operands of all 16 steps first (one LDS round trip), then the MFMAs
      float rr[16], xx[16][DS];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int p = 16 * (q >> 2) + 4 * g + (q & 3);
        rr[q] = sc[p * SS + c];
#pragma unroll
        for (int t = 0; t < DS; ++t) xx[q][t] = xs[p * XS + 16 * t + c];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        nk += rr[q];
#pragma unroll
        for (int t = 0; t < DS; ++t) {
          SX[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(rr[q], xx[q][t], SX[t], 0, 0, 0);
          SXX[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(rr[q], xx[q][t] * xx[q][t], SXX[t], 0, 0, 0);
        }
      }
    } else {
      // 4. statistics as split-bf16 products on the bf16 MFMA (16x16x32): each
      //    fp32 operand v = hi + lo + d with hi = bf16(v), lo = bf16(v - hi),
      //    |d| <= 2^-16 |v|, and a*b is taken as hi*hi + hi*lo + lo*hi (exact
      //    products, fp32 accumulation): per product |error| <= 3.0001 * 2^-16 |a b|
      //    before the accumulation's rounding. Block kb covers points
      //    32 kb + 8 g + t (t < 8) of lane (g, c): r of component c is the A
      //    operand, x or x^2 of feature 16 t2 + c the B operand.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float rr[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          rr[t] = sc[(32 * kb + 8 * g + t) * SS + c];
          nk += rr[t];
        }
        v8bf rh, rl;
        split_bf16(rr, rh, rl);
#pragma unroll
        for (int t2 = 0; t2 < DS; ++t2) {
          float xx[8], x2[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            xx[t] = xs[(32 * kb + 8 * g + t) * XS + 16 * t2 + c];
            x2[t] = xx[t] * xx[t];
          }
          v8bf xh, xl, qh, ql;
          split_bf16(xx, xh, xl);
          split_bf16(x2, qh, ql);
          SX[t2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rh, xh, SX[t2], 0, 0, 0);
          SXX[t2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rh, qh, SXX[t2], 0, 0, 0);
          SX[t2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rh, xl, SX[t2], 0, 0, 0);
          SXX[t2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rh, ql, SXX[t2], 0, 0, 0);
          SX[t2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rl, xh, SX[t2], 0, 0, 0);
          SXX[t2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rl, qh, SXX[t2], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
    wave_lds_sync();  // the tiles are rewritten by the next iteration
  }

  // block partial: waves -> LDS (own tile space) -> fixed-order sum
  float* ws = &tiles[wave][0];
#pragma unroll
  for (int t = 0; t < DS; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int comp = 4 * g + j, f = 16 * t + c;
      ws[comp * E + 1 + f] = SX[t][j];
      ws[comp * E + 1 + DP + f] = SXX[t][j];
    }
  nk += __shfl_xor(nk, 16, 64);
  nk += __shfl_xor(nk, 32, 64);
  if (g == 0) ws[c * E] = nk;
  for (int o = 1; o < 64; o <<= 1) ll += __shfl_xor(ll, o, 64);
  if (lane == 0) lls[wave] = ll;
  __syncthreads();
  float* part = partials + (size_t)blockIdx.x * 16 * E;
  for (int i = tid; i < 16 * E; i += blockDim.x) {
    float a = 0.f;
    for (int v = 0; v < kSmallWaves; ++v) a += tiles[v][i];
    part[i] = a;
  }
  if (tid == 0) {
    double a = 0.0;
    for (int v = 0; v < kSmallWaves; ++v) a += lls[v];
    llpart[blockIdx.x] = a;
  }
}

// ---------------------------------------------------------------------------
// fp64 MFMA score pass: top-2 assignment, and the normaliser of the rows the
// fp32 first pass's merge could not settle
// ---------------------------------------------------------------------------
//
// Block = 4 waves, one 64-point tile. With NP = 4, wave w takes the
// 16-component tiles w, w+4, ... for all four 16-point groups; with fewer
// component tiles (NP = 2 or 1) the component tiles are dealt to NP wave
// classes and each wave takes NP of the point groups, so that no wave idles.
// Scores come from 16x16x4 f64 MFMAs (layout: D[comp][point]),
// so each lane holds four components of one point per accumulator and keeps
// an online (max, sum of exp) per point; lanes and waves are merged at the
// end in a fixed order. The sum takes fp32 exponentials of the fp64
// differences (each within about one fp32 ulp), so l carries about 1e-7
// relative error on top of fp64 scores. Output per row: (m_ref, lZ) with m_ref = fp32 of the
// row max and lZ = l - m_ref, the per-point l, and optionally the top-2.
__device__ __forceinline__ bool better(double v, int i, double w, int j) {
  return v > w || (v == w && i < j);
}
__device__ __forceinline__ void lse_merge(double& m, double& z, double mo, double zo) {
  const double mn = fmax(m, mo);
  if (mn == -INFINITY) return;
  z = (m == -INFINITY ? 0.0 : z * exp(m - mn)) + (mo == -INFINITY ? 0.0 : zo * exp(mo - mn));
  m = mn;
}
__device__ __forceinline__ void top2_insert(double v, int i, double& v1, int& i1, double& v2, int& i2) {
  if (better(v, i, v1, i1)) {
    v2 = v1;
    i2 = i1;
    v1 = v;
    i1 = i;
  } else if (better(v, i, v2, i2)) {
    v2 = v;
    i2 = i;
  }
}

// Four waves per SIMD (at most 128 registers): the fp64 MFMA chains of four
// blocks per CU hide each other's LDS and L2 latency.
// Rows: the 64 consecutive rows of the block (rows == nullptr), or, as the
// fallback of the fp32 first pass, slots blockIdx.x * 64 + t of the row list
// `rows` (its length in *nrows; blocks past it return at once).
template <int DT, bool TOP2, typename XT, int NP>
__global__ void __launch_bounds__(256, 4)
estep_lse_kernel(const XT* __restrict__ X, int64_t N, int d, int K, int Kp16,
                 const double* __restrict__ W64p, const double* __restrict__ c64e,
                 const int32_t* __restrict__ rows, const int32_t* __restrict__ nrows,
                 const float* __restrict__ rowE, float4* __restrict__ rowref, double* __restrict__ lrow,
                 int32_t* __restrict__ tidx, float* __restrict__ tresp) {
  constexpr int DP = 32 * DT, S = DP / 2, XS = DP + 1;
  __shared__ float xs[64 * XS];
  __shared__ double sm[kLseWaves][64], sz[kLseWaves][64], sv1[kLseWaves][64], sv2[kLseWaves][64];
  __shared__ int si1[kLseWaves][64], si2[kLseWaves][64];
  __shared__ int64_t srow[64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int64_t nr = rows ? (int64_t)*nrows : N;
  if (r0 >= nr) return;
  if (tid < 64) srow[tid] = r0 + tid < nr ? (rows ? (int64_t)rows[r0 + tid] : r0 + tid) : -1;
  __syncthreads();

  for (int e = tid; e < 64 * DP; e += blockDim.x) {
    const int row = e / DP, f = e - row * DP;
    const int64_t gr = srow[row];
    xs[row * XS + f] = (gr >= 0 && f < d) ? load_x(X, gr * d + f) : 0.f;
  }
  __syncthreads();

  // this wave's point groups: pg + i * (4 / NP), i < NP
  constexpr int PS = 4 / NP;
  const int pg = wave / NP;
  double m[NP], z[NP], v1[NP], v2[NP];
  int i1[NP], i2[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    m[p] = -INFINITY;
    z[p] = 0.0;
    v1[p] = v2[p] = -INFINITY;
    i1[p] = i2[p] = 0x7fffffff;
  }
  const int Kt = Kp16 / 16;
  // Score operands through a buffer resource (opaque to the IR optimiser, so
  // the prefetch below stays a prefetch), two steps ahead in two register
  // pairs that swap roles; the last steps of a component tile prefetch the
  // first steps of the wave's next tile (offsets past the end read zero).
  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<double*>(W64p), (short)0, Kt * S * 64 * 8, kBufferRsrcWord3);
  auto wl = [&](int kt, int s) {
    return __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(wrs, ((kt * S + s) * 64 + lane) * 8, 0, 0));
  };
  static_assert(S % 4 == 0, "the score loop takes four steps at a time");
  int kt = wave % NP;
  double wa = wl(kt, 0), wb = wl(kt, 1);
  for (; kt < Kt; kt += NP) {
    double ce[4];
    int comp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      comp[j] = kt * 16 + 4 * j + g;
      ce[j] = c64e[comp[j]];
    }
    v4d D[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) D[p] = (v4d){0.0, 0.0, 0.0, 0.0};
    // Feature block j (features 4j..4j+3; lane group g takes feature 4j + g
    // of its point): the x^2 step with the operands of step 2j, then the x
    // step with those of step 2j + 1. Each lane converts and squares only its
    // own x.
    auto block = [&](int j, double asq, double alin) {
      double xv[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p) xv[p] = (double)xs[((pg + p * PS) * 16 + c) * XS + 4 * j + g];
#pragma unroll
      for (int p = 0; p < NP; ++p) D[p] = __builtin_amdgcn_mfma_f64_16x16x4f64(asq, xv[p] * xv[p], D[p], 0, 0, 0);
#pragma unroll
      for (int p = 0; p < NP; ++p) D[p] = __builtin_amdgcn_mfma_f64_16x16x4f64(alin, xv[p], D[p], 0, 0, 0);
    };
#pragma unroll 1
    for (int s = 0; s < S; s += 4) {
      const double wc = wl(kt, s + 2), wd = wl(kt, s + 3);
      __builtin_amdgcn_sched_barrier(0);
      block(s >> 1, wa, wb);
      __builtin_amdgcn_sched_barrier(0);
      wa = s + 4 < S ? wl(kt, s + 4) : wl(kt + NP, 0);
      wb = s + 4 < S ? wl(kt, s + 5) : wl(kt + NP, 1);
      __builtin_amdgcn_sched_barrier(0);
      block((s >> 1) + 1, wc, wd);
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      double s[4];
      double mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[j] = D[p][j] + ce[j];
        mx = fmax(mx, s[j]);
      }
      if (mx > m[p]) {
        z[p] = (m[p] == -INFINITY) ? 0.0 : z[p] * exp(m[p] - mx);
        m[p] = mx;
      }
      if (m[p] > -INFINITY)
#pragma unroll
        for (int j = 0; j < 4; ++j) z[p] += (double)expf((float)(s[j] - m[p]));
      if (TOP2)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (comp[j] < K) top2_insert(s[j], comp[j], v1[p], i1[p], v2[p], i2[p]);
    }
  }
  // merge the four lane groups that hold the same points
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const double mo = __shfl_xor(m[p], o, 64), zo = __shfl_xor(z[p], o, 64);
      lse_merge(m[p], z[p], mo, zo);
      if (TOP2) {
        const double w1 = __shfl_xor(v1[p], o, 64), w2 = __shfl_xor(v2[p], o, 64);
        const int j1 = __shfl_xor(i1[p], o, 64), j2 = __shfl_xor(i2[p], o, 64);
        top2_insert(w1, j1, v1[p], i1[p], v2[p], i2[p]);
        top2_insert(w2, j2, v1[p], i1[p], v2[p], i2[p]);
      }
    }
  }
  if (g == 0) {
    if (NP < 4)  // neutral values for the point groups this wave did not score
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sm[wave][q * 16 + c] = -INFINITY;
        sz[wave][q * 16 + c] = 0.0;
        if (TOP2) {
          sv1[wave][q * 16 + c] = sv2[wave][q * 16 + c] = -INFINITY;
          si1[wave][q * 16 + c] = si2[wave][q * 16 + c] = 0x7fffffff;
        }
      }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int q = pg + p * PS;
      sm[wave][q * 16 + c] = m[p];
      sz[wave][q * 16 + c] = z[p];
      if (TOP2) {
        sv1[wave][q * 16 + c] = v1[p];
        sv2[wave][q * 16 + c] = v2[p];
        si1[wave][q * 16 + c] = i1[p];
        si2[wave][q * 16 + c] = i2[p];
      }
    }
  }
  __syncthreads();
  if (tid < 64) {
    double mm = sm[0][tid], zz = sz[0][tid];
    double a1 = TOP2 ? sv1[0][tid] : 0.0, a2 = TOP2 ? sv2[0][tid] : 0.0;
    int b1 = TOP2 ? si1[0][tid] : 0, b2 = TOP2 ? si2[0][tid] : 0;
    for (int w = 1; w < kLseWaves; ++w) {
      lse_merge(mm, zz, sm[w][tid], sz[w][tid]);
      if (TOP2) {
        top2_insert(sv1[w][tid], si1[w][tid], a1, b1, a2, b2);
        top2_insert(sv2[w][tid], si2[w][tid], a1, b1, a2, b2);
      }
    }
    const double l = mm + log(zz);
    const int64_t gr = srow[tid];
    if (gr >= 0) {
      if (rowref) {
        // (m, lZ, theta) in base 2 for the fp32 second pass: with this l (fp64
        // scores) an entry left unrefined is off by <= E r, so the entries
        // with r >= tau / E, i.e. s32 - m >= lZ + log2(tau / E), are re-scored
        const float mref = (float)(mm * kLog2E);
        const float lZ = (float)(l * kLog2E - (double)mref);
        const float E = fmaxf(rowE[gr], 1e-30f);
        rowref[gr] = make_float4(mref, lZ, lZ + log2f(kGateTau / E) - 1.f / 64, E);
        lrow[gr] = l;
      }
      if (TOP2) {
        tidx[2 * gr] = b1;
        tresp[2 * gr] = (float)exp(a1 - l);
        const bool has2 = b2 != 0x7fffffff;
        tidx[2 * gr + 1] = has2 ? b2 : -1;
        tresp[2 * gr + 1] = has2 ? (float)exp(a2 - l) : 0.f;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Reductions, M-step, fills
// ---------------------------------------------------------------------------

// Fixed-order fp64 sum over the P statistics partials of output element e
// (0: Nk, 1..d: Sx, d+1..2d: Sxx) of component k.
__device__ __forceinline__ double sum_partials(const float* __restrict__ partials, int64_t P, int Kp, int E,
                                               int DP, int d, int k, int e) {
  const int src = e == 0 ? 0 : (e <= d ? e : DP + (e - d));
  const float* p0 = partials + (size_t)k * E + src;
  const size_t stride = (size_t)Kp * E;
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  int64_t p = 0;
  for (; p + 4 <= P; p += 4) {
    s0 += p0[(p + 0) * stride];
    s1 += p0[(p + 1) * stride];
    s2 += p0[(p + 2) * stride];
    s3 += p0[(p + 3) * stride];
  }
  for (; p < P; ++p) s0 += p0[p * stride];
  return (s0 + s1) + (s2 + s3);
}

__global__ void reduce_stats_kernel(const float* __restrict__ partials, int64_t P, int Kp, int E, int DP,
                                    int K, int d, float* __restrict__ Nk, float* __restrict__ Sx,
                                    float* __restrict__ Sxx) {
  const int W = 1 + 2 * d;
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t >= (int64_t)K * W) return;
  const int k = (int)(t / W), e = (int)(t - (int64_t)k * W);
  const float s = (float)sum_partials(partials, P, Kp, E, DP, d, k, e);
  if (e == 0)
    Nk[k] = s;
  else if (e <= d)
    Sx[(size_t)k * d + e - 1] = s;
  else
    Sxx[(size_t)k * d + e - 1 - d] = s;
}

// Two-stage form for few outputs: segment g of the partials (in order) per
// thread, then the G segment sums per output, in order.
__global__ void reduce_stats_seg_kernel(const float* __restrict__ partials, int64_t P, int G, int Kp, int E,
                                        int DP, int K, int d, double* __restrict__ tmp) {
  const int W = 1 + 2 * d;
  const int64_t n = (int64_t)K * W;
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int g = blockIdx.y;
  if (t >= n) return;
  const int k = (int)(t / W), e = (int)(t - (int64_t)k * W);
  const int64_t p0 = P * g / G, p1 = P * (g + 1) / G;
  const size_t stride = (size_t)Kp * E;
  tmp[g * n + t] = sum_partials(partials + p0 * stride, p1 - p0, Kp, E, DP, d, k, e);
}

__global__ void reduce_stats_final_kernel(const double* __restrict__ tmp, int G, int K, int d,
                                          float* __restrict__ Nk, float* __restrict__ Sx,
                                          float* __restrict__ Sxx) {
  const int W = 1 + 2 * d;
  const int64_t n = (int64_t)K * W;
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t >= n) return;
  // in segment order; eight loads in flight at a time (the sum order is unchanged)
  double s = 0.0;
  int g = 0;
  for (; g + 8 <= G; g += 8) {
    double v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = tmp[(g + i) * n + t];
#pragma unroll
    for (int i = 0; i < 8; ++i) s += v[i];
  }
  for (; g < G; ++g) s += tmp[g * n + t];
  const int k = (int)(t / W), e = (int)(t - (int64_t)k * W);
  if (e == 0)
    Nk[k] = (float)s;
  else if (e <= d)
    Sx[(size_t)k * d + e - 1] = (float)s;
  else
    Sxx[(size_t)k * d + e - 1 - d] = (float)s;
}

// Row-chunked E-step: the statistics of one chunk of rows are added (in
// chunk order) to fp64 accumulators acc[k * (1 + 2d) + e], e as above.
__global__ void accum_stats_kernel(const float* __restrict__ partials, int64_t P, int Kp, int E, int DP, int K,
                                   int d, double* __restrict__ acc, int first) {
  const int W = 1 + 2 * d;
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t >= (int64_t)K * W) return;
  const int k = (int)(t / W), e = (int)(t - (int64_t)k * W);
  const double s = sum_partials(partials, P, Kp, E, DP, d, k, e);
  acc[t] = first ? s : acc[t] + s;
}

__global__ void finalize_stats_kernel(const double* __restrict__ acc, int K, int d, float* __restrict__ Nk,
                                      float* __restrict__ Sx, float* __restrict__ Sxx,
                                      double* __restrict__ loglik_total) {
  const int W = 1 + 2 * d;
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t == 0) loglik_total[0] = acc[(int64_t)K * W];
  if (t >= (int64_t)K * W) return;
  const int k = (int)(t / W), e = (int)(t - (int64_t)k * W);
  const float s = (float)acc[t];
  if (e == 0)
    Nk[k] = s;
  else if (e <= d)
    Sx[(size_t)k * d + e - 1] = s;
  else
    Sxx[(size_t)k * d + e - 1 - d] = s;
}

// One block of 256: fixed-order sum of n doubles, stored to out[0] (or, with
// accumulate, added to it).
template <bool ACCUM>
__global__ void reduce_ll_kernel(const double* __restrict__ part, int64_t n, double* __restrict__ out, int first) {
  __shared__ double s[256];
  const int64_t per = (n + 255) / 256;
  const int64_t lo = threadIdx.x * per, hi = min(n, lo + per);
  double a = 0.0;
  for (int64_t i = lo; i < hi; ++i) a += part[i];
  s[threadIdx.x] = a;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) s[threadIdx.x] += s[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = (!ACCUM || first) ? s[0] : out[0] + s[0];
}

__global__ void zero_outputs_kernel(float* __restrict__ Nk, float* __restrict__ Sx, float* __restrict__ Sxx,
                                    int d, int K, double* __restrict__ ll) {
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t Kd = (int64_t)K * d;
  if (t < K && Nk) Nk[t] = 0.f;
  if (t < Kd) {
    if (Sx) Sx[t] = 0.f;
    if (Sxx) Sxx[t] = 0.f;
  }
  if (t == 0 && ll) ll[0] = 0.0;
}

// One thread per (k, j): w = Nk/N, mu = Sx/Nk, var = max(Sxx/Nk - mu^2, floor).
__global__ void mstep_kernel(const float* __restrict__ Nk, const float* __restrict__ Sx,
                             const float* __restrict__ Sxx, double Nd, int d, int K, float var_floor,
                             float* __restrict__ mu, float* __restrict__ var, float* __restrict__ logw) {
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t >= (int64_t)K * d) return;
  const int k = (int)(t / d), j = (int)(t - (int64_t)k * d);
  const double nk = (double)Nk[k];
  if (j == 0) {
    const double nkc = nk < 1e-300 ? 1e-300 : nk;
    logw[k] = (float)log(nkc / Nd);
  }
  if (nk >= 1e-12 * Nd) {
    const double m = (double)Sx[t] / nk;
    double v = (double)Sxx[t] / nk - m * m;
    if (v < (double)var_floor) v = (double)var_floor;
    mu[t] = (float)m;
    var[t] = (float)v;
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

static inline unsigned nblocks(int64_t n, int b) { return (unsigned)((n + b - 1) / b); }

// Log-likelihood partials of an E-step: one per row chunk, or per kLlRows
// rows in the two-pass regime.
static inline int64_t ll_parts(const Plan& p) {
  return p.regime == 2 ? (p.N + kLlRows - 1) / kLlRows : p.P;
}

hipError_t launch_precompute(const Plan& p, const float* mu, const float* var, const float* logw,
                             hipStream_t stream) {
  const Workspace& w = p.ws;
  comp_consts_kernel<<<nblocks(p.Kp, 4), 256, 0, stream>>>(mu, var, logw, p.K, p.d, p.Kp, p.Kp16, w.c32,
                                                               w.c64e, w.c64d, w.compmax);
  pack_kernel<<<nblocks((int64_t)p.Kp * p.DP, 256), 256, 0, stream>>>(mu, var, p.K, p.d, p.Kp, p.Kp16, p.DP,
                                                                        w.W32p, w.W64p, w.iv64, w.mup, w.ivp);
  errc_kernel<<<1, 256, 0, stream>>>(w.compmax, p.K, w.errc);
  return hipGetLastError();
}

template <int DT, int MODE, typename XT>
static hipError_t run_stats(const Plan& p, const XT* X, const float* mu, float* ll_point, float* R,
                            hipStream_t stream) {
  const Workspace& w = p.ws;
  const int nthr = p.waves * 64;
  const int KS = p.waves * 32;
  // the first pass: one X tile and a 32-row score tile
  const size_t lds = MODE == 2 ? (size_t)(64 * (32 * DT + 4) + 32 * (KS + 8)) * sizeof(float)
                               : (size_t)(2 * 64 * (32 * DT + 4) + 64 * (KS + 8) + 256) * sizeof(float) +
                                     (size_t)nthr * sizeof(double) +
                                     (size_t)(p.waves * kRefCap + 64) * sizeof(uint32_t);
  const bool split = p.stats_split && MODE != 2;
  // exact fp16 splits of the second pass's statistics for half-precision X
  constexpr bool kF16 = MODE == 1 && std::is_same<XT, _Float16>::value;
  const bool f16 = kF16 && p.stats_f16 && !split;
  auto fn = p.waves == 8 ? (split ? estep_stats_kernel<DT, MODE, XT, 1, 8> : estep_stats_kernel<DT, MODE, XT, 0, 8>)
                         : (split ? estep_stats_kernel<DT, MODE, XT, 1, 0> : estep_stats_kernel<DT, MODE, XT, 0, 0>);
  auto fn16 = fn;
  if constexpr (kF16)
    fn16 = p.waves == 8 ? estep_stats_kernel<DT, MODE, XT, 2, 8> : estep_stats_kernel<DT, MODE, XT, 2, 0>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  if (f16) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn16), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  // The first pass accumulates nothing per chunk, so its chunks are cut for
  // one round of resident blocks (two per CU, 256 CUs): 8 * floor(64 /
  // slabs) chunks.
  int64_t chunks = p.P, rpc = p.rows_per_chunk;
  if (MODE == 2) {
    chunks = std::min<int64_t>(8 * std::max(1, 64 / p.kslabs), std::max<int64_t>(p.tiles, 1));
    rpc = (p.tiles + chunks - 1) / chunks * 64;
  }
  const unsigned grid = (unsigned)(chunks * p.kslabs);
  // 1: fp32 rows of d % 4 == 0 floats, 2: half-precision rows of d % 8 == 0
  // values, both 16-byte aligned; 0 otherwise
  const bool al16 = reinterpret_cast<uintptr_t>(X) % 16 == 0;
  const int vec = sizeof(XT) == 4 ? (p.d % 4 == 0 && al16 ? 1 : 0) : (p.d % 8 == 0 && al16 ? 2 : 0);
  const Pass1Out p1{w.p1h, w.p1v, w.p1k, w.rowE, w.rowSq};
  // the second pass walks the slabs' row lists, except when it also writes R
  const bool lists = MODE == 1 && p.pass1 && !R;
  // with f16: the fp16-split variant, then the fp32 one; each returns at
  // once unless the first pass's |x|^2 records select it
  const int32_t* xf = f16 ? w.xflag : nullptr;
  if (f16)
    fn16<<<grid, nthr, lds, stream>>>(X, p.N, p.d, p.K, p.Kp, p.waves, p.kslabs, rpc,
                                      reinterpret_cast<const float4*>(w.W32p), w.c32, w.mup, w.ivp, w.c64d, w.errc,
                                      w.rowref, w.partials, w.llpart, ll_point, R, p1, p.drop_rho,
                                      lists ? w.slist : nullptr, lists ? w.slen : nullptr, xf, vec);
  fn<<<grid, nthr, lds, stream>>>(X, p.N, p.d, p.K, p.Kp, p.waves, p.kslabs, rpc,
                                  reinterpret_cast<const float4*>(w.W32p), w.c32, w.mup, w.ivp, w.c64d, w.errc,
                                  w.rowref, w.partials, w.llpart, ll_point, R, p1, p.drop_rho,
                                  lists ? w.slist : nullptr, lists ? w.slen : nullptr, xf, vec);
  return hipGetLastError();
}

// The fp64 score pass: top-2 (TOP2) over all rows, or the normaliser
// fallback over the rows the first pass's merge listed.
template <int DT, bool TOP2, typename XT>
static hipError_t run_lse(const Plan& p, const XT* X, int32_t* idx, float* resp, hipStream_t stream) {
  const Workspace& w = p.ws;
  const int Kt = p.Kp16 / 16;
  const int32_t* rows = TOP2 ? nullptr : w.fblist;
  const int32_t* nrows = TOP2 ? nullptr : w.fbcount;
  float4* rowref = TOP2 ? nullptr : w.rowref;
  // Top-2 takes two point groups per wave even with many component tiles:
  // its extra state would otherwise keep the kernel from four waves per SIMD.
  if (Kt >= kLseWaves && !TOP2)
    estep_lse_kernel<DT, TOP2, XT, 4><<<(unsigned)p.tiles, 256, 0, stream>>>(
        X, p.N, p.d, p.K, p.Kp16, w.W64p, w.c64e, rows, nrows, w.rowE, rowref, w.lrow, idx, resp);
  else if (Kt >= 2)
    estep_lse_kernel<DT, TOP2, XT, 2><<<(unsigned)p.tiles, 256, 0, stream>>>(
        X, p.N, p.d, p.K, p.Kp16, w.W64p, w.c64e, rows, nrows, w.rowE, rowref, w.lrow, idx, resp);
  else
    estep_lse_kernel<DT, TOP2, XT, 1><<<(unsigned)p.tiles, 256, 0, stream>>>(
        X, p.N, p.d, p.K, p.Kp16, w.W64p, w.c64e, rows, nrows, w.rowE, rowref, w.lrow, idx, resp);
  return hipGetLastError();
}

// Sets *flag when some row's |x|^2, as the fp32 first pass recorded it, is at
// least 225 (or not a number): then some |x_j| may reach 15, where the fp16
// split of (16 x)^2 would leave the fp16 range. (Each record is a sum of
// nonnegative rounded squares, so it is at least every x_j^2 of its row.)
__global__ void __launch_bounds__(256) xrange_kernel(const float* __restrict__ rowSq, int64_t N,
                                                     int32_t* __restrict__ flag) {
  int out = 0;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < N; i += (int64_t)gridDim.x * blockDim.x)
    out |= !(rowSq[i] < 225.f);
  if (__syncthreads_or(out) && threadIdx.x == 0) atomicOr(flag, 1);
}

// Normalisers of the two-pass regime: the fp32 first pass, the merge of its
// records per row, the fp64 fallback for the rows the merge lists, and the
// per-tile log-likelihood sums.
template <int DT, typename XT>
static hipError_t run_normalisers(const Plan& p, const XT* X, const float* mu, float* ll_point,
                                  hipStream_t stream) {
  const Workspace& w = p.ws;
  fill_int_kernel<<<1, 64, 0, stream>>>(w.fbcount, 2, 0);  // fbcount and xflag
  hipError_t e = run_stats<DT, 2>(p, X, mu, nullptr, nullptr, stream);
  if (e != hipSuccess) return e;
  // the merge reads X rows four values at a time when d % 4 == 0 and the
  // base is aligned for it (16 bytes for fp32, 8 for half precision)
  const int mvec = p.d % 4 == 0 && reinterpret_cast<uintptr_t>(X) % (4 * sizeof(XT)) == 0 ? 1 : 0;
  lse_merge_kernel<DT, XT><<<(unsigned)p.tiles, 64, 0, stream>>>(
      X, p.N, p.d, p.kslabs, 32 * p.waves, w.p1h, w.p1v, w.p1k, w.rowE, w.mup, w.ivp, w.c64d, w.rowref, w.lrow,
      w.fblist, w.fbcount, mvec);
  e = run_lse<DT, false>(p, X, nullptr, nullptr, stream);
  if (e != hipSuccess) return e;
  row_ll_sum_kernel<<<(unsigned)ll_parts(p), 256, 0, stream>>>(w.lrow, p.N, ll_point, w.llpart);
  // whether IEEE-half X stays in the fp16 split's range (every |x| < 15);
  // bfloat16 X never takes the fp16 split
  if (std::is_same<XT, _Float16>::value && p.stats_f16 && !p.stats_split)
    xrange_kernel<<<256, 256, 0, stream>>>(w.rowSq, p.N, w.xflag);
  // the second pass's row lists
  const dim3 tg((unsigned)p.tiles, (unsigned)p.kslabs), sg((unsigned)kSlabSegs, (unsigned)p.kslabs);
  slab_keep_kernel<<<tg, 64, 0, stream>>>(w.p1h, w.rowref, w.rowSq, p.N, p.tiles, p.drop_rho, w.smask, w.soff);
  slab_seg_kernel<<<sg, 256, 0, stream>>>(w.soff, p.tiles, w.sseg);
  slab_scan_kernel<<<(unsigned)p.kslabs, kSlabSegs, 0, stream>>>(w.sseg, w.slen);
  slab_scatter_kernel<<<sg, 64, 0, stream>>>(w.smask, w.sseg, p.N, p.tiles, w.slist);
  return hipGetLastError();
}

template <int DS, typename XT>
static hipError_t run_small(const Plan& p, const XT* X, const float* mu, float* ll_point, float* R,
                            hipStream_t stream) {
  const Workspace& w = p.ws;
  const int vec = (sizeof(XT) == 4 && p.d % 4 == 0 && reinterpret_cast<uintptr_t>(X) % 16 == 0) ? 1 : 0;
  auto fn = p.stats_split ? estep_small_kernel<DS, XT, true> : estep_small_kernel<DS, XT, false>;
  fn<<<(unsigned)p.P, 64 * kSmallWaves, 0, stream>>>(X, p.N, p.d, p.K, p.rows_per_chunk / kSmallWaves, w.W64p,
                                                      w.c64e, mu, w.iv64, w.c64d, w.errc, w.partials, w.llpart,
                                                      ll_point, R, vec);
  return hipGetLastError();
}

template <typename XT>
static hipError_t estep_typed(const Plan& p, const XT* X, const float* mu, float* ll_point, float* R,
                              hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (p.regime == 3) {
    switch (p.DP / 16) {
      case 1: e = run_small<1>(p, X, mu, ll_point, R, stream); break;
      case 2: e = run_small<2>(p, X, mu, ll_point, R, stream); break;
      case 3: e = run_small<3>(p, X, mu, ll_point, R, stream); break;
      default: e = run_small<4>(p, X, mu, ll_point, R, stream); break;
    }
    return e;
  }
  if (p.regime == 1) {
    switch (p.DT) {
      case 1: e = run_stats<1, 0>(p, X, mu, ll_point, R, stream); break;
      case 2: e = run_stats<2, 0>(p, X, mu, ll_point, R, stream); break;
      case 3: e = run_stats<3, 0>(p, X, mu, ll_point, R, stream); break;
      default: e = run_stats<4, 0>(p, X, mu, ll_point, R, stream); break;
    }
    return e;
  }
  switch (p.DT) {
    case 1: e = run_normalisers<1>(p, X, mu, ll_point, stream); break;
    case 2: e = run_normalisers<2>(p, X, mu, ll_point, stream); break;
    case 3: e = run_normalisers<3>(p, X, mu, ll_point, stream); break;
    default: e = run_normalisers<4>(p, X, mu, ll_point, stream); break;
  }
  if (e != hipSuccess) return e;
  switch (p.DT) {
    case 1: e = run_stats<1, 1>(p, X, mu, nullptr, R, stream); break;
    case 2: e = run_stats<2, 1>(p, X, mu, nullptr, R, stream); break;
    case 3: e = run_stats<3, 1>(p, X, mu, nullptr, R, stream); break;
    default: e = run_stats<4, 1>(p, X, mu, nullptr, R, stream); break;
  }
  return e;
}

static thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

void set_timing_events(hipEvent_t start, hipEvent_t stop) {
  t_ev_start = start;
  t_ev_stop = stop;
}

hipError_t launch_estep(const Plan& p, const void* X, int x_dtype, const float* mu, float* Nk, float* Sx,
                        float* Sxx, double* loglik_total, float* loglik_point, float* R, hipStream_t stream) {
  if (p.N == 0) return launch_zero_outputs(Nk, Sx, Sxx, p.d, p.K, loglik_total, stream);
  hipEvent_t ev0 = t_ev_start, ev1 = t_ev_stop;
  t_ev_start = t_ev_stop = nullptr;
  hipError_t e = hipSuccess;
  if (ev0) e = hipEventRecord(ev0, stream);
  if (e != hipSuccess) return e;
  e = with_x_type(x_dtype, X, [&](auto x) { return estep_typed(p, x, mu, loglik_point, R, stream); });
  if (e != hipSuccess) return e;
  if (ev1) e = hipEventRecord(ev1, stream);
  if (e != hipSuccess) return e;
  const Workspace& w = p.ws;
  if (Nk && Sx && Sxx) {
    const int64_t n = (int64_t)p.K * (1 + 2 * p.d);
    if (p.G > 1) {
      reduce_stats_seg_kernel<<<dim3(nblocks(n, 256), p.G), 256, 0, stream>>>(w.partials, p.P, p.G, p.Kp, p.E,
                                                                              p.DP, p.K, p.d, w.redtmp);
      reduce_stats_final_kernel<<<nblocks(n, 256), 256, 0, stream>>>(w.redtmp, p.G, p.K, p.d, Nk, Sx, Sxx);
    } else {
      reduce_stats_kernel<<<nblocks(n, 256), 256, 0, stream>>>(w.partials, p.P, p.Kp, p.E, p.DP, p.K, p.d, Nk,
                                                                 Sx, Sxx);
    }
  }
  if (loglik_total) {
    const int64_t nll = ll_parts(p);
    reduce_ll_kernel<false><<<1, 256, 0, stream>>>(w.llpart, nll, loglik_total, 0);
  }
  return hipGetLastError();
}

hipError_t launch_estep_accum(const Plan& p, const void* X, int x_dtype, const float* mu, double* acc, int first,
                              float* loglik_point, hipStream_t stream) {
  hipError_t e =
      with_x_type(x_dtype, X, [&](auto x) { return estep_typed(p, x, mu, loglik_point, nullptr, stream); });
  if (e != hipSuccess) return e;
  const Workspace& w = p.ws;
  const int64_t n = (int64_t)p.K * (1 + 2 * p.d);
  accum_stats_kernel<<<nblocks(n, 256), 256, 0, stream>>>(w.partials, p.P, p.Kp, p.E, p.DP, p.K, p.d, acc, first);
  const int64_t nll = ll_parts(p);
  reduce_ll_kernel<true><<<1, 256, 0, stream>>>(w.llpart, nll, acc + n, first);
  return hipGetLastError();
}

hipError_t launch_finalize_stats(const double* acc, int K, int d, float* Nk, float* Sx, float* Sxx,
                                 double* loglik_total, hipStream_t stream) {
  const int64_t n = (int64_t)K * (1 + 2 * d);
  finalize_stats_kernel<<<nblocks(n, 256), 256, 0, stream>>>(acc, K, d, Nk, Sx, Sxx, loglik_total);
  return hipGetLastError();
}

hipError_t launch_top2(const Plan& p, const void* X, int x_dtype, int32_t* idx, float* resp,
                       hipStream_t stream) {
  if (p.N == 0) return hipSuccess;
  return with_x_type(x_dtype, X, [&](auto x) {
    switch (p.DT) {
      case 1: return run_lse<1, true>(p, x, idx, resp, stream);
      case 2: return run_lse<2, true>(p, x, idx, resp, stream);
      case 3: return run_lse<3, true>(p, x, idx, resp, stream);
      default: return run_lse<4, true>(p, x, idx, resp, stream);
    }
  });
}

template <int DT, typename XT>
static hipError_t run_kmeans_assign(const Plan& p, const XT* X, int32_t* assign, float* dist2, double* inertia,
                                    hipStream_t stream) {
  const Workspace& w = p.ws;
  const int nthr = p.waves * 64;
  const int KS = p.waves * 32;
  const size_t lds = (size_t)(64 * (32 * DT + 4) + 64 * (KS + 8) + 128) * sizeof(float) +
                     (size_t)(64 + nthr + p.waves * kRefCap) * sizeof(double) + 64 * sizeof(int) +
                     (size_t)p.waves * kRefCap * sizeof(uint32_t);
  auto fn = kmeans_assign_kernel<DT, XT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  // One block walks every slab of its rows, so the row chunks are cut for
  // exactly the blocks that can be resident at once (by LDS, registers and
  // waves) over 256 CUs: one more chunk than fits would run as a second
  // round on a nearly idle chip. There are at most `tiles` chunks, which the
  // workspace's per-chunk sums hold.
  static std::atomic<int> resident[kSlabWaves + 1];
  int per_cu = resident[p.waves].load(std::memory_order_relaxed);
  if (per_cu == 0) {
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, nthr, lds);
    if (e != hipSuccess) return e;
    per_cu = std::max(per_cu, 1);
    resident[p.waves].store(per_cu, std::memory_order_relaxed);
  }
  const int64_t target = std::max<int64_t>(1, std::min<int64_t>(256 * (int64_t)per_cu, p.tiles));
  const int64_t rows_per_chunk = (p.tiles + target - 1) / target * 64;
  const int64_t chunks = (p.N + rows_per_chunk - 1) / rows_per_chunk;
  const bool al16 = reinterpret_cast<uintptr_t>(X) % 16 == 0;
  const int vec = sizeof(XT) == 4 ? (p.d % 4 == 0 && al16 ? 1 : 0) : (p.d % 8 == 0 && al16 ? 2 : 0);
  fn<<<(unsigned)chunks, nthr, lds, stream>>>(X, p.N, p.d, p.K, p.waves, p.kslabs, rows_per_chunk,
                                              reinterpret_cast<const float4*>(w.W32p), w.c32, w.mup, w.errc,
                                              assign, dist2, w.llpart, vec);
  e = hipGetLastError();
  if (e == hipSuccess && inertia) {
    reduce_ll_kernel<false><<<1, 256, 0, stream>>>(w.llpart, chunks, inertia, 0);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_kmeans_assign(const Plan& p, const void* X, int x_dtype, int32_t* assign, float* dist2,
                                double* inertia, hipStream_t stream) {
  if (p.N == 0) return hipSuccess;
  return with_x_type(x_dtype, X, [&](auto x) {
    switch (p.DT) {
      case 1: return run_kmeans_assign<1>(p, x, assign, dist2, inertia, stream);
      case 2: return run_kmeans_assign<2>(p, x, assign, dist2, inertia, stream);
      case 3: return run_kmeans_assign<3>(p, x, assign, dist2, inertia, stream);
      default: return run_kmeans_assign<4>(p, x, assign, dist2, inertia, stream);
    }
  });
}

__global__ void fill_kernel(float* __restrict__ a, int64_t n, float v) {
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t < n) a[t] = v;
}

hipError_t launch_fill(float* a, int64_t n, float v, hipStream_t stream) {
  if (n > 0) fill_kernel<<<nblocks(n, 256), 256, 0, stream>>>(a, n, v);
  return hipGetLastError();
}

hipError_t launch_mstep(const float* Nk, const float* Sx, const float* Sxx, int64_t N, int d, int K,
                        float var_floor, float* mu, float* var, float* logw, hipStream_t stream) {
  const int64_t n = (int64_t)K * d;
  mstep_kernel<<<nblocks(n, 256), 256, 0, stream>>>(Nk, Sx, Sxx, (double)N, d, K, var_floor, mu, var, logw);
  return hipGetLastError();
}

hipError_t launch_zero_outputs(float* Nk, float* Sx, float* Sxx, int d, int K, double* loglik_total,
                               hipStream_t stream) {
  const int64_t n = (int64_t)K * d > K ? (int64_t)K * d : K;
  zero_outputs_kernel<<<nblocks(n, 256), 256, 0, stream>>>(Nk, Sx, Sxx, d, K, loglik_total);
  return hipGetLastError();
}

}  // namespace gmm
