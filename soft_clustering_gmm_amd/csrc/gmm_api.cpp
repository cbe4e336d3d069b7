// C-ABI of libgmm_mi355x.so: argument checks, workspace planning and dispatch.
// Every check runs on the host before anything is enqueued; a rejected call
// touches neither the device nor the caller's buffers.
#include "../../include/gmm.h"

#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <map>
#include <mutex>

#include "gmm_internal.hpp"

namespace gmm {

// Statistics contraction of the fused kernels (gmm_set_stats_precision).
static std::atomic<int> g_stats_precision{GMM_STATS_AUTO};

// Scratch of the allocation-free E-step (gmm_estep_stats_static): one array
// per GPU, allocated with the code object and held until the process ends.
// In host code `scratch` names a host-side stand-in, never the device
// memory: kernels and copies get the per-device address that
// hipGetSymbolAddress returns (static_scratch below).
constexpr size_t kStaticScratchBytes = (size_t)GMM_STATIC_SCRATCH_MIB << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
#define GMM_STR2(x) #x
#define GMM_STR(x) GMM_STR2(x)

static std::mutex g_scratch_mutex;
static void* g_scratch_ptr[kMaxDevices];

// Device address of this GPU's scratch array, looked up once per device
// with that device current.
static hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr || reinterpret_cast<uintptr_t>(ptr) % 256 != 0) return hipErrorInvalidValue;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int pow2_waves(int K) {
  int w = 1;
  while (w * 32 < K) w <<= 1;
  return w;
}

static int make_plan_impl(int64_t N, int d, int K, int regime, void* base, Plan* plan, bool records) {
  if (N < 0 || d < 1 || K < 1) return GMM_EINVAL;
  if (d > kMaxD || K > kMaxK || N >= ((int64_t)1 << 40)) return GMM_EUNSUPPORTED;
  if (regime < GMM_REGIME_AUTO || regime > GMM_REGIME_SMALLK) return GMM_EINVAL;
  const bool small_ok = K <= kSmallMaxK && d <= kSmallMaxD;
  if (regime == GMM_REGIME_AUTO)
    regime = small_ok ? GMM_REGIME_SMALLK : K <= kSingleMaxK ? GMM_REGIME_SINGLE : GMM_REGIME_TWOPASS;
  if (regime == GMM_REGIME_SINGLE && K > kSingleMaxK) return GMM_EUNSUPPORTED;
  if (regime == GMM_REGIME_SMALLK && !small_ok) return GMM_EUNSUPPORTED;

  Plan p{};
  p.N = N;
  p.d = d;
  p.K = K;
  p.regime = regime;
  p.tiles = ceil_div(N, kTileN);
  if (regime == GMM_REGIME_SMALLK) {
    // 16-component tiles; each wave streams its own rows in 64-point tiles.
    p.DT = 0;
    p.DP = 16 * (int)ceil_div(d, 16);
    p.waves = kSmallWaves;
    p.kslabs = 1;
    p.Kp = 16;
    const int64_t blocks = 256 * 2;  // two 4-wave blocks per CU (LDS-bound)
    int64_t wave_rows = ceil_div(std::max<int64_t>(ceil_div(N, blocks * kSmallWaves), 1), 64) * 64;
    wave_rows = std::min<int64_t>(wave_rows, kMaxChunkRows / kSmallWaves);
    p.rows_per_chunk = wave_rows * kSmallWaves;
    p.P = N == 0 ? 0 : ceil_div(N, p.rows_per_chunk);
  } else {
    p.DT = (d + 31) / 32;
    p.DP = 32 * p.DT;
    if (K <= kSingleMaxK) {
      p.waves = pow2_waves(K);
      p.kslabs = 1;
    } else {
      p.waves = kSlabWaves;
      p.kslabs = (int)ceil_div(K, 32 * kSlabWaves);
    }
    p.Kp = 32 * p.waves * p.kslabs;
    // Row chunks: one statistics partial per chunk. Aim for one resident block
    // per SIMD-set (8 waves per CU) across 256 CUs.
    int64_t target = p.kslabs > 1 ? std::max<int64_t>(1, 256 / p.kslabs)
                                   : 256 * std::max(1, 8 / p.waves);
    target = std::max<int64_t>(1, std::min<int64_t>(target, p.tiles));
    p.rows_per_chunk = ceil_div(std::max<int64_t>(p.tiles, 1), target) * kTileN;
    // Each chunk accumulates its statistics in fp32 MFMA accumulators; capping
    // its rows keeps that accumulation error near 1e-5 relative.
    p.rows_per_chunk = std::min<int64_t>(p.rows_per_chunk, kMaxChunkRows);
    p.P = N == 0 ? 0 : ceil_div(N, p.rows_per_chunk);
  }
  p.Kp16 = (int)ceil_div(K, 16) * 16;
  p.E = 1 + 2 * p.DP;
  const int sp = g_stats_precision.load(std::memory_order_relaxed);
  p.stats_split = sp == GMM_STATS_SPLIT_BF16;
  p.stats_f16 = sp == GMM_STATS_AUTO;
  p.pass1 = regime == GMM_REGIME_TWOPASS && records;
  p.drop_rho = (float)(std::ldexp(1.0, -20) / (double)std::max<int64_t>(N, 1));

  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  // the fp32 operand layout is built in whole 32-component tiles
  const size_t o_W32p = take((size_t)ceil_div(p.Kp, 32) * 32 * 2 * p.DP * sizeof(float));
  const size_t o_c32 = take((size_t)p.Kp * sizeof(float));
  const size_t o_W64p = take((size_t)p.Kp16 * 2 * p.DP * sizeof(double));
  const size_t o_c64e = take((size_t)p.Kp16 * sizeof(double));
  const size_t o_iv64 = take((size_t)K * d * sizeof(double));
  const size_t o_c64d = take((size_t)K * sizeof(double));
  const size_t o_mup = take((size_t)p.Kp * p.DP * sizeof(float));
  const size_t o_ivp = take((size_t)p.Kp * p.DP * sizeof(double));
  // (the parameter regions above do not depend on N: the row-chunked E-step
  // packs them once for plans of several chunk sizes)
  const size_t o_cmax = take((size_t)K * 4 * sizeof(float));
  const size_t o_errc = take(4 * sizeof(float));
  // per-row normalisers and first-pass records: only the two-pass regime has a first pass
  const size_t n1 = (size_t)std::max<int64_t>(N, 1);
  const size_t o_rowref = take(regime == GMM_REGIME_TWOPASS ? n1 * sizeof(float4) : 0);
  const size_t nrec = p.pass1 ? (size_t)p.kslabs * n1 : 0;
  const size_t o_p1h = take(nrec * sizeof(float4));
  const size_t o_p1v = take(nrec * kCandT * sizeof(float));
  const size_t o_p1k = take(nrec * kCandT);
  const size_t o_rowE = take(p.pass1 ? n1 * sizeof(float) : 0);
  const size_t o_lrow = take(p.pass1 ? n1 * sizeof(double) : 0);
  const size_t o_fbl = take(p.pass1 ? n1 * sizeof(int32_t) : 0);
  const size_t o_fbc = take(p.pass1 ? 2 * sizeof(int32_t) : 0);  // fbcount, xflag
  const size_t o_rsq = take(p.pass1 ? n1 * sizeof(float) : 0);
  const size_t o_slist = take(nrec * sizeof(int32_t));
  const size_t nst = p.pass1 ? (size_t)p.kslabs * std::max<int64_t>(p.tiles, 1) : 0;
  const size_t o_smask = take(nst * sizeof(uint64_t));
  const size_t o_soff = take(nst * sizeof(int32_t));
  const size_t o_sseg = take(p.pass1 ? (size_t)p.kslabs * kSlabSegs * sizeof(int32_t) : 0);
  const size_t o_slen = take(p.pass1 ? (size_t)p.kslabs * sizeof(int32_t) : 0);
  const size_t o_part = take((size_t)std::max<int64_t>(p.P, 1) * p.Kp * p.E * sizeof(float));
  const size_t o_ll = take((size_t)std::max<int64_t>(std::max(p.P, p.tiles), 1) * sizeof(double));
  const size_t o_stats = take((size_t)K * (1 + 2 * d) * sizeof(float));
  // Few outputs (small K x d) give the one-stage reduction too few threads, each
  // summing many partials in sequence: split the partials into G segments.
  {
    const int64_t n = (int64_t)K * (1 + 2 * d);
    p.G = (int)std::max<int64_t>(1, std::min<int64_t>({(int64_t)262144 / n, (int64_t)64, std::max<int64_t>(p.P, 1)}));
  }
  const size_t o_red = take(p.G > 1 ? (size_t)p.G * K * (1 + 2 * d) * sizeof(double) : 0);
  p.bytes = off;
  if (base) {
    char* b = static_cast<char*>(base);
    p.ws.W32p = reinterpret_cast<float*>(b + o_W32p);
    p.ws.c32 = reinterpret_cast<float*>(b + o_c32);
    p.ws.W64p = reinterpret_cast<double*>(b + o_W64p);
    p.ws.c64e = reinterpret_cast<double*>(b + o_c64e);
    p.ws.iv64 = reinterpret_cast<double*>(b + o_iv64);
    p.ws.c64d = reinterpret_cast<double*>(b + o_c64d);
    p.ws.mup = reinterpret_cast<float*>(b + o_mup);
    p.ws.ivp = reinterpret_cast<double*>(b + o_ivp);
    p.ws.compmax = reinterpret_cast<float*>(b + o_cmax);
    p.ws.errc = reinterpret_cast<float*>(b + o_errc);
    p.ws.rowref = regime == GMM_REGIME_TWOPASS ? reinterpret_cast<float4*>(b + o_rowref) : nullptr;
    p.ws.p1h = p.pass1 ? reinterpret_cast<float4*>(b + o_p1h) : nullptr;
    p.ws.p1v = p.pass1 ? reinterpret_cast<float*>(b + o_p1v) : nullptr;
    p.ws.p1k = p.pass1 ? reinterpret_cast<uint8_t*>(b + o_p1k) : nullptr;
    p.ws.rowE = p.pass1 ? reinterpret_cast<float*>(b + o_rowE) : nullptr;
    p.ws.lrow = p.pass1 ? reinterpret_cast<double*>(b + o_lrow) : nullptr;
    p.ws.fblist = p.pass1 ? reinterpret_cast<int32_t*>(b + o_fbl) : nullptr;
    p.ws.fbcount = p.pass1 ? reinterpret_cast<int32_t*>(b + o_fbc) : nullptr;
    p.ws.xflag = p.pass1 ? reinterpret_cast<int32_t*>(b + o_fbc) + 1 : nullptr;
    p.ws.rowSq = p.pass1 ? reinterpret_cast<float*>(b + o_rsq) : nullptr;
    p.ws.slist = p.pass1 ? reinterpret_cast<int32_t*>(b + o_slist) : nullptr;
    p.ws.smask = p.pass1 ? reinterpret_cast<uint64_t*>(b + o_smask) : nullptr;
    p.ws.soff = p.pass1 ? reinterpret_cast<int32_t*>(b + o_soff) : nullptr;
    p.ws.sseg = p.pass1 ? reinterpret_cast<int32_t*>(b + o_sseg) : nullptr;
    p.ws.slen = p.pass1 ? reinterpret_cast<int32_t*>(b + o_slen) : nullptr;
    p.ws.partials = reinterpret_cast<float*>(b + o_part);
    p.ws.llpart = reinterpret_cast<double*>(b + o_ll);
    p.ws.stats = reinterpret_cast<float*>(b + o_stats);
    p.ws.redtmp = reinterpret_cast<double*>(b + o_red);
  }
  *plan = p;
  return GMM_OK;
}

int make_plan(int64_t N, int d, int K, int regime, void* base, Plan* plan) {
  return make_plan_impl(N, d, K, regime, base, plan, true);
}

int make_plan_params(int64_t N, int d, int K, int regime, void* base, Plan* plan) {
  return make_plan_impl(N, d, K, regime, base, plan, false);
}

static size_t workspace_bytes(int64_t N, int d, int K) {
  size_t best = 0;
  for (int r = GMM_REGIME_SINGLE; r <= GMM_REGIME_SMALLK; ++r) {
    Plan p;
    if (make_plan(N, d, K, r, nullptr, &p) == GMM_OK) best = std::max(best, p.bytes);
  }
  return best;
}

static int check_ws(void* ws, size_t ws_bytes, int64_t N, int d, int K) {
  if (!ws) return GMM_EWORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return GMM_EWORKSPACE;
  if (ws_bytes < workspace_bytes(N, d, K)) return GMM_EWORKSPACE;
  return GMM_OK;
}

static int check_common(const void* X, int32_t xt, int64_t N, int32_t d, int32_t K, const float* mu,
                        const float* var, const float* logw) {
  if (xt != GMM_F32 && xt != GMM_F16 && xt != GMM_BF16) return GMM_EINVAL;
  if (N < 0 || d < 1 || K < 1) return GMM_EINVAL;
  if (d > kMaxD || K > kMaxK || N >= ((int64_t)1 << 40)) return GMM_EUNSUPPORTED;
  if ((N > 0 && !X) || !mu || !var || !logw) return GMM_EINVAL;
  return GMM_OK;
}

static int hip_status(hipError_t e) { return e == hipSuccess ? GMM_OK : GMM_EHIP; }

// Row-chunked E-step: workspace = [chunk plan region (the larger of the
// full-chunk and tail-chunk plans; the parameter regions at its start are
// laid out identically for every chunk size)] [staging 0] [staging 1]
// [fp64 accumulators: K * (1 + 2d) statistics + 1 log-likelihood].
struct ChunkLayout {
  int64_t chunk;
  size_t plan_bytes, stage_bytes, stage_off[2], acc_off, total;
};

static int chunk_layout(int64_t N, int d, int K, int64_t chunk_rows, int x_dtype, ChunkLayout* L) {
  if (N < 0 || d < 1 || K < 1 || chunk_rows < 1) return GMM_EINVAL;
  if (x_dtype != GMM_F32 && x_dtype != GMM_F16 && x_dtype != GMM_BF16) return GMM_EINVAL;
  if (d > kMaxD || K > kMaxK || N >= ((int64_t)1 << 40)) return GMM_EUNSUPPORTED;
  const int64_t c = std::max<int64_t>(std::min(chunk_rows, N), 1);
  const int64_t tail = N % c;
  size_t pb = workspace_bytes(c, d, K);
  if (tail) pb = std::max(pb, workspace_bytes(tail, d, K));
  L->chunk = c;
  L->plan_bytes = align_up(pb, 256);
  L->stage_bytes = align_up((size_t)c * d * (x_dtype == GMM_F32 ? 4 : 2), 256);
  L->stage_off[0] = L->plan_bytes;
  L->stage_off[1] = L->plan_bytes + L->stage_bytes;
  L->acc_off = L->plan_bytes + 2 * L->stage_bytes;
  L->total = L->acc_off + align_up(((size_t)K * (1 + 2 * d) + 1) * sizeof(double), 256);
  return GMM_OK;
}

// Per-device copy stream and events of the chunked E-step, created on first
// use and kept for the life of the process. The mutex serialises the
// enqueue sequence of concurrent calls (events are re-recorded per call).
struct ChunkRes {
  hipStream_t copy = nullptr;
  hipEvent_t entry = nullptr, copied[2] = {nullptr, nullptr}, done[2] = {nullptr, nullptr};
};
static std::mutex g_chunk_mutex;
static std::map<int, ChunkRes> g_chunk_res;

static hipError_t chunk_resources(ChunkRes** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  ChunkRes& r = g_chunk_res[dev];
  if (!r.copy) {
    if ((e = hipStreamCreateWithFlags(&r.copy, hipStreamNonBlocking)) != hipSuccess) return e;
    hipEvent_t* evs[5] = {&r.entry, &r.copied[0], &r.copied[1], &r.done[0], &r.done[1]};
    for (hipEvent_t* ev : evs)
      if ((e = hipEventCreateWithFlags(ev, hipEventDisableTiming)) != hipSuccess) return e;
  }
  *out = &r;
  return hipSuccess;
}

}  // namespace gmm

using namespace gmm;

extern "C" {

int gmm_version(void) { return 10000; }

const char* gmm_error_string(int code) {
  switch (code) {
    case GMM_OK: return "ok";
    case GMM_EINVAL: return "invalid argument (null pointer, negative size, bad dtype or regime)";
    case GMM_EUNSUPPORTED:
      return "unsupported shape or regime (1<=d<=128, 1<=K<=65536; single sweep needs K<=256, small-K K<=16 and d<=64)";
    case GMM_EWORKSPACE: return "workspace missing, misaligned (256 B) or smaller than gmm_workspace_bytes()";
    case GMM_EHIP: return "HIP launch failed";
    case GMM_ESCRATCH:
      return "the allocation-free E-step needs more scratch for this shape than its static array holds "
             "(" GMM_STR(GMM_STATIC_SCRATCH_MIB) " MiB per GPU); use gmm_estep_stats with a workspace";
    default: return "unknown status";
  }
}

size_t gmm_workspace_bytes(int64_t N, int32_t d, int32_t K) {
  if (N < 0 || d < 1 || K < 1 || d > kMaxD || K > kMaxK || N >= ((int64_t)1 << 40)) return 0;
  return workspace_bytes(N, d, K);
}

int gmm_estep_stats_regime(const void* X, int32_t x_dtype, int64_t N, int32_t d, const float* mu,
                           const float* var, const float* logw, int32_t K, float* Nk, float* Sx, float* Sxx,
                           double* loglik_total, float* loglik_point, void* workspace, size_t ws_bytes,
                           int32_t regime, void* stream) {
  int st = check_common(X, x_dtype, N, d, K, mu, var, logw);
  if (st) return st;
  if (!Nk || !Sx || !Sxx || !loglik_total) return GMM_EINVAL;
  if ((st = check_ws(workspace, ws_bytes, N, d, K))) return st;
  Plan p;
  if ((st = make_plan(N, d, K, regime, workspace, &p))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N == 0) return hip_status(launch_zero_outputs(Nk, Sx, Sxx, d, K, loglik_total, s));
  hipError_t e = launch_precompute(p, mu, var, logw, s);
  if (e == hipSuccess) e = launch_estep(p, X, x_dtype, mu, Nk, Sx, Sxx, loglik_total, loglik_point, nullptr, s);
  return hip_status(e);
}

int gmm_estep_stats(const void* X, int32_t x_dtype, int64_t N, int32_t d, const float* mu, const float* var,
                    const float* logw, int32_t K, float* Nk, float* Sx, float* Sxx, double* loglik_total,
                    float* loglik_point, void* workspace, size_t ws_bytes, void* stream) {
  return gmm_estep_stats_regime(X, x_dtype, N, d, mu, var, logw, K, Nk, Sx, Sxx, loglik_total, loglik_point,
                                workspace, ws_bytes, GMM_REGIME_AUTO, stream);
}

int gmm_estep_stats_static(const void* X, int32_t x_dtype, int64_t N, int32_t d, const float* mu,
                           const float* var, const float* logw, int32_t K, float* Nk, float* Sx, float* Sxx,
                           double* loglik_total, float* loglik_point, void* stream) {
  int st = check_common(X, x_dtype, N, d, K, mu, var, logw);
  if (st) return st;
  if (!Nk || !Sx || !Sxx || !loglik_total) return GMM_EINVAL;
  Plan p;
  if ((st = make_plan(N, d, K, GMM_REGIME_AUTO, nullptr, &p))) return st;
  if (p.bytes > kStaticScratchBytes) return GMM_ESCRATCH;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N == 0) return hip_status(launch_zero_outputs(Nk, Sx, Sxx, d, K, loglik_total, s));
  void* base = nullptr;
  hipError_t e = static_scratch(&base);
  if (e != hipSuccess) return GMM_EHIP;
  make_plan(N, d, K, GMM_REGIME_AUTO, base, &p);
  // Every kernel of the E-step writes the scratch regions it later reads
  // (packed parameters, per-block partials, block sums), so nothing left by
  // an earlier call is read.
  e = launch_precompute(p, mu, var, logw, s);
  if (e == hipSuccess) e = launch_estep(p, X, x_dtype, mu, Nk, Sx, Sxx, loglik_total, loglik_point, nullptr, s);
  return hip_status(e);
}

int gmm_estep_resp(const void* X, int32_t x_dtype, int64_t N, int32_t d, const float* mu, const float* var,
                   const float* logw, int32_t K, float* R, float* loglik_point, void* workspace, size_t ws_bytes,
                   int32_t regime, void* stream) {
  int st = check_common(X, x_dtype, N, d, K, mu, var, logw);
  if (st) return st;
  if (N > 0 && !R) return GMM_EINVAL;
  if ((st = check_ws(workspace, ws_bytes, N, d, K))) return st;
  Plan p;
  if ((st = make_plan(N, d, K, regime, workspace, &p))) return st;
  if (N == 0) return GMM_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_precompute(p, mu, var, logw, s);
  if (e == hipSuccess) e = launch_estep(p, X, x_dtype, mu, nullptr, nullptr, nullptr, nullptr, loglik_point, R, s);
  return hip_status(e);
}

int gmm_mstep(const float* Nk, const float* Sx, const float* Sxx, int64_t N, int32_t d, int32_t K,
              float var_floor, float* mu, float* var, float* logw, void* stream) {
  if (!Nk || !Sx || !Sxx || !mu || !var || !logw) return GMM_EINVAL;
  if (N < 1 || d < 1 || K < 1 || !(var_floor >= 0.f)) return GMM_EINVAL;
  if (d > kMaxD || K > kMaxK) return GMM_EUNSUPPORTED;
  return hip_status(launch_mstep(Nk, Sx, Sxx, N, d, K, var_floor, mu, var, logw, static_cast<hipStream_t>(stream)));
}

int gmm_em_iterate(const void* X, int32_t x_dtype, int64_t N, int32_t d, int32_t K, int32_t iters,
                   float var_floor, float* mu, float* var, float* logw, double* loglik_hist, void* workspace,
                   size_t ws_bytes, void* stream) {
  int st = check_common(X, x_dtype, N, d, K, mu, var, logw);
  if (st) return st;
  if (N < 1 || iters < 0 || !(var_floor >= 0.f)) return GMM_EINVAL;
  if (iters > 0 && !loglik_hist) return GMM_EINVAL;
  if ((st = check_ws(workspace, ws_bytes, N, d, K))) return st;
  Plan p;
  if ((st = make_plan(N, d, K, GMM_REGIME_AUTO, workspace, &p))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* Nk = p.ws.stats;
  float* Sx = Nk + K;
  float* Sxx = Sx + (size_t)K * d;
  for (int it = 0; it < iters; ++it) {
    hipError_t e = launch_precompute(p, mu, var, logw, s);
    if (e == hipSuccess) e = launch_estep(p, X, x_dtype, mu, Nk, Sx, Sxx, loglik_hist + it, nullptr, nullptr, s);
    if (e == hipSuccess) e = launch_mstep(Nk, Sx, Sxx, N, d, K, var_floor, mu, var, logw, s);
    if (e != hipSuccess) return GMM_EHIP;
  }
  return GMM_OK;
}

size_t gmm_workspace_bytes_chunked(int64_t N, int32_t d, int32_t K, int64_t chunk_rows, int32_t x_dtype) {
  ChunkLayout L;
  return chunk_layout(N, d, K, chunk_rows, x_dtype, &L) == GMM_OK ? L.total : 0;
}

int gmm_estep_stats_chunked(const void* X_host, int32_t x_dtype, int64_t N, int32_t d, const float* mu,
                            const float* var, const float* logw, int32_t K, float* Nk, float* Sx, float* Sxx,
                            double* loglik_total, float* loglik_point, int64_t chunk_rows, void* workspace,
                            size_t ws_bytes, void* stream) {
  int st = check_common(X_host, x_dtype, N, d, K, mu, var, logw);
  if (st) return st;
  if (!Nk || !Sx || !Sxx || !loglik_total) return GMM_EINVAL;
  ChunkLayout L;
  if ((st = chunk_layout(N, d, K, chunk_rows, x_dtype, &L))) return st;
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % 256 != 0 || ws_bytes < L.total) return GMM_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N == 0) return hip_status(launch_zero_outputs(Nk, Sx, Sxx, d, K, loglik_total, s));
  char* base = static_cast<char*>(workspace);
  void* stage[2] = {base + L.stage_off[0], base + L.stage_off[1]};
  double* acc = reinterpret_cast<double*>(base + L.acc_off);
  const size_t row_bytes = (size_t)d * (x_dtype == GMM_F32 ? 4 : 2);
  const char* xh = static_cast<const char*>(X_host);

  // Both chunk plans (full chunks and the ragged tail) are built before
  // anything is enqueued, so a rejected plan leaves the stream untouched.
  Plan p, ptail;
  const int64_t tail = N % L.chunk;
  if (make_plan(L.chunk, d, K, GMM_REGIME_AUTO, workspace, &p) != GMM_OK) return GMM_EINVAL;
  if (make_plan(tail ? tail : L.chunk, d, K, GMM_REGIME_AUTO, workspace, &ptail) != GMM_OK) return GMM_EINVAL;
  if (p.bytes > L.plan_bytes || ptail.bytes > L.plan_bytes) return GMM_EWORKSPACE;
  // the statistics skip threshold is set by the rows of the whole call
  p.drop_rho = ptail.drop_rho = (float)(std::ldexp(1.0, -20) / (double)N);

  std::lock_guard<std::mutex> lock(g_chunk_mutex);
  ChunkRes* r = nullptr;
  hipError_t e = chunk_resources(&r);
  if (e == hipSuccess) e = launch_precompute(p, mu, var, logw, s);
  // the staging buffers may still be read by earlier work on `stream`
  if (e == hipSuccess) e = hipEventRecord(r->entry, s);
  if (e == hipSuccess) e = hipStreamWaitEvent(r->copy, r->entry, 0);
  const int64_t nchunks = (N + L.chunk - 1) / L.chunk;
  for (int64_t i = 0; i < nchunks && e == hipSuccess; ++i) {
    const int b = (int)(i & 1);
    const int64_t off = i * L.chunk, n = std::min(L.chunk, N - off);
    if (i >= 2) e = hipStreamWaitEvent(r->copy, r->done[b], 0);  // chunk i-2 is done with buffer b
    if (e == hipSuccess)
      e = hipMemcpyAsync(stage[b], xh + (size_t)off * row_bytes, (size_t)n * row_bytes, hipMemcpyHostToDevice,
                         r->copy);
    if (e == hipSuccess) e = hipEventRecord(r->copied[b], r->copy);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, r->copied[b], 0);
    const Plan& pc = n == L.chunk ? p : ptail;
    if (e == hipSuccess)
      e = launch_estep_accum(pc, stage[b], x_dtype, mu, acc, i == 0 ? 1 : 0,
                             loglik_point ? loglik_point + off : nullptr, s);
    if (e == hipSuccess) e = hipEventRecord(r->done[b], s);
  }
  if (e == hipSuccess) e = launch_finalize_stats(acc, K, d, Nk, Sx, Sxx, loglik_total, s);
  return hip_status(e);
}

static bool lists_args_ok(int64_t N, int32_t K) {
  return N >= 0 && N <= INT32_MAX && K >= 1 && K <= kMaxK;
}

size_t gmm_border_lists_workspace_bytes(int64_t N, int32_t K) {
  return lists_args_ok(N, K) ? lists_layout(N, K).bytes : 0;
}

int gmm_border_lists(const int32_t* idx, const float* resp, int64_t N, int32_t K, float border_threshold,
                     int64_t* offsets, int32_t* members, int64_t members_capacity, void* workspace,
                     size_t ws_bytes, void* stream) {
  if (N < 0 || K < 1) return GMM_EINVAL;
  if (!lists_args_ok(N, K)) return GMM_EUNSUPPORTED;
  if (!offsets || (N > 0 && (!idx || !resp || !members))) return GMM_EINVAL;
  if (reinterpret_cast<uintptr_t>(idx) % 8 != 0) return GMM_EINVAL;  // read as (first, second) pairs
  if (members_capacity < 2 * N) return GMM_EINVAL;
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % 256 != 0 || ws_bytes < lists_layout(N, K).bytes)
    return GMM_EWORKSPACE;
  return hip_status(launch_border_lists(idx, resp, N, K, border_threshold, offsets, members, workspace,
                                        static_cast<hipStream_t>(stream)));
}

// k-means workspace: [two-pass plan region] [unit variances K x d] [zero
// log-weights K] [list-build region] [offsets K+1] [members N] [segment
// counts K] [segment offsets K+1] [scan scratch] [segment sums] [assign N].
struct KmLayout {
  size_t plan, ones, zeros, lists, offsets, members, seg, segoff, scan, part, assign, total;
  int64_t max_segments;
};

static bool kmeans_args_ok(int64_t N, int d, int K) {
  return N >= 0 && N <= INT32_MAX && d >= 1 && d <= kMaxD && K >= 1 && K <= kMaxK;
}

static KmLayout kmeans_layout(int64_t N, int d, int K) {
  KmLayout L{};
  Plan p;
  make_plan_params(N, d, K, GMM_REGIME_TWOPASS, nullptr, &p);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + std::max<size_t>(bytes, 1), 256);
    return o;
  };
  L.plan = take(p.bytes);
  L.ones = take((size_t)K * d * sizeof(float));
  L.zeros = take((size_t)K * sizeof(float));
  L.lists = take(lists_layout(N, K).bytes);
  L.offsets = take((size_t)(K + 1) * sizeof(int64_t));
  L.members = take((size_t)N * sizeof(int32_t));
  L.seg = take((size_t)K * sizeof(int32_t));
  L.segoff = take((size_t)(K + 1) * sizeof(int64_t));
  L.scan = take((size_t)((K + 1023) / 1024 + 1) * sizeof(int64_t));
  L.max_segments = kmeans_max_segments(N, K);
  L.part = take((size_t)L.max_segments * d * sizeof(double));
  L.assign = take((size_t)N * sizeof(int32_t));
  L.total = off;
  return L;
}

size_t gmm_kmeans_workspace_bytes(int64_t N, int32_t d, int32_t K) {
  return kmeans_args_ok(N, d, K) ? kmeans_layout(N, d, K).total : 0;
}

static int kmeans_check(const void* X, int32_t xt, int64_t N, int32_t d, int32_t K, const float* C, void* ws,
                        size_t ws_bytes) {
  if (xt != GMM_F32 && xt != GMM_F16 && xt != GMM_BF16) return GMM_EINVAL;
  if (N < 0 || d < 1 || K < 1) return GMM_EINVAL;
  if (!kmeans_args_ok(N, d, K)) return GMM_EUNSUPPORTED;
  if ((N > 0 && !X) || !C) return GMM_EINVAL;
  if (!ws || reinterpret_cast<uintptr_t>(ws) % 256 != 0 || ws_bytes < kmeans_layout(N, d, K).total)
    return GMM_EWORKSPACE;
  return GMM_OK;
}

static hipError_t kmeans_assign_impl(const void* X, int32_t xt, int64_t N, int32_t d, const float* C, int32_t K,
                                     int32_t* assign, float* dist2, double* inertia, char* w, const KmLayout& L,
                                     hipStream_t s) {
  float* ones = reinterpret_cast<float*>(w + L.ones);
  float* zeros = reinterpret_cast<float*>(w + L.zeros);
  Plan p;
  make_plan_params(N, d, K, GMM_REGIME_TWOPASS, w + L.plan, &p);
  hipError_t e = launch_fill(ones, (int64_t)K * d, 1.f, s);
  if (e == hipSuccess) e = launch_fill(zeros, K, 0.f, s);
  if (e == hipSuccess) e = launch_precompute(p, C, ones, zeros, s);
  if (e == hipSuccess) e = launch_kmeans_assign(p, X, xt, assign, dist2, inertia, s);
  return e;
}

static hipError_t kmeans_update_impl(const void* X, int32_t xt, int64_t N, int32_t d, const int32_t* assign,
                                     int32_t K, float* C, int64_t* counts, char* w, const KmLayout& L,
                                     hipStream_t s) {
  int64_t* offsets = reinterpret_cast<int64_t*>(w + L.offsets);
  int32_t* members = reinterpret_cast<int32_t*>(w + L.members);
  hipError_t e = launch_border_lists(assign, nullptr, N, K, 0.f, offsets, members, w + L.lists, s);
  if (e == hipSuccess)
    e = launch_kmeans_update(X, xt, N, d, K, offsets, members, reinterpret_cast<int32_t*>(w + L.seg),
                             reinterpret_cast<int64_t*>(w + L.segoff), reinterpret_cast<int64_t*>(w + L.scan),
                             reinterpret_cast<double*>(w + L.part), L.max_segments, C, counts, s);
  return e;
}

int gmm_kmeans_assign(const void* X, int32_t x_dtype, int64_t N, int32_t d, const float* C, int32_t K,
                      int32_t* assign, float* dist2, double* inertia, void* workspace, size_t ws_bytes,
                      void* stream) {
  int st = kmeans_check(X, x_dtype, N, d, K, C, workspace, ws_bytes);
  if (st) return st;
  if (N > 0 && !assign) return GMM_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N == 0) return inertia ? hip_status(launch_zero_outputs(nullptr, nullptr, nullptr, d, K, inertia, s)) : GMM_OK;
  const KmLayout L = kmeans_layout(N, d, K);
  return hip_status(kmeans_assign_impl(X, x_dtype, N, d, C, K, assign, dist2, inertia,
                                       static_cast<char*>(workspace), L, s));
}

int gmm_kmeans_update(const void* X, int32_t x_dtype, int64_t N, int32_t d, const int32_t* assign, int32_t K,
                      float* C, int64_t* counts, void* workspace, size_t ws_bytes, void* stream) {
  int st = kmeans_check(X, x_dtype, N, d, K, C, workspace, ws_bytes);
  if (st) return st;
  if (N > 0 && !assign) return GMM_EINVAL;
  const KmLayout L = kmeans_layout(N, d, K);
  return hip_status(kmeans_update_impl(X, x_dtype, N, d, assign, K, C, counts, static_cast<char*>(workspace), L,
                                       static_cast<hipStream_t>(stream)));
}

int gmm_kmeans_iterate(const void* X, int32_t x_dtype, int64_t N, int32_t d, int32_t K, int32_t iters, float* C,
                       double* inertia_hist, void* workspace, size_t ws_bytes, void* stream) {
  int st = kmeans_check(X, x_dtype, N, d, K, C, workspace, ws_bytes);
  if (st) return st;
  if (N < 1 || iters < 0 || (iters > 0 && !inertia_hist)) return GMM_EINVAL;
  const KmLayout L = kmeans_layout(N, d, K);
  char* w = static_cast<char*>(workspace);
  int32_t* assign = reinterpret_cast<int32_t*>(w + L.assign);
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int it = 0; it < iters; ++it) {
    hipError_t e = kmeans_assign_impl(X, x_dtype, N, d, C, K, assign, nullptr, inertia_hist + it, w, L, s);
    if (e == hipSuccess) e = kmeans_update_impl(X, x_dtype, N, d, assign, K, C, nullptr, w, L, s);
    if (e != hipSuccess) return GMM_EHIP;
  }
  return GMM_OK;
}

int gmm_plan_info(int64_t N, int32_t d, int32_t K, int32_t regime, int64_t* info) {
  if (!info) return GMM_EINVAL;
  Plan p;
  const int st = make_plan(N, d, K, regime, nullptr, &p);
  if (st) return st;
  const int64_t v[7] = {p.regime, p.waves, p.kslabs, p.rows_per_chunk, p.P, p.tiles, (int64_t)p.bytes};
  for (int i = 0; i < 7; ++i) info[i] = v[i];
  return GMM_OK;
}

int gmm_set_stats_precision(int32_t mode) {
  if (mode != GMM_STATS_FP32 && mode != GMM_STATS_SPLIT_BF16 && mode != GMM_STATS_AUTO) return GMM_EINVAL;
  g_stats_precision.store(mode, std::memory_order_relaxed);
  return GMM_OK;
}

int gmm_set_timing_events(void* start, void* stop) {
  set_timing_events(static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop));
  return GMM_OK;
}

int gmm_assign_top2(const void* X, int32_t x_dtype, int64_t N, int32_t d, const float* mu, const float* var,
                    const float* logw, int32_t K, int32_t* idx, float* resp, void* workspace, size_t ws_bytes,
                    void* stream) {
  int st = check_common(X, x_dtype, N, d, K, mu, var, logw);
  if (st) return st;
  if (N > 0 && (!idx || !resp)) return GMM_EINVAL;
  if ((st = check_ws(workspace, ws_bytes, N, d, K))) return st;
  Plan p;
  if ((st = make_plan_params(N, d, K, GMM_REGIME_TWOPASS, workspace, &p))) return st;
  if (N == 0) return GMM_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_precompute(p, mu, var, logw, s);
  if (e == hipSuccess) e = launch_top2(p, X, x_dtype, idx, resp, s);
  return hip_status(e);
}

}  // extern "C"
