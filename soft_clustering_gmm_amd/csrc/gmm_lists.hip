// Inverted lists with border vectors, built from the top-2 assignment.
//
// "Flash-GMM: a memory-efficient kernel for scalable soft clustering",
// abstract: the responsibilities of a soft coarse quantizer let vectors near
// cluster borders be assigned to several clusters. Point n is listed under
// its first pick idx[n][0] and, when resp[n][1] >= threshold, also under its
// second pick idx[n][1]; every list holds point indices in increasing order.
//
// The lists are a stable sort of (list, point) items by list id, done as an
// LSD counting sort with 8-bit digits (one pass for K <= 256, two for
// K <= 65536), in the spirit of the sort-inverse update of the Flash-KMeans
// articles (sorting by cluster id instead of scattering with atomics). Per
// pass: per-block digit histograms, one exclusive scan over them (digit
// major), then a scatter in which each one-wave block ranks its items
// stably with ballots into an LDS stage ordered by digit, and writes each
// digit's run out contiguously. Everything is integer work and deterministic.
#include <atomic>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gmm_device.hpp"
#include "gmm_internal.hpp"

namespace gmm {

constexpr int kListPoints = 1024;  // points per block in the pass over (idx, resp)
constexpr int kListItems = 2048;   // items per block in the second pass (= the LDS stage)

// Orders this wave's LDS accesses (all lanes) before its later ones.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Lanes of the wave whose digit equals x, from the 8 bit-plane ballots of
// the wave's digits and the ballot of valid lanes.
__device__ __forceinline__ uint64_t digit_match(int x, const uint64_t* b, uint64_t valid) {
  uint64_t m = valid;
#pragma unroll
  for (int i = 0; i < 8; ++i) m &= ((x >> i) & 1) ? b[i] : ~b[i];
  return m;
}

__device__ __forceinline__ void digit_ballots(bool v, int dg, uint64_t* b, uint64_t* valid) {
  *valid = __ballot(v);
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = __ballot(v && ((dg >> i) & 1));
}

// Items of point n: (idx[n][0], n) always, and (idx[n][1], n) when
// idx[n][1] >= 0 and resp[n][1] >= thr (a border vector). Items of a block
// are ordered by point, first pick before second pick. With resp == nullptr
// idx is one list id per point (hard assignments) and there are no second
// picks.

// Histogram of the block's item digits -> H[digit * B + block].
template <bool FROM_POINTS>
__global__ void __launch_bounds__(64)
lists_hist_kernel(const int32_t* __restrict__ idx, const float* __restrict__ resp, int64_t N, float thr,
                  const int32_t* __restrict__ keys, const int64_t* __restrict__ total, int shift,
                  int32_t* __restrict__ H, int64_t B) {
  __shared__ int32_t h[256];
  const int lane = threadIdx.x;
  for (int i = lane; i < 256; i += 64) h[i] = 0;
  __syncthreads();
  if (FROM_POINTS) {
    constexpr int R = kListPoints / 64;
    const int64_t lo = blockIdx.x * (int64_t)kListPoints, hi = min(N, lo + kListPoints);
    int2 pk[R];
    float r1[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {  // all loads in flight at once
      const int64_t n = lo + 64 * r + lane;
      if (resp) {  // top-2 pairs
        pk[r] = n < hi ? reinterpret_cast<const int2*>(idx)[n] : make_int2(0, -1);
        r1[r] = n < hi ? resp[2 * n + 1] : 0.f;
      } else {  // one assignment per point
        pk[r] = make_int2(n < hi ? idx[n] : 0, -1);
        r1[r] = 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (lo + 64 * r + lane < hi) {
        atomicAdd(&h[(pk[r].x >> shift) & 255], 1);
        if (pk[r].y >= 0 && r1[r] >= thr) atomicAdd(&h[(pk[r].y >> shift) & 255], 1);
      }
    }
  } else {
    constexpr int R = kListItems / 64;
    const int64_t M = *total;
    const int64_t lo = blockIdx.x * (int64_t)kListItems, hi = min(M, lo + kListItems);
    int ki[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t i = lo + 64 * r + lane;
      ki[r] = i < hi ? keys[i] : 0;
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (lo + 64 * r + lane < hi) atomicAdd(&h[(ki[r] >> shift) & 255], 1);
  }
  __syncthreads();
  for (int i = lane; i < 256; i += 64) H[(int64_t)i * B + blockIdx.x] = h[i];
}

// Exclusive scan of H (n = 256 * B entries, in index order) -> O, with the
// grand total in *total: per-1024-entry segment sums, a scan of those sums
// in one block, then each segment scanned locally on top of its offset.
constexpr int kScanSeg = 1024;  // entries per segment (256 threads x 4)

__device__ __forceinline__ int64_t block_excl_scan256(int64_t v, int64_t* s, int64_t* block_total) {
  const int t = threadIdx.x;
  s[t] = v;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {  // inclusive Hillis-Steele scan
    const int64_t a = t >= o ? s[t - o] : 0;
    __syncthreads();
    s[t] += a;
    __syncthreads();
  }
  const int64_t incl = s[t];
  *block_total = s[255];
  __syncthreads();
  return incl - v;
}

__global__ void __launch_bounds__(256)
lists_seg_sums_kernel(const int32_t* __restrict__ H, int64_t n, int64_t* __restrict__ S) {
  __shared__ int64_t s[256];
  const int64_t base = blockIdx.x * (int64_t)kScanSeg + 4 * threadIdx.x;
  int64_t a = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) a += base + j < n ? H[base + j] : 0;
  int64_t tot;
  block_excl_scan256(a, s, &tot);
  if (threadIdx.x == 0) S[blockIdx.x] = tot;
}

// In place: S[i] <- sum of S[0..i), for nseg segment sums; *total <- sum of all.
__global__ void __launch_bounds__(256)
lists_seg_scan_kernel(int64_t* __restrict__ S, int64_t nseg, int64_t* __restrict__ total) {
  __shared__ int64_t s[256];
  const int64_t per = (nseg + 255) / 256;
  const int64_t lo = min(nseg, threadIdx.x * per), hi = min(nseg, lo + per);
  int64_t a = 0;
  for (int64_t i = lo; i < hi; ++i) a += S[i];
  int64_t tot;
  int64_t run = block_excl_scan256(a, s, &tot);
  for (int64_t i = lo; i < hi; ++i) {
    const int64_t v = S[i];
    S[i] = run;
    run += v;
  }
  if (threadIdx.x == 0) *total = tot;
}

__global__ void __launch_bounds__(256)
lists_seg_apply_kernel(const int32_t* __restrict__ H, int64_t n, const int64_t* __restrict__ S,
                       int64_t* __restrict__ O) {
  __shared__ int64_t s[256];
  const int64_t base = blockIdx.x * (int64_t)kScanSeg + 4 * threadIdx.x;
  int64_t v[4], a = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = base + j < n ? H[base + j] : 0;
    a += v[j];
  }
  int64_t tot;
  int64_t run = S[blockIdx.x] + block_excl_scan256(a, s, &tot);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (base + j < n) O[base + j] = run;
    run += v[j];
  }
}

static hipError_t excl_scan(const int32_t* H, int64_t n, int64_t* O, int64_t* S, int64_t* total,
                            hipStream_t stream) {
  const int64_t nseg = (n + kScanSeg - 1) / kScanSeg;
  lists_seg_sums_kernel<<<(unsigned)nseg, 256, 0, stream>>>(H, n, S);
  lists_seg_scan_kernel<<<1, 256, 0, stream>>>(S, nseg, total);
  lists_seg_apply_kernel<<<(unsigned)nseg, 256, 0, stream>>>(H, n, S, O);
  return hipGetLastError();
}

// Stable scatter of the block's items by digit. Each 64-item round is ranked
// with ballots on top of per-digit running positions, into an LDS stage laid
// out by digit (the block's exclusive digit offsets come from its histogram
// column of H); the stage is then written out in order, so each digit's run
// of the block lands contiguously at O[digit][block].
template <bool FROM_POINTS>
__global__ void __launch_bounds__(64)
lists_scatter_kernel(const int32_t* __restrict__ idx, const float* __restrict__ resp, int64_t N, float thr,
                     const int32_t* __restrict__ keys_in, const int32_t* __restrict__ vals_in,
                     const int64_t* __restrict__ total, int shift, const int32_t* __restrict__ H,
                     const int64_t* __restrict__ O, int64_t B, int32_t* __restrict__ keys_out,
                     int32_t* __restrict__ vals_out) {
  __shared__ int32_t sk[kListItems], sv[kListItems];
  __shared__ int32_t loc[256], loff[256];
  __shared__ int64_t gofs[256];
  const int lane = threadIdx.x;
  // local exclusive offsets of the 256 digits (lane holds digits 4 lane .. 4 lane + 3)
  int h[4], hs = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = H[(int64_t)(4 * lane + j) * B + blockIdx.x];
    hs += h[j];
  }
  int run = wave_incl_scan(hs) - hs;
  const int nitems = __builtin_amdgcn_readlane(run + hs, 63);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    loff[4 * lane + j] = run;
    loc[4 * lane + j] = run;
    gofs[4 * lane + j] = O[(int64_t)(4 * lane + j) * B + blockIdx.x];
    run += h[j];
  }
  __syncthreads();
  const uint64_t lt = (1ull << lane) - 1ull, le = lt | (1ull << lane);
  const uint64_t gt = ~le, ge = ~lt;
  if (FROM_POINTS) {
    // all of the block's inputs are requested up front (one memory latency per block)
    constexpr int R = kListPoints / 64;
    const int64_t lo = blockIdx.x * (int64_t)kListPoints, hi = min(N, lo + kListPoints);
    int2 pk[R];
    float r1[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t n = lo + 64 * r + lane;
      if (resp) {  // top-2 pairs
        pk[r] = n < hi ? reinterpret_cast<const int2*>(idx)[n] : make_int2(0, -1);
        r1[r] = n < hi ? resp[2 * n + 1] : 0.f;
      } else {  // one assignment per point
        pk[r] = make_int2(n < hi ? idx[n] : 0, -1);
        r1[r] = 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t n = lo + 64 * r + lane;
      if (lo + 64 * r >= hi) break;
      const bool vp = n < hi;
      const int kp = pk[r].x;
      if (!resp) {  // one label per point (uniform): no second pick to rank
        const int dg = (kp >> shift) & 255;
        uint64_t b[8], mv;
        digit_ballots(vp, dg, b, &mv);
        const uint64_t m = digit_match(dg, b, mv);
        const int pos = loc[dg] + __popcll(m & lt);
        wave_lds_fence();
        if (vp) {
          sk[pos] = kp;
          sv[pos] = (int32_t)n;
          if ((m & gt) == 0) loc[dg] = pos + 1;
        }
        wave_lds_fence();
        continue;
      }
      const bool vs = vp && pk[r].y >= 0 && r1[r] >= thr;
      const int ks = vs ? pk[r].y : 0;
      const int dp = (kp >> shift) & 255, ds = (ks >> shift) & 255;
      uint64_t bp[8], bs[8], mvp, mvs;
      digit_ballots(vp, dp, bp, &mvp);
      digit_ballots(vs, ds, bs, &mvs);
      // item order in the round: (lane 0 first pick, lane 0 second pick, lane 1 first pick, ...)
      const uint64_t pp = digit_match(dp, bp, mvp), ps = digit_match(dp, bs, mvs);
      const uint64_t sp = digit_match(ds, bp, mvp), ss = digit_match(ds, bs, mvs);
      const int pos_p = loc[dp] + __popcll(pp & lt) + __popcll(ps & lt);
      const int pos_s = loc[ds] + __popcll(sp & le) + __popcll(ss & lt);
      wave_lds_fence();
      if (vp) {
        sk[pos_p] = kp;
        sv[pos_p] = (int32_t)n;
        if ((pp & gt) == 0 && (ps & ge) == 0) loc[dp] = pos_p + 1;  // last item of this digit
      }
      if (vs) {
        sk[pos_s] = ks;
        sv[pos_s] = (int32_t)n;
        if ((sp & gt) == 0 && (ss & gt) == 0) loc[ds] = pos_s + 1;
      }
      wave_lds_fence();
    }
  } else {
    constexpr int R = kListItems / 64;
    const int64_t M = *total;
    const int64_t lo = blockIdx.x * (int64_t)kListItems, hi = min(M, lo + kListItems);
    int ki[R], vi[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t i = lo + 64 * r + lane;
      ki[r] = i < hi ? keys_in[i] : 0;
      vi[r] = i < hi ? vals_in[i] : 0;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t i = lo + 64 * r + lane;
      if (lo + 64 * r >= hi) break;
      const bool v = i < hi;
      const int k = ki[r];
      const int dg = (k >> shift) & 255;
      uint64_t b[8], mv;
      digit_ballots(v, dg, b, &mv);
      const uint64_t m = digit_match(dg, b, mv);
      const int pos = loc[dg] + __popcll(m & lt);
      wave_lds_fence();
      if (v) {
        sk[pos] = k;
        sv[pos] = vi[r];
        if ((m & gt) == 0) loc[dg] = pos + 1;
      }
      wave_lds_fence();
    }
  }
  __syncthreads();
  for (int j = lane; j < nitems; j += 64) {
    const int k = sk[j];
    const int dg = (k >> shift) & 255;
    const int64_t g = gofs[dg] + (j - loff[dg]);
    keys_out[g] = k;
    vals_out[g] = sv[j];
  }
}

__global__ void lists_zero_total_kernel(int64_t* __restrict__ total) {
  if (threadIdx.x == 0) total[0] = 0;
}

// offsets[k] = first position of list k in the sorted keys (lower bound),
// offsets[K] = number of items.
__global__ void lists_offsets_kernel(const int32_t* __restrict__ keys, const int64_t* __restrict__ total, int K,
                                     int64_t* __restrict__ offsets) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k > K) return;
  const int64_t M = *total;
  int64_t lo = 0, hi = M;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (keys[mid] < k)
      lo = mid + 1;
    else
      hi = mid;
  }
  offsets[k] = lo;
}

ListsLayout lists_layout(int64_t N, int K) {
  ListsLayout L{};
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const int64_t BA = (N + kListPoints - 1) / kListPoints;
  const int64_t BB = (2 * N + kListItems - 1) / kListItems;
  L.blocks_a = BA;
  L.blocks_b = K > 256 ? BB : 0;
  const int64_t Bmax = BA > L.blocks_b ? BA : L.blocks_b;
  size_t off = 0;
  L.o_H = off;
  off += up((size_t)256 * (Bmax > 0 ? Bmax : 1) * sizeof(int32_t));
  L.o_O = off;
  off += up((size_t)256 * (Bmax > 0 ? Bmax : 1) * sizeof(int64_t));
  L.o_total = off;
  off += up(2 * sizeof(int64_t));
  L.o_S = off;  // segment sums of the scan
  off += up((size_t)((256 * (Bmax > 0 ? Bmax : 1) + kScanSeg - 1) / kScanSeg) * sizeof(int64_t));
  L.o_keys = off;  // final keys (sorted by list)
  off += up((size_t)(2 * N > 0 ? 2 * N : 1) * sizeof(int32_t));
  L.o_tmp_keys = off;
  off += up((size_t)(K > 256 && N > 0 ? 2 * N : 1) * sizeof(int32_t));
  L.o_tmp_vals = off;
  off += up((size_t)(K > 256 && N > 0 ? 2 * N : 1) * sizeof(int32_t));
  L.bytes = off;
  return L;
}

hipError_t launch_border_lists(const int32_t* idx, const float* resp, int64_t N, int K, float thr,
                               int64_t* offsets, int32_t* members, void* workspace, hipStream_t stream) {
  const ListsLayout L = lists_layout(N, K);
  char* w = static_cast<char*>(workspace);
  int32_t* H = reinterpret_cast<int32_t*>(w + L.o_H);
  int64_t* O = reinterpret_cast<int64_t*>(w + L.o_O);
  int64_t* total = reinterpret_cast<int64_t*>(w + L.o_total);
  int64_t* S = reinterpret_cast<int64_t*>(w + L.o_S);
  int32_t* keys = reinterpret_cast<int32_t*>(w + L.o_keys);
  int32_t* tkeys = reinterpret_cast<int32_t*>(w + L.o_tmp_keys);
  int32_t* tvals = reinterpret_cast<int32_t*>(w + L.o_tmp_vals);
  if (N > 0) {
    const bool two = K > 256;
    const int64_t BA = L.blocks_a;
    // pass A: digit 0 of every item, straight from (idx, resp)
    lists_hist_kernel<true><<<(unsigned)BA, 64, 0, stream>>>(idx, resp, N, thr, nullptr, nullptr, 0, H, BA);
    hipError_t e = excl_scan(H, 256 * BA, O, S, total, stream);
    if (e != hipSuccess) return e;
    lists_scatter_kernel<true><<<(unsigned)BA, 64, 0, stream>>>(idx, resp, N, thr, nullptr, nullptr, nullptr, 0,
                                                                 H, O, BA, two ? tkeys : keys, two ? tvals : members);
    if (two) {  // pass B: digit 1, from the pass-A order (stable)
      const int64_t BB = L.blocks_b;
      lists_hist_kernel<false><<<(unsigned)BB, 64, 0, stream>>>(nullptr, nullptr, 0, 0.f, tkeys, total, 8, H, BB);
      e = excl_scan(H, 256 * BB, O, S, total + 1, stream);
      if (e != hipSuccess) return e;
      lists_scatter_kernel<false><<<(unsigned)BB, 64, 0, stream>>>(nullptr, nullptr, 0, 0.f, tkeys, tvals, total, 8,
                                                                    H, O, BB, keys, members);
    }
  } else {
    lists_zero_total_kernel<<<1, 64, 0, stream>>>(total);
  }
  lists_offsets_kernel<<<(unsigned)((K + 1 + 255) / 256), 256, 0, stream>>>(keys, total, K, offsets);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Lloyd's k-means update through the sorted lists (sort-inverse update of
// the Flash-KMeans articles): each list is summed as contiguous segments of
// seg_rows members, segment sums are combined per list in segment order, and
// the centre becomes sum / count (a list with no members keeps its centre).
// seg_rows is at least kSegRows and grows with N so that all segments fit in
// one round of resident blocks (enough to fill the chip, and few partials for
// the per-list combine). Fixed orders throughout: deterministic.
// ---------------------------------------------------------------------------

constexpr int kSegRows = 512;

__global__ void kmeans_segcount_kernel(const int64_t* __restrict__ offsets, int K, int64_t seg_rows,
                                       int32_t* __restrict__ seg) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k < K) seg[k] = (int32_t)((offsets[k + 1] - offsets[k] + seg_rows - 1) / seg_rows);
}

// Block b sums segment b: rows members[start, end) of list k, where k is the
// last list whose first segment is <= b. Fixed orders throughout.
//  - fp32 rows with d % 4 == 0 (16-byte aligned): a row takes LPR lanes (the
//    power of two >= d/4) with four features each, so a wave reads 64 / LPR
//    rows per load and eight loads per lane are in flight; the row groups are
//    combined by an xor butterfly, then the four waves in order.
//  - half-precision rows with d % 8 == 0 (16-byte aligned): the same with
//    eight features per lane (LPR the power of two >= d/8), widened in
//    registers.
//  - otherwise: lanes hold features lane and lane + 64, wave w takes rows
//    start + w + 4i in groups of 8.
template <typename XT>
__global__ void __launch_bounds__(256)
kmeans_segsum_kernel(const XT* __restrict__ X, int d, const int64_t* __restrict__ offsets,
                     const int32_t* __restrict__ members, const int64_t* __restrict__ segoff, int K,
                     int64_t seg_rows, double* __restrict__ part, int vec) {
  __shared__ double s[4][128];
  const int64_t b = blockIdx.x;
  if (b >= segoff[K]) return;
  int lo = 0, hi = K - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (segoff[mid] <= b)
      lo = mid;
    else
      hi = mid - 1;
  }
  const int k = lo;
  const int64_t start = offsets[k] + (b - segoff[k]) * seg_rows;
  const int64_t end = min(start + seg_rows, offsets[k + 1]);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int G = 8;
  if (sizeof(XT) == 4 && vec == 1) {
    int LPR = 1;
    while (4 * LPR < d) LPR <<= 1;
    const int RPW = 64 / LPR, rsub = lane / LPR, q = lane - rsub * LPR;
    const bool fin = 4 * q < d;
    const float* Xf = reinterpret_cast<const float*>(X);
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    for (int64_t i0 = start + wave * RPW + rsub; i0 < end; i0 += 4 * RPW * G) {
      float4 v[G];
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const int64_t i = i0 + 4 * RPW * j;
        v[j] = (i < end && fin) ? *reinterpret_cast<const float4*>(Xf + (int64_t)members[i] * d + 4 * q)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int j = 0; j < G; ++j) {
        a0 += (double)v[j].x;
        a1 += (double)v[j].y;
        a2 += (double)v[j].z;
        a3 += (double)v[j].w;
      }
    }
    for (int o = LPR; o < 64; o <<= 1) {
      a0 += __shfl_xor(a0, o, 64);
      a1 += __shfl_xor(a1, o, 64);
      a2 += __shfl_xor(a2, o, 64);
      a3 += __shfl_xor(a3, o, 64);
    }
    if (rsub == 0 && fin) {
      s[wave][4 * q] = a0;
      s[wave][4 * q + 1] = a1;
      s[wave][4 * q + 2] = a2;
      s[wave][4 * q + 3] = a3;
    }
  } else if (sizeof(XT) == 2 && vec == 2) {
    int LPR = 1;
    while (8 * LPR < d) LPR <<= 1;
    const int RPW = 64 / LPR, rsub = lane / LPR, q = lane - rsub * LPR;
    const bool fin = 8 * q < d;
    double a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] = 0.0;
    for (int64_t i0 = start + wave * RPW + rsub; i0 < end; i0 += 4 * RPW * G) {
      uint4 v[G];
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const int64_t i = i0 + 4 * RPW * j;
        v[j] = (i < end && fin) ? *reinterpret_cast<const uint4*>(X + (int64_t)members[i] * d + 8 * q)
                                : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const XT* hv = reinterpret_cast<const XT*>(&v[j]);
#pragma unroll
        for (int u = 0; u < 8; ++u) a[u] += (double)(float)hv[u];
      }
    }
    for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
      for (int u = 0; u < 8; ++u) a[u] += __shfl_xor(a[u], o, 64);
    if (rsub == 0 && fin)
#pragma unroll
      for (int u = 0; u < 8; ++u) s[wave][8 * q + u] = a[u];
  } else {
    const int f0 = lane, f1 = lane + 64;
    double a0 = 0.0, a1 = 0.0;
    for (int64_t i0 = start + wave; i0 < end; i0 += 4 * G) {
      float v0[G], v1[G];
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const int64_t i = i0 + 4 * j;
        const bool in = i < end;
        const XT* row = X + (int64_t)(in ? members[i] : 0) * d;
        v0[j] = in && f0 < d ? (float)row[f0] : 0.f;
        v1[j] = in && f1 < d ? (float)row[f1] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < G; ++j) {
        a0 += (double)v0[j];
        a1 += (double)v1[j];
      }
    }
    s[wave][f0] = a0;
    s[wave][f1] = a1;
  }
  __syncthreads();
  if (threadIdx.x < d)
    part[b * d + threadIdx.x] = (s[0][threadIdx.x] + s[1][threadIdx.x]) + (s[2][threadIdx.x] + s[3][threadIdx.x]);
}

// One block per list: lanes take features (64 at a time), wave w the
// segments congruent to w mod 4 with eight independent sums per lane (their
// loads in flight together); the sums and then the waves combine in a fixed
// order. The centre becomes sum / count; a list with no members keeps it.
__global__ void __launch_bounds__(256)
kmeans_finalize_kernel(const double* __restrict__ part, const int64_t* __restrict__ segoff,
                       const int64_t* __restrict__ offsets, int K, int d, float* __restrict__ C,
                       int64_t* __restrict__ counts) {
  __shared__ double s[4][64];
  const int k = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t L = offsets[k + 1] - offsets[k];
  if (threadIdx.x == 0 && counts) counts[k] = L;
  if (L == 0) return;  // the whole block: the centre keeps its value
  const int64_t g0 = segoff[k], g1 = segoff[k + 1];
  for (int j0 = 0; j0 < d; j0 += 64) {
    const int j = j0 + lane;
    double a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] = 0.0;
    for (int64_t g = g0 + wave; g < g1; g += 32) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t gg = g + 4 * u;
        if (gg < g1 && j < d) a[u] += part[gg * d + j];
      }
    }
    s[wave][lane] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
    __syncthreads();
    if (wave == 0 && j < d)
      C[(int64_t)k * d + j] = (float)(((s[0][lane] + s[1][lane]) + (s[2][lane] + s[3][lane])) / (double)L);
    __syncthreads();
  }
}

// An upper bound for every choice of seg_rows >= kSegRows: the lists'
// segments number at most ceil(N / kSegRows) + K.
int64_t kmeans_max_segments(int64_t N, int K) { return (N + kSegRows - 1) / kSegRows + K; }

hipError_t launch_kmeans_update(const void* X, int x_dtype, int64_t N, int d, int K, const int64_t* offsets,
                                const int32_t* members, int32_t* seg, int64_t* segoff, int64_t* scan_tmp,
                                double* part, int64_t max_segments, float* C, int64_t* counts,
                                hipStream_t stream) {
  hipError_t e = with_x_type(x_dtype, X, [&](auto x) {
    using XT = std::remove_cv_t<std::remove_pointer_t<decltype(x)>>;
    auto fn = kmeans_segsum_kernel<XT>;
    // Blocks resident at once over 256 CUs; the lists' segments number at
    // most ceil(N / seg_rows) + K, so seg_rows is chosen to keep that within
    // one such round (never below kSegRows, which the workspace is sized for).
    static std::atomic<int> resident{0};
    int per_cu = resident.load(std::memory_order_relaxed);
    if (per_cu == 0) {
      hipError_t q = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0);
      if (q != hipSuccess) return q;
      per_cu = std::max(per_cu, 1);
      resident.store(per_cu, std::memory_order_relaxed);
    }
    const int64_t round = 256 * (int64_t)per_cu - K;
    const int64_t seg_rows = round > 0 ? std::max<int64_t>(kSegRows, (N + round - 1) / round) : kSegRows;
    kmeans_segcount_kernel<<<(unsigned)((K + 255) / 256), 256, 0, stream>>>(offsets, K, seg_rows, seg);
    hipError_t e2 = excl_scan(seg, K, segoff, scan_tmp, segoff + K, stream);
    if (e2 != hipSuccess) return e2;
    const bool al16 = reinterpret_cast<uintptr_t>(x) % 16 == 0;
    const int vec = sizeof(XT) == 4 ? (d % 4 == 0 && al16 ? 1 : 0) : (d % 8 == 0 && al16 ? 2 : 0);
    const int64_t blocks = std::min<int64_t>(max_segments, (N + seg_rows - 1) / seg_rows + K);
    fn<<<(unsigned)blocks, 256, 0, stream>>>(x, d, offsets, members, segoff, K, seg_rows, part, vec);
    return hipGetLastError();
  });
  if (e != hipSuccess) return e;
  kmeans_finalize_kernel<<<(unsigned)K, 256, 0, stream>>>(part, segoff, offsets, K, d, C, counts);
  return hipGetLastError();
}

}  // namespace gmm
