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
// stably with ballots. Everything is integer work and deterministic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gmm_internal.hpp"

namespace gmm {

constexpr int kListPoints = 2048;  // points per block in the pass over (idx, resp)
constexpr int kListItems = 4096;   // items per block in the second pass

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

// Items of point n: (idx[n][0], n) always, (idx[n][1], n) if it is a border vector.
__device__ __forceinline__ bool second_pick(const int32_t* idx, const float* resp, int64_t n, float thr) {
  return idx[2 * n + 1] >= 0 && resp[2 * n + 1] >= thr;
}

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
    const int64_t lo = blockIdx.x * (int64_t)kListPoints, hi = min(N, lo + kListPoints);
    for (int64_t n = lo + lane; n < hi; n += 64) {
      atomicAdd(&h[(idx[2 * n] >> shift) & 255], 1);
      if (second_pick(idx, resp, n, thr)) atomicAdd(&h[(idx[2 * n + 1] >> shift) & 255], 1);
    }
  } else {
    const int64_t M = *total;
    const int64_t lo = blockIdx.x * (int64_t)kListItems, hi = min(M, lo + kListItems);
    for (int64_t i = lo + lane; i < hi; i += 64) atomicAdd(&h[(keys[i] >> shift) & 255], 1);
  }
  __syncthreads();
  for (int i = lane; i < 256; i += 64) H[(int64_t)i * B + blockIdx.x] = h[i];
}

// Exclusive scan of H (n = 256 * B entries, in index order) -> O; the grand
// total goes to *total. One block of 1024 threads, each summing a contiguous
// segment, then a scan of the 1024 segment sums.
__global__ void __launch_bounds__(1024)
lists_scan_kernel(const int32_t* __restrict__ H, int64_t n, int64_t* __restrict__ O, int64_t* __restrict__ total) {
  __shared__ int64_t s[1024];
  const int t = threadIdx.x;
  const int64_t per = (n + 1023) / 1024;
  const int64_t lo = min(n, t * per), hi = min(n, lo + per);
  int64_t a = 0;
  for (int64_t i = lo; i < hi; ++i) a += H[i];
  s[t] = a;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive Hillis-Steele scan
    const int64_t v = t >= o ? s[t - o] : 0;
    __syncthreads();
    s[t] += v;
    __syncthreads();
  }
  int64_t run = s[t] - a;
  for (int64_t i = lo; i < hi; ++i) {
    O[i] = run;
    run += H[i];
  }
  if (t == 1023) *total = s[1023];
}

// Stable scatter of the block's items by digit: each 64-item round is ranked
// with ballots, on top of per-digit running positions kept in LDS.
template <bool FROM_POINTS>
__global__ void __launch_bounds__(64)
lists_scatter_kernel(const int32_t* __restrict__ idx, const float* __restrict__ resp, int64_t N, float thr,
                     const int32_t* __restrict__ keys_in, const int32_t* __restrict__ vals_in,
                     const int64_t* __restrict__ total, int shift, const int64_t* __restrict__ O, int64_t B,
                     int32_t* __restrict__ keys_out, int32_t* __restrict__ vals_out) {
  __shared__ int64_t base[256];
  const int lane = threadIdx.x;
  for (int i = lane; i < 256; i += 64) base[i] = O[(int64_t)i * B + blockIdx.x];
  __syncthreads();
  const uint64_t lt = (1ull << lane) - 1ull, le = lt | (1ull << lane);
  const uint64_t gt = ~le, ge = ~lt;
  if (FROM_POINTS) {
    const int64_t lo = blockIdx.x * (int64_t)kListPoints, hi = min(N, lo + kListPoints);
    for (int64_t r0 = lo; r0 < hi; r0 += 64) {
      const int64_t n = r0 + lane;
      const bool vp = n < hi;
      const int kp = vp ? idx[2 * n] : 0;
      const bool vs = vp && second_pick(idx, resp, n, thr);
      const int ks = vs ? idx[2 * n + 1] : 0;
      const int dp = (kp >> shift) & 255, ds = (ks >> shift) & 255;
      uint64_t bp[8], bs[8], mvp, mvs;
      digit_ballots(vp, dp, bp, &mvp);
      digit_ballots(vs, ds, bs, &mvs);
      // item order in the round: (lane 0 first pick, lane 0 second pick, lane 1 first pick, ...)
      const uint64_t pp = digit_match(dp, bp, mvp), ps = digit_match(dp, bs, mvs);
      const uint64_t sp = digit_match(ds, bp, mvp), ss = digit_match(ds, bs, mvs);
      const int64_t pos_p = base[dp] + __popcll(pp & lt) + __popcll(ps & lt);
      const int64_t pos_s = base[ds] + __popcll(sp & le) + __popcll(ss & lt);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (vp) {
        keys_out[pos_p] = kp;
        vals_out[pos_p] = (int32_t)n;
        if ((pp & gt) == 0 && (ps & ge) == 0) base[dp] = pos_p + 1;  // last item of this digit
      }
      if (vs) {
        keys_out[pos_s] = ks;
        vals_out[pos_s] = (int32_t)n;
        if ((sp & gt) == 0 && (ss & gt) == 0) base[ds] = pos_s + 1;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  } else {
    const int64_t M = *total;
    const int64_t lo = blockIdx.x * (int64_t)kListItems, hi = min(M, lo + kListItems);
    for (int64_t r0 = lo; r0 < hi; r0 += 64) {
      const int64_t i = r0 + lane;
      const bool v = i < hi;
      const int k = v ? keys_in[i] : 0;
      const int dg = (k >> shift) & 255;
      uint64_t b[8], mv;
      digit_ballots(v, dg, b, &mv);
      const uint64_t m = digit_match(dg, b, mv);
      const int64_t pos = base[dg] + __popcll(m & lt);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (v) {
        keys_out[pos] = k;
        vals_out[pos] = vals_in[i];
        if ((m & gt) == 0) base[dg] = pos + 1;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
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
  int32_t* keys = reinterpret_cast<int32_t*>(w + L.o_keys);
  int32_t* tkeys = reinterpret_cast<int32_t*>(w + L.o_tmp_keys);
  int32_t* tvals = reinterpret_cast<int32_t*>(w + L.o_tmp_vals);
  if (N > 0) {
    const bool two = K > 256;
    const int64_t BA = L.blocks_a;
    // pass A: digit 0 of every item, straight from (idx, resp)
    lists_hist_kernel<true><<<(unsigned)BA, 64, 0, stream>>>(idx, resp, N, thr, nullptr, nullptr, 0, H, BA);
    lists_scan_kernel<<<1, 1024, 0, stream>>>(H, 256 * BA, O, total);
    lists_scatter_kernel<true><<<(unsigned)BA, 64, 0, stream>>>(idx, resp, N, thr, nullptr, nullptr, nullptr, 0,
                                                                 O, BA, two ? tkeys : keys, two ? tvals : members);
    if (two) {  // pass B: digit 1, from the pass-A order (stable)
      const int64_t BB = L.blocks_b;
      lists_hist_kernel<false><<<(unsigned)BB, 64, 0, stream>>>(nullptr, nullptr, 0, 0.f, tkeys, total, 8, H, BB);
      lists_scan_kernel<<<1, 1024, 0, stream>>>(H, 256 * BB, O, total + 1);
      lists_scatter_kernel<false><<<(unsigned)BB, 64, 0, stream>>>(nullptr, nullptr, 0, 0.f, tkeys, tvals, total, 8,
                                                                    O, BB, keys, members);
    }
  } else {
    lists_zero_total_kernel<<<1, 64, 0, stream>>>(total);
  }
  lists_offsets_kernel<<<(unsigned)((K + 1 + 255) / 256), 256, 0, stream>>>(keys, total, K, offsets);
  return hipGetLastError();
}

}  // namespace gmm
