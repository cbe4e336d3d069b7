// Peak-rate probes: the rates this GPU actually reaches on the two resources
// that bound the E-step kernels (matrix-core issue for the score and
// statistics contractions, HBM reads for streaming X). The kernels do no
// useful work; they exist so that a measured fraction can be quoted beside
// the datasheet fraction.
#include "../../include/gmm_peaks.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gmm {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef double v4d __attribute__((ext_vector_type(4)));

// Each wave keeps four independent 32x32x2 fp32 accumulator chains and
// issues eight MFMAs per loop trip, so the matrix core always has an
// independent instruction ready; the operands change every trip.
__global__ void __launch_bounds__(256) peak_mfma_f32_kernel(int64_t trips, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  float a = 1.0f + 1e-7f * (float)lane, b = 1.0f - 1e-7f * (float)lane;
  v16f c0, c1, c2, c3;
#pragma unroll
  for (int j = 0; j < 16; ++j) c0[j] = c1[j] = c2[j] = c3[j] = 0.f;
#pragma unroll 1
  for (int64_t t = 0; t < trips; ++t) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x2f32(b, b, c3, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(b, a, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x2f32(b, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, a, c3, 0, 0, 0);
    a += 1e-9f;
    b -= 1e-9f;
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += (c0[j] + c1[j]) + (c2[j] + c3[j]);
  out[blockIdx.x * (int64_t)blockDim.x + threadIdx.x] = s;
}

// The same on the 16x16x4 fp64 MFMA (four chains, eight per trip).
__global__ void __launch_bounds__(256) peak_mfma_f64_kernel(int64_t trips, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  double a = 1.0 + 1e-12 * (double)lane, b = 1.0 - 1e-12 * (double)lane;
  v4d c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
#pragma unroll 1
  for (int64_t t = 0; t < trips; ++t) {
    c0 = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f64_16x16x4f64(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f64_16x16x4f64(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f64_16x16x4f64(b, b, c3, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f64_16x16x4f64(b, a, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f64_16x16x4f64(b, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f64_16x16x4f64(a, a, c3, 0, 0, 0);
    a += 1e-15;
    b -= 1e-15;
  }
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) s += (c0[j] + c1[j]) + (c2[j] + c3[j]);
  out[blockIdx.x * (int64_t)blockDim.x + threadIdx.x] = (float)s;
}

// Streams `n16` 16-byte chunks (grid-stride, four loads in flight per
// thread) and folds them into one word per thread; the store is taken only
// for a value no real input produces in practice, so the loads cannot be
// dropped and almost nothing is written.
__global__ void __launch_bounds__(256) peak_hbm_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                            uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 v0 = p[i], v1 = p[i + stride], v2 = p[i + 2 * stride], v3 = p[i + 3 * stride];
    acc ^= (v0.x + v1.y) ^ (v2.z + v3.w) ^ (v0.w + v1.z) ^ (v2.y + v3.x) ^ (v0.y ^ v1.x ^ v2.w ^ v3.z) ^
           (v0.z + v1.w + v2.x + v3.y);
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= (v.x + v.y) ^ (v.z + v.w);
  }
  if (acc == 0x9e3779b9u) out[blockIdx.x * (int64_t)blockDim.x + threadIdx.x] = acc;
}

// Co-issue probe: whether fp32 vector work runs beside fp32 matrix-core work
// on a SIMD. Blocks of eight waves; with one block per CU (the registers
// allow no more) waves w and w + 4 share SIMD w % 4. Per trip a wave that
// does matrix work issues eight independent 32x32x2 fp32 MFMAs (eight
// chains), and a wave that does vector work issues 128 independent fp32
// FMAs (32 chains, four each), about the same SIMD time each. Modes: 0
// matrix only, 1 vector only, 2 both in every wave (interleaved), 3 waves
// 0-3 matrix only and waves 4-7 vector only.
template <int MODE>
__global__ void __launch_bounds__(512) peak_coissue_kernel(int64_t trips, float* __restrict__ out) {
  const int tid = threadIdx.x, wave = tid >> 6;
  const bool mat = MODE == 0 || MODE == 2 || (MODE == 3 && wave < 4);
  const bool vec = MODE == 1 || MODE == 2 || (MODE == 3 && wave >= 4);
  v16f acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = 1.0f + 1e-3f * (float)i + 1e-7f * (float)tid;
  const float a = 0.999f, b = 1e-6f;
  float x = 1.0f + 1e-7f * (float)(tid & 63), y = 1.0f;
#pragma unroll 1
  for (int64_t t = 0; t < trips; ++t) {
    if (mat) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, acc[i], 0, 0, 0);
    }
    if (vec) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = __builtin_fmaf(v[i], a, b);
    }
    x += 1e-9f;
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][15];
#pragma unroll
  for (int i = 0; i < 32; ++i) s += v[i];
  out[blockIdx.x * (int64_t)blockDim.x + tid] = s;
}

}  // namespace gmm

using namespace gmm;

extern "C" {

int gmm_peak_mfma(int32_t precision, int64_t trips, int32_t blocks, float* out, void* stream) {
  if ((precision != GMM_PEAK_FP32 && precision != GMM_PEAK_FP64) || trips < 1 || blocks < 1 || !out) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (precision == GMM_PEAK_FP32)
    peak_mfma_f32_kernel<<<blocks, 256, 0, s>>>(trips, out);
  else
    peak_mfma_f64_kernel<<<blocks, 256, 0, s>>>(trips, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

double gmm_peak_mfma_flops(int32_t precision, int64_t trips, int32_t blocks) {
  // 8 MFMAs per trip and wave, four waves per block; a 32x32x2 fp32 MFMA is
  // 32*32*2 multiply-adds (4096 flops), a 16x16x4 fp64 one 16*16*4 (2048).
  const double per = precision == GMM_PEAK_FP32 ? 4096.0 : 2048.0;
  return 8.0 * per * 4.0 * (double)blocks * (double)trips;
}

int gmm_peak_hbm_read(const void* buf, size_t bytes, int32_t blocks, uint32_t* out, void* stream) {
  if (!buf || !out || blocks < 1 || bytes < 16 || reinterpret_cast<uintptr_t>(buf) % 16 != 0) return -1;
  peak_hbm_read_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4*>(buf), (int64_t)(bytes / 16), out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int gmm_peak_coissue(int32_t mode, int64_t trips, int32_t blocks, float* out, void* stream) {
  if (mode < 0 || mode > 3 || trips < 1 || blocks < 1 || !out) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (mode) {
    case 0: peak_coissue_kernel<0><<<blocks, 512, 0, s>>>(trips, out); break;
    case 1: peak_coissue_kernel<1><<<blocks, 512, 0, s>>>(trips, out); break;
    case 2: peak_coissue_kernel<2><<<blocks, 512, 0, s>>>(trips, out); break;
    default: peak_coissue_kernel<3><<<blocks, 512, 0, s>>>(trips, out); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
