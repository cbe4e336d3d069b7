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

}  // extern "C"
