// Device helpers shared by the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>

namespace gmm {

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts by 1, 2,
// 4 and 8 within each row of 16 lanes, then the last lane of row 0 (row 2)
// is added to row 1 (row 3), and the last lane of row 1 to rows 2 and 3.
// Lanes whose DPP source lies outside the row (or whose row is masked off)
// read 0.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return v;
}

// Calls f with X cast to its element type: 0 float, 1 IEEE half, 2 bfloat16.
template <typename F>
hipError_t with_x_type(int x_dtype, const void* X, F&& f) {
  if (x_dtype == 1) return f(reinterpret_cast<const _Float16*>(X));
  if (x_dtype == 2) return f(reinterpret_cast<const __bf16*>(X));
  return f(reinterpret_cast<const float*>(X));
}

}  // namespace gmm
