// Small device helpers shared by the scoring and attention kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tri {

// 32-bit word i (0..3) of a 16-byte fragment; i is a constant after unrolling, so this folds
// to a register selection.
__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// The two bfloat16 halves of a word, widened exactly to float32 (one shift or one mask).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Sum over the 8 lanes of an aligned 8-lane group (lanes 8k..8k+7): two quad swaps and a
// half-row mirror, all DPP.
__device__ __forceinline__ float sum8(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  return v;
}

}  // namespace tri
