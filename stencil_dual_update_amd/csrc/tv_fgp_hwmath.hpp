// Single gfx950 instructions that the dual update builds its correctly
// rounded square root and quotients from (tv_fgp_device.hpp), and the
// duality gap its double square root (tv_fgp_gap_kernel.hpp), and the wave
// controls of the three-step kernel (tv_fgp_tb3_kernel.hpp).  Included as
// <tv_fgp_hwmath.hpp> so that a host build of the kernel headers can put its
// own stand-ins first on the include path.
#pragma once

#include <hip/hip_runtime.h>

namespace tvfgp {

// v_sqrt_f32: the square root, within one ulp.
__device__ __forceinline__ float hw_sqrt_estimate(float x) { return __builtin_amdgcn_sqrtf(x); }

// v_rcp_f32: the reciprocal, within one ulp.
__device__ __forceinline__ float hw_rcp_estimate(float x) { return __builtin_amdgcn_rcpf(x); }

// v_rsq_f64: the reciprocal square root of a double, to about single
// precision (the seed of the double square root's refinement).
__device__ __forceinline__ double hw_rsq_estimate(double x) { return __builtin_amdgcn_rsq(x); }

// v_readfirstlane_b32: v as the wave's first active lane holds it, a value
// the compiler knows to be the same in every lane (scalar).
__device__ __forceinline__ int hw_wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// s_setprio 1: the wave's instructions issue ahead of priority-0 waves on
// its SIMD.
__device__ __forceinline__ void hw_raise_priority() { __builtin_amdgcn_s_setprio(1); }

// v_div_fixup_f32: the last instruction of the IEEE division sequence.  It
// returns quot with the sign of num / den, or the special value that zero,
// infinite or NaN operands call for.
__device__ __forceinline__ float hw_div_fixup(float quot, float den, float num) {
  return __builtin_amdgcn_div_fixupf(quot, den, num);
}

}  // namespace tvfgp
