// Host stand-ins for the three gfx950 instructions of tv_fgp_hwmath.hpp, so
// the kernel headers compile and run as ordinary C++ (this directory comes
// first on the include path of the CPU builds).  Test infrastructure only.
// The estimates here are the correctly rounded values, which lie within the
// one ulp the device code allows for, so the emulated kernels produce the
// same bits as the GPU.
#pragma once

#include <math.h>

namespace tvfgp {

inline float hw_sqrt_estimate(float x) { return sqrtf(x); }

inline float hw_rcp_estimate(float x) { return 1.0f / x; }

inline double hw_rsq_estimate(double x) { return 1.0 / sqrt(x); }

// One thread stands for its wave, and there is no issue priority.
inline int hw_wave_uniform(int v) { return v; }
inline void hw_raise_priority() {}

// The cases the dual update reaches: a finite divisor above 1 and a finite
// numerator; the quotient takes the sign of num / den, a zero numerator gives
// a zero of that sign.
inline float hw_div_fixup(float quot, float den, float num) {
  const bool neg = signbit(den) != signbit(num);
  if (num == 0.0f) return neg ? -0.0f : 0.0f;
  return neg ? -fabsf(quot) : fabsf(quot);
}

}  // namespace tvfgp
