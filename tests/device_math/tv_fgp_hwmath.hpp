// Host stand-ins for the gfx950 estimate instructions that return either
// faithful neighbour of the true value, chosen by hw_mode (0: the correctly
// rounded one, 1: the other float on the far side of the true value), so the
// correctly rounded square root and quotients of tv_fgp_device.hpp can be
// checked against every estimate the hardware's one-ulp bound admits.  This
// directory comes first on the include path of seq.cpp.  Test
// infrastructure only.
#pragma once

#include <math.h>

namespace tvfgp {

extern int hw_mode;

// The faithful neighbour of rn away from it, given whether the true value
// lies above rn.
inline float other_side(float rn, bool above) {
  return nextafterf(rn, above ? INFINITY : -INFINITY);
}

inline float hw_sqrt_estimate(float x) {
  const float rn = sqrtf(x);
  if (hw_mode == 0 || isinf(x)) return rn;
  return other_side(rn, (double)rn * (double)rn < (double)x);  // exact in double
}

inline float hw_rcp_estimate(float x) {
  const float rn = 1.0f / x;
  if (hw_mode == 0) return rn;
  return other_side(rn, (double)rn * (double)x < 1.0);
}

inline double hw_rsq_estimate(double x) { return 1.0 / sqrt(x); }

inline float hw_div_fixup(float quot, float den, float num) {
  const bool neg = signbit(den) != signbit(num);
  if (num == 0.0f) return neg ? -0.0f : 0.0f;
  return neg ? -fabsf(quot) : fabsf(quot);
}

}  // namespace tvfgp
