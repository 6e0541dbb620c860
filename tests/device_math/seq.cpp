// Checks the correctly rounded square root and the shared-reciprocal
// quotients of the dual update (tv_fgp_device.hpp) against the host's IEEE
// sqrtf and division, for both faithful estimates of the hardware square
// root and reciprocal (tv_fgp_hwmath.hpp in this directory):
//  - the square root is the rounded one from either estimate;
//  - the refined reciprocal is the rounded 1/d from either estimate, except
//    for a divisor whose significand is all ones, where one Newton step from
//    the lower estimate stops half an ulp short;
//  - from the rounded reciprocal the quotients are the IEEE ones, and from
//    the other estimate too but for those divisors.
// So besides its one-ulp bound the hardware must give a rounded refined
// reciprocal at all-ones divisors; the GPU test checks every divisor.
// Prints mismatch counts and exits nonzero on any unexpected mismatch.
// Test infrastructure only.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tv_fgp_device.hpp"

thread_local EmulDim3 threadIdx, blockIdx, gridDim, blockDim;

namespace tvfgp {
int hw_mode = 0;
}

static uint32_t bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}
static float from_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// splitmix64
static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static uint64_t next_u64() {
  uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

static bool all_ones(float d) { return (bits(d) & 0x7fffffu) == 0x7fffffu; }

// 1 for a quotient that differs from the IEEE one where it must not (with
// the lower reciprocal estimate, all-ones divisors are not counted; they
// are tallied in ones_missed instead)
static long ones_missed = 0;
static long div_check(float n, float d) {
  const float r = tvfgp::recip_refined(d);
  const bool miss = bits(tvfgp::div_by_refined(n, d, r)) != bits(n / d);
  if (miss && tvfgp::hw_mode == 1 && all_ones(d)) {
    ++ones_missed;
    return 0;
  }
  return miss;
}

int main() {
  long bad_sqrt = 0, bad_div = 0, bad_key = 0, n_sqrt = 0, n_div = 0;
  long bad_recip[2] = {0, 0}, ones_recip[2] = {0, 0};
  for (int mode = 0; mode < 2; ++mode) {
    tvfgp::hw_mode = mode;
    // every float in [1 + 2^-22, 4): all significands at both exponent
    // parities (scaling by 4 is exact, so this covers every x > 1 short of
    // the top binade), then the top binades and +inf
    for (uint32_t u = bits(1.0f) + 2; u < bits(4.0f); ++u, ++n_sqrt) {
      const float x = from_bits(u);
      bad_sqrt += bits(tvfgp::sqrt_above_one(x)) != bits(sqrtf(x));
    }
    for (uint32_t u = bits(0x1p+126f); u <= bits(INFINITY); ++u, ++n_sqrt) {
      const float x = from_bits(u);
      bad_sqrt += bits(tvfgp::sqrt_above_one(x)) != bits(sqrtf(x));
    }
    // the refined reciprocal of every d in (1, 2) (and so, scaling by
    // powers of two being exact, of every d in (1, 2^26))
    for (uint32_t u = bits(1.0f) + 1; u < bits(2.0f); ++u) {
      const float d = from_bits(u);
      if (bits(tvfgp::recip_refined(d)) != bits(1.0f / d)) {
        if (all_ones(d))
          ++ones_recip[mode];
        else
          ++bad_recip[mode];
      }
    }
    // quotients n / d with d in (1, 2^26) and |n| in [2^-100, d] or 0
    for (long i = 0; i < (1l << 23); ++i, ++n_div) {
      const uint64_t a = next_u64(), b = next_u64();
      const int ed = (int)(a % 26);
      float d = ldexpf(1.0f + (float)((a >> 8) & 0x7fffff) * 0x1p-23f, ed);
      if (d <= 1.0f) d = 0x1.000002p+0f;
      const int en = (int)((b >> 40) % 128);  // |n| from about d down to 2^-100
      float n = ldexpf(1.0f + (float)(b & 0x7fffff) * 0x1p-23f, ed - en);
      if (fabsf(n) < 0x1p-100f) n = 0x1p-100f;
      if (fabsf(n) > d) n = d;
      if (b >> 63) n = -n;
      bad_div += div_check(n, d);
      // divisor with an all-ones significand, and n = d, -d, 0, -0
      const float dm = ldexpf(0x1.fffffep+0f, ed) > 1.0f ? ldexpf(0x1.fffffep+0f, ed) : 0x1.fffffep+0f;
      bad_div += div_check(n > dm ? dm : (n < -dm ? -dm : n), dm);
      if ((i & 1023) == 0) {
        bad_div += div_check(d, d) + div_check(-d, d) + div_check(0.0f, d) + div_check(-0.0f, d);
        n_div += 4;
      }
      // quotients next to a rounding midpoint: n = d (y + ulp(y) / 2 + t)
      const float y = 0.5f + (float)((a >> 31) & 0x7fffff) * 0x1p-24f;
      const double mid = (double)y + 0x1p-25 + (double)((int)(b % 5) - 2) * 0x1p-49;
      const float nm = (float)((double)d * mid);
      if (fabsf(nm) <= d && nm != 0.0f) bad_div += div_check(nm, d);
      n_div += 2;
    }
  }
  // the range key: below kTinyKey exactly for nonzero |a| < 2^-100
  const float probes[] = {0.0f, -0.0f, 0x1p-100f, -0x1p-100f, nextafterf(0x1p-100f, 0.0f),
                          -nextafterf(0x1p-100f, 0.0f), 0x1p-149f, -0x1p-149f, 0x1p-126f,
                          1.0f, -1.0f, 3.0e38f, INFINITY, -INFINITY};
  const bool tiny[] = {false, false, false, false, true, true, true, true, true,
                       false, false, false, false, false};
  for (int i = 0; i < (int)(sizeof(probes) / sizeof(probes[0])); ++i)
    bad_key += (tvfgp::tiny_key(probes[i]) < tvfgp::kTinyKey) != tiny[i];
  printf("sqrt %ld of %ld\n", bad_sqrt, n_sqrt);
  printf("recip rounded-estimate %ld (all-ones %ld), other-estimate %ld (all-ones %ld)\n",
         bad_recip[0], ones_recip[0], bad_recip[1], ones_recip[1]);
  printf("div %ld of %ld (other estimate, all-ones divisors: %ld)\nkey %ld\n", bad_div, n_div,
         ones_missed, bad_key);
  return (bad_sqrt || bad_div || bad_key || bad_recip[0] || bad_recip[1] || ones_recip[0]) ? 1 : 0;
}
