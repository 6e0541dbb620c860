// Device-side building blocks of the FGP step, shared by every kernel variant.
//
// Every variant evaluates the primal z and the dual update through these two
// functions, so all variants produce the same bits.  Expressions follow the
// page "TV solver: the FGP step on the GPU", section "What one step does";
// the evaluation order is fixed here and multiply-add contraction is off.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <tv_fgp_hwmath.hpp>

#pragma clang fp contract(off)

namespace tvfgp {

// Tiling shared by the kernels: a workgroup of 256 threads covers a
// 64 (x) by 4 (y) tile, one wave64 per x-row, so every wave load is a
// contiguous run of 64 floats.
constexpr int kTileX = 64;
constexpr int kTileY = 4;
constexpr int kBlock = kTileX * kTileY;
// Upper bound on the grid; larger problems loop over tiles.  A multiple of
// 8 so that tile t keeps landing on XCD t % 8 in later rounds.
constexpr int64_t kMaxGrid = 1 << 20;

template <typename I>
struct Geometry {
  I nx, ny, nz;
  I sy, sz;  // strides of y and z
  I tiles_x, tiles_y, tiles_z;
  I ntiles;
  I planes;  // planes per tile along z (marching kernels)
};

template <typename I>
inline Geometry<I> make_geometry(int64_t nx, int64_t ny, int64_t nz,
                                 int64_t planes) {
  Geometry<I> g;
  g.nx = (I)nx;
  g.ny = (I)ny;
  g.nz = (I)nz;
  g.sy = (I)nx;
  g.sz = (I)(nx * ny);
  g.tiles_x = (I)((nx + kTileX - 1) / kTileX);
  g.tiles_y = (I)((ny + kTileY - 1) / kTileY);
  g.planes = (I)planes;
  g.tiles_z = (I)((nz + planes - 1) / planes);
  g.ntiles = g.tiles_x * g.tiles_y * g.tiles_z;
  return g;
}

inline unsigned grid_for(int64_t ntiles) {
  return (unsigned)(ntiles < kMaxGrid ? ntiles : kMaxGrid);
}


// z(j) = max(b(j) - lambda * L(r)(j), 0) with
// L(r)(j) = (r_x(j) - r_x(j-e_x)) + (r_y(j) - r_y(j-e_y)) + (r_z(j) - r_z(j-e_z)),
// summed as (d_x + d_y) + d_z.  The *_lo arguments are the lower neighbours,
// already replaced by 0 below the lower face.  max(u, 0) is (u > 0) ? u : +0,
// which maps NaN and -0 to +0.
__device__ __forceinline__ float primal_z(float bj, float rx, float rx_lo,
                                          float ry, float ry_lo, float rz,
                                          float rz_lo, float lam) {
  const float dx = rx - rx_lo;
  const float dy = ry - ry_lo;
  const float dz = rz - rz_lo;
  const float lr = (dx + dy) + dz;
  const float u = bj - lam * lr;
  return u > 0.0f ? u : 0.0f;
}

// Correctly rounded square root of x > 1 (+inf included).  The hardware
// estimate s is within one ulp; the residuals x - s's of its two neighbours
// s' decide whether a neighbour is the rounded root.  This is the correction
// the compiler wraps around v_sqrt_f32 for sqrtf, without the rescaling of
// tiny inputs and the pass-through of zero, which inputs above 1 never need
// (+inf comes out as +inf), so the bits are those of sqrtf.
__device__ __forceinline__ float sqrt_above_one(float x) {
  const float s = hw_sqrt_estimate(x);
  const uint32_t u = __builtin_bit_cast(uint32_t, s);
  const float sd = __builtin_bit_cast(float, u - 1u);
  const float su = __builtin_bit_cast(float, u + 1u);
  const float vd = __builtin_fmaf(-sd, s, x);
  const float vu = __builtin_fmaf(-su, s, x);
  const float t = vd <= 0.0f ? sd : s;
  return vu > 0.0f ? su : t;
}

// 1/d from the hardware estimate and one Newton step, r + r (1 - d r): the
// reciprocal half of the compiler's IEEE division sequence, here computed
// once for the three quotients that share the divisor d.
__device__ __forceinline__ float recip_refined(float d) {
  const float r = hw_rcp_estimate(d);
  const float e = __builtin_fmaf(-d, r, 1.0f);
  return __builtin_fmaf(e, r, r);
}

// n / d given r = recip_refined(d): the estimate n r, two corrections by the
// residual n - d y, then the fix-up of sign and special cases.  These are the
// steps of the compiler's IEEE division n / d with its operand rescaling
// left out, so the result is bit for bit the IEEE quotient wherever that
// rescaling is the identity; it is for d in (1, 2^26) and n either zero or
// of magnitude at least 2^-100 (quotient and divisor well inside the normal
// range).
__device__ __forceinline__ float div_by_refined(float n, float d, float r) {
  float y = n * r;
  float e = __builtin_fmaf(-d, y, n);
  y = __builtin_fmaf(e, r, y);
  e = __builtin_fmaf(-d, y, n);
  y = __builtin_fmaf(e, r, y);
  return hw_div_fixup(y, d, n);
}

// Twice the bit pattern of a (the sign shifted out) minus one, so that zero
// wraps round to the top: the key lies below kTinyKey exactly when a is
// nonzero with |a| < 2^-100 (whose pattern is 0x0d800000).
__device__ __forceinline__ uint32_t tiny_key(float a) {
  return (__builtin_bit_cast(uint32_t, a) << 1) - 1u;
}
constexpr uint32_t kTinyKey = 0x1affffffu;

// Dual step, projection and momentum at voxel i.
//   g_a = z(i) - z(i+e_a), 0 at the upper a-face (has_a false)
//   q_a = r_a(i) + c * g_a,  c = 1/(12 lambda)
//   p'  = q / max(1, |q|),   |q| = sqrt((q_x^2 + q_y^2) + q_z^2)
//         (IEEE square root and divisions, skipped where they cannot matter)
//   r_out = p' + m (p' - p);  p <- p'
// p0..p2 hold p(i) on entry and p' on return.
__device__ __forceinline__ void dual_update(float zi, float zx, float zy,
                                            float zz, bool has_x, bool has_y,
                                            bool has_z, float r0, float r1,
                                            float r2, float &p0, float &p1,
                                            float &p2, float c, float m,
                                            float &o0, float &o1, float &o2) {
  const float gx = has_x ? zi - zx : 0.0f;
  const float gy = has_y ? zi - zy : 0.0f;
  const float gz = has_z ? zi - zz : 0.0f;
  const float qx = r0 + c * gx;
  const float qy = r1 + c * gy;
  const float qz = r2 + c * gz;
  const float s2 = (qx * qx + qy * qy) + qz * qz;
  // s = max(1, |q|) and p' = q / s.  The rounded square root exceeds 1 exactly
  // when s2 > 1 + 2^-23 (sqrt(1 + 2^-23) rounds to 1), so below that s = 1 and
  // p' = q / 1 = q: the square root and the three divisions are skipped, and
  // a wave whose lanes all stay inside the ball skips them entirely.  NaN
  // takes the s = 1 branch, as max(1, NaN) does.
  // Above it |q| > 1: the root comes from sqrt_above_one and, where every
  // operand lies in div_by_refined's range (always, short of components
  // below 2^-100 or |q| of 2^26 and more), the quotients share one refined
  // reciprocal; elsewhere they are plain IEEE divisions.  Both give the bits
  // of q / sqrtf(s2).
  float px = qx, py = qy, pz = qz;
  if (s2 > 0x1.000002p+0f) {
    const float nq = sqrt_above_one(s2);
    uint32_t key = tiny_key(qx) < tiny_key(qy) ? tiny_key(qx) : tiny_key(qy);
    key = key < tiny_key(qz) ? key : tiny_key(qz);
    if ((nq < 0x1p+26f) & (key >= kTinyKey)) {
      const float rq = recip_refined(nq);
      px = div_by_refined(qx, nq, rq);
      py = div_by_refined(qy, nq, rq);
      pz = div_by_refined(qz, nq, rq);
    } else {
      px = qx / nq;
      py = qy / nq;
      pz = qz / nq;
    }
  }
  o0 = px + m * (px - p0);
  o1 = py + m * (py - p1);
  o2 = pz + m * (pz - p2);
  p0 = px;
  p1 = py;
  p2 = pz;
}

// Load src[cond ? idx : alt] (widened to float) and return it if cond, else
// +0.  Both indices must be in bounds; the address is clamped instead of
// branching.
template <typename T, typename I>
__device__ __forceinline__ float load_or_zero(const T *__restrict__ src,
                                              bool cond, I idx, I alt) {
  const float v = (float)src[cond ? idx : alt];
  return cond ? v : 0.0f;
}

// Workgroup -> tile mapping that keeps each XCD on one contiguous range of
// tiles.  The dispatcher hands workgroup t to XCD t % 8; the tiles are cut
// into 8 consecutive groups (sizes differ by at most one) and XCD k walks
// group k in order, so neighbouring tiles share that XCD's L2.
template <typename I>
__device__ __forceinline__ I xcd_tile(I t, I ntiles) {
  constexpr I kXcd = 8;
  const I q = ntiles / kXcd;
  const I rem = ntiles % kXcd;
  const I k = t % kXcd;
  const I slot = t / kXcd;
  return k * q + (k < rem ? k : rem) + slot;
}

}  // namespace tvfgp
