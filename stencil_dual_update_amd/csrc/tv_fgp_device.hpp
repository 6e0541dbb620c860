// Device-side building blocks of the FGP step, shared by every kernel variant.
//
// Every variant evaluates the primal z and the dual update through these two
// functions, so all variants produce the same bits.  Expressions follow the
// page "TV solver: the FGP step on the GPU", section "What one step does";
// the evaluation order is fixed here and multiply-add contraction is off.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

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
  float px = qx, py = qy, pz = qz;
  if (s2 > 0x1.000002p+0f) {
    const float nq = __builtin_sqrtf(s2);
    px = qx / nq;
    py = qy / nq;
    pz = qz / nq;
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
