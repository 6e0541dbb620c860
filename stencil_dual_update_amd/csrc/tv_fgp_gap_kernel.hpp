// Duality-gap reduction for the FGP iteration (gfx950).
//
// For a dual field p, with z = max(b - lambda L(p), 0) (the primal of the
// step's first formula, "TV solver: the FGP step on the GPU", section "What
// one step does") and g = D z (its forward differences, same section), the
// gap between the primal value P(z) = 1/2||z - b||^2 + lambda sum_i |g(i)| and
// the dual value d(p) = 1/2||b||^2 - 1/2||z||^2 equals
//     G = lambda * sum_i ( |g(i)| - g(i).p(i) ),
// because z (z - w) = 0 for z = max(w, 0) and <z, L p> = <D z, p> when the
// upper-face slots of p are zero.  Every term is >= 0 when |p(i)| <= 1, so
// the sum has no cancellation; G -> 0 as the iteration converges.
//
// z and g are computed in fp32 exactly as the step computes them (shared
// primal_z, same boundary rule); the per-voxel terms and all sums are fp64.
// The reduction is deterministic: a fixed number of workgroups each sum a
// fixed set of tiles in a fixed order into one partial triple, and a single
// workgroup adds the partials in a fixed order.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_device.hpp"

#pragma clang fp contract(off)

namespace tvfgp {

constexpr int kGapGrid = 1024;    // partial triples (upper bound)
constexpr int kGapPlanes = 8;     // planes per tile
constexpr int kGapFinalBlock = 256;

// Per-voxel contribution: |g|, |g| - g.p and 1/2 (z - b)^2, in fp64.
__device__ __forceinline__ void gap_terms(float gx, float gy, float gz, float px,
                                          float py, float pz, float z, float b,
                                          double &norm, double &gap,
                                          double &fid) {
  const double dx = (double)gx, dy = (double)gy, dz = (double)gz;
  norm = __builtin_sqrt((dx * dx + dy * dy) + dz * dz);
  const double dot = (dx * (double)px + dy * (double)py) + dz * (double)pz;
  gap = norm - dot;
  const double d = (double)z - (double)b;
  fid = 0.5 * (d * d);
}

// Block-wide sum of three doubles in a fixed order; thread 0 gets the result.
template <int kThreads>
__device__ __forceinline__ void block_sum3(double &a, double &b, double &c,
                                           double (*sh)[kThreads]) {
  const int t = (int)threadIdx.x;
  sh[0][t] = a;
  sh[1][t] = b;
  sh[2][t] = c;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (t < s) {
      sh[0][t] = sh[0][t] + sh[0][t + s];
      sh[1][t] = sh[1][t] + sh[1][t + s];
      sh[2][t] = sh[2][t] + sh[2][t + s];
    }
    __syncthreads();
  }
  a = sh[0][0];
  b = sh[1][0];
  c = sh[2][0];
}

// Pass 1: each workgroup walks tiles t = blockIdx.x, blockIdx.x + gridDim.x,
// ... (64 x 4 x kGapPlanes voxels each); each thread walks its column along
// z, carrying z and p of the plane above.  Writes partial[3*blockIdx.x + k].
template <typename I>
__global__ __launch_bounds__(kBlock) void gap_partial_kernel(
    const float *__restrict__ b, const float *__restrict__ p0,
    const float *__restrict__ p1, const float *__restrict__ p2, float lam,
    Geometry<I> g, double *__restrict__ partial) {
  __shared__ double sh[3][kBlock];
  const I lx = (I)(threadIdx.x % kTileX);
  const I ly = (I)(threadIdx.x / kTileX);
  double s_norm = 0.0, s_gap = 0.0, s_fid = 0.0;
  for (I t = (I)blockIdx.x; t < g.ntiles; t += (I)gridDim.x) {
    const I tx = t % g.tiles_x;
    const I rest = t / g.tiles_x;
    const I ty = rest % g.tiles_y;
    const I tz = rest / g.tiles_y;
    const I x = tx * kTileX + lx;
    const I y = ty * kTileY + ly;
    if (x >= g.nx || y >= g.ny) continue;
    const I z0 = tz * g.planes;
    const I z1 = (z0 + g.planes < g.nz) ? z0 + g.planes : g.nz;
    const bool has_x = x + 1 < g.nx, has_y = y + 1 < g.ny;
    const bool low_x = x > 0, low_y = y > 0;
    const I sy = g.sy, sz = g.sz;
    I i = x + sy * y + sz * z0;
    float pc0 = p0[i], pc1 = p1[i], pc2 = p2[i];
    float bc = b[i];
    float zc = primal_z(bc, pc0, load_or_zero(p0, low_x, i - 1, i), pc1,
                        load_or_zero(p1, low_y, i - sy, i), pc2,
                        load_or_zero(p2, z0 > 0, i - sz, i), lam);
    const I ixs = has_x ? i + 1 : i;
    const I iys = has_y ? i + sy : i;
    float p2x_lo = load_or_zero(p2, z0 > 0, ixs - sz, ixs);
    float p2y_lo = load_or_zero(p2, z0 > 0, iys - sz, iys);
    for (I zp = z0; zp < z1; ++zp, i += sz) {
      const bool has_z = zp + 1 < g.nz;
      const I ix = has_x ? i + 1 : i;
      const float p2x = p2[ix];
      const float zx = primal_z(b[ix], p0[ix], pc0, p1[ix],
                                load_or_zero(p1, low_y, ix - sy, ix), p2x, p2x_lo, lam);
      p2x_lo = p2x;
      const I iy = has_y ? i + sy : i;
      const float p2y = p2[iy];
      const float zy = primal_z(b[iy], p0[iy], load_or_zero(p0, low_x, iy - 1, iy),
                                p1[iy], pc1, p2y, p2y_lo, lam);
      p2y_lo = p2y;
      const I iz = has_z ? i + sz : i;
      const float bz = b[iz], pz0 = p0[iz], pz1 = p1[iz], pz2 = p2[iz];
      const float zz = primal_z(bz, pz0, load_or_zero(p0, low_x, iz - 1, iz), pz1,
                                load_or_zero(p1, low_y, iz - sy, iz), pz2, pc2, lam);
      const float gx = has_x ? zc - zx : 0.0f;
      const float gy = has_y ? zc - zy : 0.0f;
      const float gz = has_z ? zc - zz : 0.0f;
      double n, gp, f;
      gap_terms(gx, gy, gz, pc0, pc1, pc2, zc, bc, n, gp, f);
      s_norm = s_norm + n;
      s_gap = s_gap + gp;
      s_fid = s_fid + f;
      zc = zz;
      bc = bz;
      pc0 = pz0;
      pc1 = pz1;
      pc2 = pz2;
    }
  }
  block_sum3<kBlock>(s_gap, s_norm, s_fid, sh);
  if (threadIdx.x == 0) {
    partial[3 * blockIdx.x + 0] = s_gap;
    partial[3 * blockIdx.x + 1] = s_norm;
    partial[3 * blockIdx.x + 2] = s_fid;
  }
}

// Pass 2: one workgroup adds `count` partial triples in a fixed order.
// out[0] = lambda * sum(|g| - g.p), out[1] = sum |g|, out[2] = 1/2 sum (z-b)^2.
__global__ __launch_bounds__(kGapFinalBlock) void gap_final_kernel(
    const double *__restrict__ partial, int count, double lam,
    double *__restrict__ out) {
  __shared__ double sh[3][kGapFinalBlock];
  double a = 0.0, c = 0.0, d = 0.0;
  for (int k = (int)threadIdx.x; k < count; k += kGapFinalBlock) {
    a = a + partial[3 * k + 0];
    c = c + partial[3 * k + 1];
    d = d + partial[3 * k + 2];
  }
  block_sum3<kGapFinalBlock>(a, c, d, sh);
  if (threadIdx.x == 0) {
    out[0] = lam * a;
    out[1] = c;
    out[2] = d;
  }
}

// Number of partial triples for these dimensions.
inline int gap_grid(int64_t nx, int64_t ny, int64_t nz) {
  const int64_t tiles = ((nx + kTileX - 1) / kTileX) * ((ny + kTileY - 1) / kTileY) *
                        ((nz + kGapPlanes - 1) / kGapPlanes);
  return (int)(tiles < kGapGrid ? tiles : kGapGrid);
}

}  // namespace tvfgp
