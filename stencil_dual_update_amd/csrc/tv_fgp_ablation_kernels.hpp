// Ablation kernels of the FGP step for gfx950: the register z-march, the
// page's plain fused kernel (one voxel per thread), and the two kernels of
// the two-kernel variant.  Launchers and dispatch are in tv_fgp_kernels.hip.
//
// The step ("TV solver: the FGP step on the GPU", section "What one step
// does") is bound by HBM traffic: per voxel it must read b, r (3) and p (3)
// and write p (3) and r_out (3), 52 bytes, against about 60 flops.  The
// kernels differ only in how they reach the neighbour values; the arithmetic
// is the shared primal_z / dual_update pair, so all variants give the same
// bits.  A workgroup of 256 threads covers a 64 (x) by 4 (y) tile, one wave64
// per row; workgroups are mapped to tiles through xcd_tile.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_device.hpp"

#pragma clang fp contract(off)

namespace tvfgp {

// --------------------------------------------------------------------------
// Ablation: fused pass with a register march along z.
//
// Each thread owns the column (x, y) of a tile for `planes` consecutive z.
// At plane z it needs z(i), z(i+e_x), z(i+e_y), z(i+e_z).  z(i+e_z) computed
// at plane z is z(i) of plane z+1, and the r values loaded for it are the
// thread's own r at plane z+1, so both are carried in registers: per voxel
// three primal evaluations instead of four, and the own r and b are read
// once.  r_z one plane below the +x and +y neighbours is carried as well.
template <typename I>
__global__ __launch_bounds__(kBlock) void fused_march_kernel(
    const float *__restrict__ b, float *__restrict__ p0,
    float *__restrict__ p1, float *__restrict__ p2,
    const float *__restrict__ ri0, const float *__restrict__ ri1,
    const float *__restrict__ ri2, float *__restrict__ ro0,
    float *__restrict__ ro1, float *__restrict__ ro2, float lam, float c,
    float m, Geometry<I> g) {
  const I lx = (I)(threadIdx.x % kTileX);
  const I ly = (I)(threadIdx.x / kTileX);
  for (I t = (I)blockIdx.x; t < g.ntiles; t += (I)gridDim.x) {
    const I tile = xcd_tile(t, g.ntiles);
    const I tx = tile % g.tiles_x;
    const I rest = tile / g.tiles_x;
    const I ty = rest % g.tiles_y;
    const I tz = rest / g.tiles_y;
    const I x = tx * kTileX + lx;
    const I y = ty * kTileY + ly;
    if (x >= g.nx || y >= g.ny) continue;
    const I z0 = tz * g.planes;
    const I z1 = (z0 + g.planes < g.nz) ? z0 + g.planes : g.nz;
    const bool has_x = x + 1 < g.nx;
    const bool has_y = y + 1 < g.ny;
    const bool low_x = x > 0;
    const bool low_y = y > 0;
    const I sy = g.sy, sz = g.sz;

    I i = x + sy * y + sz * z0;
    // z at the first plane of the column, and the r_z below the +x / +y
    // neighbours, which the march carries from then on.
    float r0c = ri0[i];
    float r1c = ri1[i];
    float r2c = ri2[i];
    float zc;
    {
      const float r0l = load_or_zero(ri0, low_x, i - 1, i);
      const float r1l = load_or_zero(ri1, low_y, i - sy, i);
      const float r2l = load_or_zero(ri2, z0 > 0, i - sz, i);
      zc = primal_z(b[i], r0c, r0l, r1c, r1l, r2c, r2l, lam);
    }
    const I ixs = has_x ? i + 1 : i;
    const I iys = has_y ? i + sy : i;
    float r2x_lo = load_or_zero(ri2, z0 > 0, ixs - sz, ixs);
    float r2y_lo = load_or_zero(ri2, z0 > 0, iys - sz, iys);

    for (I zp = z0; zp < z1; ++zp, i += sz) {
      const bool has_z = zp + 1 < g.nz;
      // the voxel's own p first, so its latency overlaps the neighbour reads
      float pv0 = p0[i];
      float pv1 = p1[i];
      float pv2 = p2[i];

      // z(i + e_x)
      const I ix = has_x ? i + 1 : i;
      const float bx = b[ix];
      const float r0x = ri0[ix];
      const float r1x = ri1[ix];
      const float r2x = ri2[ix];
      const float r1x_lo = load_or_zero(ri1, low_y, ix - sy, ix);
      const float zx = primal_z(bx, r0x, r0c, r1x, r1x_lo, r2x, r2x_lo, lam);
      r2x_lo = r2x;

      // z(i + e_y)
      const I iy = has_y ? i + sy : i;
      const float by = b[iy];
      const float r0y = ri0[iy];
      const float r1y = ri1[iy];
      const float r2y = ri2[iy];
      const float r0y_lo = load_or_zero(ri0, low_x, iy - 1, iy);
      const float zy = primal_z(by, r0y, r0y_lo, r1y, r1c, r2y, r2y_lo, lam);
      r2y_lo = r2y;

      // z(i + e_z): also the next plane's own z and r
      const I iz = has_z ? i + sz : i;
      const float bz = b[iz];
      const float r0z = ri0[iz];
      const float r1z = ri1[iz];
      const float r2z = ri2[iz];
      const float r0z_lo = load_or_zero(ri0, low_x, iz - 1, iz);
      const float r1z_lo = load_or_zero(ri1, low_y, iz - sy, iz);
      const float zz = primal_z(bz, r0z, r0z_lo, r1z, r1z_lo, r2z, r2c, lam);

      float o0, o1, o2;
      dual_update(zc, zx, zy, zz, has_x, has_y, has_z, r0c, r1c, r2c, pv0, pv1,
                  pv2, c, m, o0, o1, o2);
      p0[i] = pv0;
      p1[i] = pv1;
      p2[i] = pv2;
      ro0[i] = o0;
      ro1[i] = o1;
      ro2[i] = o2;

      zc = zz;
      r0c = r0z;
      r1c = r1z;
      r2c = r2z;
    }
  }
}

// --------------------------------------------------------------------------
// Ablation: one voxel per thread, z recomputed at the voxel and at its three
// upper neighbours from r at those points and their lower neighbours.
template <typename I>
__global__ __launch_bounds__(kBlock) void fused_point_kernel(
    const float *__restrict__ b, float *__restrict__ p0,
    float *__restrict__ p1, float *__restrict__ p2,
    const float *__restrict__ ri0, const float *__restrict__ ri1,
    const float *__restrict__ ri2, float *__restrict__ ro0,
    float *__restrict__ ro1, float *__restrict__ ro2, float lam, float c,
    float m, Geometry<I> g) {
  const I lx = (I)(threadIdx.x % kTileX);
  const I ly = (I)(threadIdx.x / kTileX);
  for (I t = (I)blockIdx.x; t < g.ntiles; t += (I)gridDim.x) {
    const I tile = xcd_tile(t, g.ntiles);
    const I tx = tile % g.tiles_x;
    const I rest = tile / g.tiles_x;
    const I ty = rest % g.tiles_y;
    const I zp = rest / g.tiles_y;  // planes == 1
    const I x = tx * kTileX + lx;
    const I y = ty * kTileY + ly;
    if (x >= g.nx || y >= g.ny) continue;
    const I sy = g.sy, sz = g.sz;
    const I i = x + sy * y + sz * zp;
    const bool has_x = x + 1 < g.nx, has_y = y + 1 < g.ny, has_z = zp + 1 < g.nz;
    const bool low_x = x > 0, low_y = y > 0, low_z = zp > 0;

    float pv0 = p0[i];
    float pv1 = p1[i];
    float pv2 = p2[i];
    const float r0c = ri0[i];
    const float r1c = ri1[i];
    const float r2c = ri2[i];

    const float zc = primal_z(b[i], r0c, load_or_zero(ri0, low_x, i - 1, i),
                              r1c, load_or_zero(ri1, low_y, i - sy, i), r2c,
                              load_or_zero(ri2, low_z, i - sz, i), lam);
    const I ix = has_x ? i + 1 : i;
    const float zx = primal_z(b[ix], ri0[ix], r0c, ri1[ix],
                              load_or_zero(ri1, low_y, ix - sy, ix), ri2[ix],
                              load_or_zero(ri2, low_z, ix - sz, ix), lam);
    const I iy = has_y ? i + sy : i;
    const float zy = primal_z(b[iy], ri0[iy], load_or_zero(ri0, low_x, iy - 1, iy),
                              ri1[iy], r1c, ri2[iy],
                              load_or_zero(ri2, low_z, iy - sz, iy), lam);
    const I iz = has_z ? i + sz : i;
    const float zz = primal_z(b[iz], ri0[iz], load_or_zero(ri0, low_x, iz - 1, iz),
                              ri1[iz], load_or_zero(ri1, low_y, iz - sy, iz),
                              ri2[iz], r2c, lam);
    float o0, o1, o2;
    dual_update(zc, zx, zy, zz, has_x, has_y, has_z, r0c, r1c, r2c, pv0, pv1,
                pv2, c, m, o0, o1, o2);
    p0[i] = pv0;
    p1[i] = pv1;
    p2[i] = pv2;
    ro0[i] = o0;
    ro1[i] = o1;
    ro2[i] = o2;
  }
}

// --------------------------------------------------------------------------
// Two-kernel ablation, part 1 (also the primal read-out): z = max(b - lam L(r), 0).
// Each thread walks a column along z and carries r_z of the plane below.  S
// is the element type of r (float, or _Float16 for the half-storage dual).
template <typename I, typename S = float>
__global__ __launch_bounds__(kBlock) void primal_kernel(
    const float *__restrict__ b, const S *__restrict__ ri0,
    const S *__restrict__ ri1, const S *__restrict__ ri2,
    float *__restrict__ zout, float lam, Geometry<I> g) {
  const I lx = (I)(threadIdx.x % kTileX);
  const I ly = (I)(threadIdx.x / kTileX);
  for (I t = (I)blockIdx.x; t < g.ntiles; t += (I)gridDim.x) {
    const I tile = xcd_tile(t, g.ntiles);
    const I tx = tile % g.tiles_x;
    const I rest = tile / g.tiles_x;
    const I ty = rest % g.tiles_y;
    const I tz = rest / g.tiles_y;
    const I x = tx * kTileX + lx;
    const I y = ty * kTileY + ly;
    if (x >= g.nx || y >= g.ny) continue;
    const I z0 = tz * g.planes;
    const I z1 = (z0 + g.planes < g.nz) ? z0 + g.planes : g.nz;
    const bool low_x = x > 0, low_y = y > 0;
    const I sy = g.sy, sz = g.sz;
    I i = x + sy * y + sz * z0;
    float r2_lo = load_or_zero(ri2, z0 > 0, i - sz, i);
    for (I zp = z0; zp < z1; ++zp, i += sz) {
      const float r2c = (float)ri2[i];
      zout[i] = primal_z(b[i], (float)ri0[i], load_or_zero(ri0, low_x, i - 1, i),
                         (float)ri1[i], load_or_zero(ri1, low_y, i - sy, i), r2c,
                         r2_lo, lam);
      r2_lo = r2c;
    }
  }
}

// Two-kernel ablation, part 2: the dual update from the materialised z.
template <typename I>
__global__ __launch_bounds__(kBlock) void dual_kernel(
    const float *__restrict__ zv, float *__restrict__ p0,
    float *__restrict__ p1, float *__restrict__ p2,
    const float *__restrict__ ri0, const float *__restrict__ ri1,
    const float *__restrict__ ri2, float *__restrict__ ro0,
    float *__restrict__ ro1, float *__restrict__ ro2, float c, float m,
    Geometry<I> g) {
  const I lx = (I)(threadIdx.x % kTileX);
  const I ly = (I)(threadIdx.x / kTileX);
  for (I t = (I)blockIdx.x; t < g.ntiles; t += (I)gridDim.x) {
    const I tile = xcd_tile(t, g.ntiles);
    const I tx = tile % g.tiles_x;
    const I rest = tile / g.tiles_x;
    const I ty = rest % g.tiles_y;
    const I tz = rest / g.tiles_y;
    const I x = tx * kTileX + lx;
    const I y = ty * kTileY + ly;
    if (x >= g.nx || y >= g.ny) continue;
    const I z0 = tz * g.planes;
    const I z1 = (z0 + g.planes < g.nz) ? z0 + g.planes : g.nz;
    const bool has_x = x + 1 < g.nx, has_y = y + 1 < g.ny;
    const I sy = g.sy, sz = g.sz;
    I i = x + sy * y + sz * z0;
    float zc = zv[i];
    for (I zp = z0; zp < z1; ++zp, i += sz) {
      const bool has_z = zp + 1 < g.nz;
      float pv0 = p0[i];
      float pv1 = p1[i];
      float pv2 = p2[i];
      const float zx = zv[has_x ? i + 1 : i];
      const float zy = zv[has_y ? i + sy : i];
      const float zz = zv[has_z ? i + sz : i];
      float o0, o1, o2;
      dual_update(zc, zx, zy, zz, has_x, has_y, has_z, ri0[i], ri1[i], ri2[i],
                  pv0, pv1, pv2, c, m, o0, o1, o2);
      p0[i] = pv0;
      p1[i] = pv1;
      p2[i] = pv2;
      ro0[i] = o0;
      ro1[i] = o1;
      ro2[i] = o2;
      zc = zz;
    }
  }
}

// True when every index the ablation kernels form fits in int32, including
// one tile of overhang per axis.
inline bool fits_int32(int64_t nx, int64_t ny, int64_t nz) {
  const int64_t px = nx + kTileX, py = ny + kTileY, pz = nz + 1;
  return px * py * pz < (int64_t(1) << 31) - 1;
}

}  // namespace tvfgp
