// Ablation: the cube-tiled LDS kernel ("TV solver: the FGP step on the GPU",
// the shared-memory cube variant of the page's "Variants" table, whose cubes
// are 16 x 8 x 4), generalised to any TX x TY x TZ = 512 cube for a sweep of
// tile shapes.
//
// A workgroup owns one cube of voxels.  It stages b, r_x, r_y and r_z of the
// cube grown by one voxel on every side in LDS (0 outside the volume, which
// is the lower-face rule of L), computes z once for the cube and its upper
// x, y and z faces, (TX+1)(TY+1)(TZ+1) points, into LDS, and then runs the
// dual step, projection and momentum for its own voxels from there.  Two
// barriers per cube; the halo is re-read from L2 by the neighbouring cubes.
// Same device functions and operation order as the other kernels, so the
// result is bit-identical.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_device.hpp"

#pragma clang fp contract(off)

namespace tvfgp {

constexpr int kCubeBlock = 512;

template <int TX, int TY, int TZ>
struct CubeShape {
  static_assert(TX * TY * TZ == kCubeBlock, "one thread per voxel of the cube");
  static constexpr int SX = TX + 2, SY = TY + 2, SZ = TZ + 2;  // staged box
  static constexpr int NS = SX * SY * SZ;
  static constexpr int ZX = TX + 1, ZY = TY + 1, ZZ = TZ + 1;  // z points
  static constexpr int NZ = ZX * ZY * ZZ;
};

template <typename I>
struct CubeGeometry {
  I nx, ny, nz;
  I sy, sz;  // element strides of y and z
  I tiles_x, tiles_y, tiles_z;
  I ntiles;
};

template <typename I, int TX, int TY, int TZ>
__global__ __launch_bounds__(kCubeBlock) void cube_kernel(
    const float *__restrict__ b, float *__restrict__ p0, float *__restrict__ p1,
    float *__restrict__ p2, const float *__restrict__ ri0, const float *__restrict__ ri1,
    const float *__restrict__ ri2, float *__restrict__ ro0, float *__restrict__ ro1,
    float *__restrict__ ro2, float lam, float c, float m, CubeGeometry<I> g) {
  typedef CubeShape<TX, TY, TZ> S;
  // staged box: index (x+1) + SX*((y+1) + SY*(z+1)) for cube coordinates x, y, z
  __shared__ float sb[S::NS], s0[S::NS], s1[S::NS], s2[S::NS];
  // z of the cube and its upper faces: index x + ZX*(y + ZY*z)
  __shared__ float zs[S::NZ];
  const int tid = (int)threadIdx.x;
  const int lx = tid % TX, ly = (tid / TX) % TY, lz = tid / (TX * TY);

  for (I t = (I)blockIdx.x; t < g.ntiles; t += (I)gridDim.x) {
    const I tile = xcd_tile(t, g.ntiles);
    const I tx = tile % g.tiles_x;
    const I ty = (tile / g.tiles_x) % g.tiles_y;
    const I tz = tile / (g.tiles_x * g.tiles_y);
    const I x0 = tx * TX, y0 = ty * TY, z0 = tz * TZ;

    // stage b and r on the box [x0-1, x0+TX] x [y0-1, y0+TY] x [z0-1, z0+TZ]
    for (int s = tid; s < S::NS; s += kCubeBlock) {
      const int sx = s % S::SX, sy = (s / S::SX) % S::SY, sz = s / (S::SX * S::SY);
      const I gx = x0 + sx - 1, gy = y0 + sy - 1, gz = z0 + sz - 1;
      float vb = 0.0f, v0 = 0.0f, v1 = 0.0f, v2 = 0.0f;
      if (gx >= 0 && gy >= 0 && gz >= 0 && gx < g.nx && gy < g.ny && gz < g.nz) {
        const I i = gx + g.sy * gy + g.sz * gz;
        vb = b[i];
        v0 = ri0[i];
        v1 = ri1[i];
        v2 = ri2[i];
      }
      sb[s] = vb;
      s0[s] = v0;
      s1[s] = v1;
      s2[s] = v2;
    }
    __syncthreads();

    // z at the cube and its upper faces; points outside the volume are never
    // read (the forward difference there is 0 by the upper-face rule)
    for (int q = tid; q < S::NZ; q += kCubeBlock) {
      const int zx = q % S::ZX, zy = (q / S::ZX) % S::ZY, zz = q / (S::ZX * S::ZY);
      const int s = (zx + 1) + S::SX * ((zy + 1) + S::SY * (zz + 1));
      zs[q] = primal_z(sb[s], s0[s], s0[s - 1], s1[s], s1[s - S::SX], s2[s],
                       s2[s - S::SX * S::SY], lam);
    }
    __syncthreads();

    const I x = x0 + lx, y = y0 + ly, z = z0 + lz;
    if (x < g.nx && y < g.ny && z < g.nz) {
      const int q = lx + S::ZX * (ly + S::ZY * lz);
      const int s = (lx + 1) + S::SX * ((ly + 1) + S::SY * (lz + 1));
      const I i = x + g.sy * y + g.sz * z;
      float pv0 = p0[i], pv1 = p1[i], pv2 = p2[i];
      float o0, o1, o2;
      dual_update(zs[q], zs[q + 1], zs[q + S::ZX], zs[q + S::ZX * S::ZY], x + 1 < g.nx,
                  y + 1 < g.ny, z + 1 < g.nz, s0[s], s1[s], s2[s], pv0, pv1, pv2, c, m, o0,
                  o1, o2);
      p0[i] = pv0;
      p1[i] = pv1;
      p2[i] = pv2;
      ro0[i] = o0;
      ro1[i] = o1;
      ro2[i] = o2;
    }
    __syncthreads();  // the next cube restages the arrays
  }
}

template <typename I, int TX, int TY, int TZ>
inline CubeGeometry<I> cube_geometry(int64_t nx, int64_t ny, int64_t nz) {
  CubeGeometry<I> g;
  g.nx = (I)nx;
  g.ny = (I)ny;
  g.nz = (I)nz;
  g.sy = (I)nx;
  g.sz = (I)(nx * ny);
  g.tiles_x = (I)((nx + TX - 1) / TX);
  g.tiles_y = (I)((ny + TY - 1) / TY);
  g.tiles_z = (I)((nz + TZ - 1) / TZ);
  g.ntiles = g.tiles_x * g.tiles_y * g.tiles_z;
  return g;
}

// Every element index the cube kernel forms fits in int32 (the largest is
// below (nx + 64) * (ny + 64) * (nz + 64)).
inline bool cube_fits_int32(int64_t nx, int64_t ny, int64_t nz) {
  const int64_t lim = (int64_t(1) << 31) - 1;
  const int64_t px = nx + 64, py = ny + 64, pz = nz + 64;
  if (px >= lim || py >= lim || pz >= lim || px * py >= lim) return false;
  return px * py * pz < lim;
}

}  // namespace tvfgp
