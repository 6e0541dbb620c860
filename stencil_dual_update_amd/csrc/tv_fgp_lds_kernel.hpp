// LDS z-marching ablation of the FGP step for gfx950.
//
// The page "TV solver: the FGP step on the GPU" (table "Variants", and
// "What made the difference") describes x-y tiles that march along z with
// planes staged in shared memory.  Here a 64 x 4 tile marches along z; at
// every plane the workgroup computes z once per point of the tile plus its
// upper x column and upper y row (65 x 5 points, two planes kept in LDS), and
// every thread then reads z(i), z(i+e_x), z(i+e_y) from the current plane and
// z(i+e_z) from the next one.  r is read through the caches; the voxel's own
// r and r_z of the plane below are carried in registers.  The arithmetic is
// the shared primal_z / dual_update pair, so the result is bit-identical to
// the other variants.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_device.hpp"

#pragma clang fp contract(off)

namespace tvfgp {

constexpr int kZW = kTileX + 1;  // tile width plus the upper x column
constexpr int kZH = kTileY + 1;  // tile height plus the upper y row

template <typename I>
__global__ __launch_bounds__(kBlock) void lds_march_kernel(
    const float *__restrict__ b, float *__restrict__ p0,
    float *__restrict__ p1, float *__restrict__ p2,
    const float *__restrict__ ri0, const float *__restrict__ ri1,
    const float *__restrict__ ri2, float *__restrict__ ro0,
    float *__restrict__ ro1, float *__restrict__ ro2, float lam, float c,
    float m, Geometry<I> g) {
  __shared__ float zbuf[2][kZH][kZW];
  const int lx = (int)(threadIdx.x % kTileX);
  const int ly = (int)(threadIdx.x / kTileX);
  // Halo point of this thread: wave 0 takes the upper y row, lanes 0..3 of
  // wave 1 the upper x column; other threads have none.
  int hxl = -1, hyl = -1;
  if (ly == 0) {
    hxl = lx;
    hyl = kTileY;
  } else if (ly == 1 && lx < kTileY) {
    hxl = kTileX;
    hyl = lx;
  }
  const I sy = g.sy, sz = g.sz;

  for (I t = (I)blockIdx.x; t < g.ntiles; t += (I)gridDim.x) {
    const I tile = xcd_tile(t, g.ntiles);
    const I tx = tile % g.tiles_x;
    const I rest = tile / g.tiles_x;
    const I ty = rest % g.tiles_y;
    const I tz = rest / g.tiles_y;
    const I x0 = tx * kTileX, y0 = ty * kTileY;
    const I z0 = tz * g.planes;
    const I z1 = (z0 + g.planes < g.nz) ? z0 + g.planes : g.nz;

    const I x = x0 + lx, y = y0 + ly;
    const bool own_ok = x < g.nx && y < g.ny;
    const I hx = x0 + hxl, hy = y0 + hyl;
    const bool halo_ok = hxl >= 0 && hx < g.nx && hy < g.ny;
    const bool has_x = x + 1 < g.nx, has_y = y + 1 < g.ny;

    I i = own_ok ? x + sy * y + sz * z0 : 0;
    I ih = halo_ok ? hx + sy * hy + sz * z0 : 0;
    float r0c = 0.0f, r1c = 0.0f, r2c = 0.0f, r2h = 0.0f;
    int cur = 0;

    // z at the first plane
    if (own_ok) {
      r0c = ri0[i];
      r1c = ri1[i];
      r2c = ri2[i];
      zbuf[0][ly][lx] = primal_z(b[i], r0c, load_or_zero(ri0, x > 0, i - 1, i),
                                 r1c, load_or_zero(ri1, y > 0, i - sy, i), r2c,
                                 load_or_zero(ri2, z0 > 0, i - sz, i), lam);
    }
    if (halo_ok) {
      r2h = ri2[ih];
      zbuf[0][hyl][hxl] = primal_z(
          b[ih], ri0[ih], load_or_zero(ri0, hx > 0, ih - 1, ih), ri1[ih],
          load_or_zero(ri1, hy > 0, ih - sy, ih), r2h,
          load_or_zero(ri2, z0 > 0, ih - sz, ih), lam);
    }

    for (I k = z0; k < z1; ++k) {
      const int nxt = cur ^ 1;
      const bool has_z = k + 1 < g.nz;
      // own p before the barrier, so its latency overlaps the z exchange
      float pv0 = 0.0f, pv1 = 0.0f, pv2 = 0.0f;
      if (own_ok) {
        pv0 = p0[i];
        pv1 = p1[i];
        pv2 = p2[i];
      }
      // z of the next plane; the own r loaded for it is next plane's own r
      float r0n = 0.0f, r1n = 0.0f, r2n = 0.0f;
      if (has_z) {
        if (own_ok) {
          const I j = i + sz;
          r0n = ri0[j];
          r1n = ri1[j];
          r2n = ri2[j];
          zbuf[nxt][ly][lx] = primal_z(
              b[j], r0n, load_or_zero(ri0, x > 0, j - 1, j), r1n,
              load_or_zero(ri1, y > 0, j - sy, j), r2n, r2c, lam);
        }
        if (halo_ok) {
          const I jh = ih + sz;
          const float r2hn = ri2[jh];
          zbuf[nxt][hyl][hxl] = primal_z(
              b[jh], ri0[jh], load_or_zero(ri0, hx > 0, jh - 1, jh), ri1[jh],
              load_or_zero(ri1, hy > 0, jh - sy, jh), r2hn, r2h, lam);
          r2h = r2hn;
        }
      }
      __syncthreads();
      if (own_ok) {
        const float zc = zbuf[cur][ly][lx];
        const float zx = zbuf[cur][ly][lx + 1];
        const float zy = zbuf[cur][ly + 1][lx];
        const float zz = zbuf[nxt][ly][lx];
        float o0, o1, o2;
        dual_update(zc, zx, zy, zz, has_x, has_y, has_z, r0c, r1c, r2c, pv0,
                    pv1, pv2, c, m, o0, o1, o2);
        p0[i] = pv0;
        p1[i] = pv1;
        p2[i] = pv2;
        ro0[i] = o0;
        ro1[i] = o1;
        ro2[i] = o2;
      }
      // zbuf[cur] is rewritten as the next plane's "next" buffer
      __syncthreads();
      r0c = r0n;
      r1c = r1n;
      r2c = r2n;
      i += own_ok ? sz : 0;
      ih += halo_ok ? sz : 0;
      cur = nxt;
    }
  }
}

}  // namespace tvfgp
