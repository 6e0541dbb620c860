// LDS z-marching ablation of the FGP step for gfx950.
//
// The page "TV solver: the FGP step on the GPU" (table "Variants", and
// "What made the difference", with its sweep of marching tile shapes)
// describes x-y tiles that march along z with two planes of r and of z staged
// in shared memory.  Here a TX x TY tile marches along z (`planes` planes per
// tile; the default variant is 64 x 4 with 8 planes, and the shapes of the
// page's sweep, 32 x 4, 32 x 8, 32 x 16, 64 x 4 and 64 x 8, are instantiated
// for tv_fgp_step_march).  At every plane the workgroup stages r of the next
// plane on the tile grown by its lower x column and lower y row ((TX+2) x
// (TY+2) points, 0 outside the volume: the lower-face rule of L), computes z
// of the next plane once per point of the tile plus its upper x column and
// upper y row ((TX+1) x (TY+1) points) from the two staged r planes, and then
// every thread updates its voxel from z(i), z(i+e_x), z(i+e_y) of the current
// plane, z(i+e_z) of the next one and its own r of the current plane.  Three
// barriers per plane.  The arithmetic is the shared primal_z / dual_update
// pair, so the result is bit-identical to the other variants.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_device.hpp"

#pragma clang fp contract(off)

namespace tvfgp {

// Tiles of TX x TY for the marching kernel (planes per tile as given).
template <typename I>
inline Geometry<I> march_geometry(int64_t nx, int64_t ny, int64_t nz, int64_t planes, int tx,
                                  int ty) {
  Geometry<I> g = make_geometry<I>(nx, ny, nz, planes);
  g.tiles_x = (I)((nx + tx - 1) / tx);
  g.tiles_y = (I)((ny + ty - 1) / ty);
  g.ntiles = g.tiles_x * g.tiles_y * g.tiles_z;
  return g;
}

template <typename I, int TX, int TY>
__global__ __launch_bounds__(TX * TY) void lds_march_kernel(
    const float *__restrict__ b, float *__restrict__ p0,
    float *__restrict__ p1, float *__restrict__ p2,
    const float *__restrict__ ri0, const float *__restrict__ ri1,
    const float *__restrict__ ri2, float *__restrict__ ro0,
    float *__restrict__ ro1, float *__restrict__ ro2, float lam, float c,
    float m, Geometry<I> g) {
  constexpr int kB = TX * TY;
  constexpr int kZW = TX + 1;  // tile width plus the upper x column
  constexpr int kZH = TY + 1;  // tile height plus the upper y row
  constexpr int kRW = TX + 2;  // lower x column, tile, upper x column
  constexpr int kRH = TY + 2;  // lower y row, tile, upper y row
  static_assert(kB >= TX + TY, "every halo z point needs a thread");
  // r at tile coordinates (x, y) is rbuf[.][.][y + 1][x + 1], z is zbuf[.][y][x]
  __shared__ float rbuf[2][3][kRH][kRW];
  __shared__ float zbuf[2][kZH][kZW];
  const int tid = (int)threadIdx.x;
  const int lx = tid % TX;
  const int ly = tid / TX;
  // Halo z point of this thread: threads 0..TX-1 take the upper y row,
  // threads TX..TX+TY-1 the upper x column; other threads have none.
  int hxl = -1, hyl = -1;
  if (tid < TX) {
    hxl = tid;
    hyl = TY;
  } else if (tid < TX + TY) {
    hxl = TX;
    hyl = tid - TX;
  }
  const I sy = g.sy, sz = g.sz;

  for (I t = (I)blockIdx.x; t < g.ntiles; t += (I)gridDim.x) {
    const I tile = xcd_tile(t, g.ntiles);
    const I tx = tile % g.tiles_x;
    const I rest = tile / g.tiles_x;
    const I ty = rest % g.tiles_y;
    const I tz = rest / g.tiles_y;
    const I x0 = tx * TX, y0 = ty * TY;
    const I z0 = tz * g.planes;
    const I z1 = (z0 + g.planes < g.nz) ? z0 + g.planes : g.nz;

    const I x = x0 + lx, y = y0 + ly;
    const bool own_ok = x < g.nx && y < g.ny;
    const I hx = x0 + hxl, hy = y0 + hyl;
    const bool halo_ok = hxl >= 0 && hx < g.nx && hy < g.ny;
    const bool has_x = x + 1 < g.nx, has_y = y + 1 < g.ny;

    // r of plane k on the staged region, 0 outside the volume
    auto stage = [&](int slot, I k) {
      for (int s = tid; s < kRW * kRH; s += kB) {
        const int sx = s % kRW, sy2 = s / kRW;
        const I gx = x0 + sx - 1, gy = y0 + sy2 - 1;
        float v0 = 0.0f, v1 = 0.0f, v2 = 0.0f;
        if (gx >= 0 && gy >= 0 && gx < g.nx && gy < g.ny) {
          const I j = gx + sy * gy + sz * k;
          v0 = ri0[j];
          v1 = ri1[j];
          v2 = ri2[j];
        }
        rbuf[slot][0][sy2][sx] = v0;
        rbuf[slot][1][sy2][sx] = v1;
        rbuf[slot][2][sy2][sx] = v2;
      }
    };
    // z of plane k at tile point (zx, zy) from staged r of plane k (slot) and
    // r_z of plane k-1 (rz_lo, already 0 below the lower face)
    auto z_at = [&](int slot, int zx, int zy, float bj, float rz_lo) {
      const int sx = zx + 1, sy2 = zy + 1;
      return primal_z(bj, rbuf[slot][0][sy2][sx], rbuf[slot][0][sy2][sx - 1],
                      rbuf[slot][1][sy2][sx], rbuf[slot][1][sy2 - 1][sx],
                      rbuf[slot][2][sy2][sx], rz_lo, lam);
    };

    I i = own_ok ? x + sy * y + sz * z0 : 0;
    I ih = halo_ok ? hx + sy * hy + sz * z0 : 0;
    int cur = 0;

    // plane z0: stage r, then z (r_z below from memory, 0 below the volume)
    stage(0, z0);
    __syncthreads();
    if (own_ok)
      zbuf[0][ly][lx] = z_at(0, lx, ly, b[i], load_or_zero(ri2, z0 > 0, i - sz, i));
    if (halo_ok)
      zbuf[0][hyl][hxl] = z_at(0, hxl, hyl, b[ih], load_or_zero(ri2, z0 > 0, ih - sz, ih));

    for (I k = z0; k < z1; ++k) {
      const int nxt = cur ^ 1;
      const bool has_z = k + 1 < g.nz;
      // own p before the barriers, so its latency overlaps the staging
      float pv0 = 0.0f, pv1 = 0.0f, pv2 = 0.0f;
      if (own_ok) {
        pv0 = p0[i];
        pv1 = p1[i];
        pv2 = p2[i];
      }
      if (has_z) stage(nxt, k + 1);
      __syncthreads();
      // z of the next plane from the two staged r planes
      if (has_z) {
        if (own_ok)
          zbuf[nxt][ly][lx] = z_at(nxt, lx, ly, b[i + sz], rbuf[cur][2][ly + 1][lx + 1]);
        if (halo_ok)
          zbuf[nxt][hyl][hxl] =
              z_at(nxt, hxl, hyl, b[ih + sz], rbuf[cur][2][hyl + 1][hxl + 1]);
      }
      __syncthreads();
      if (own_ok) {
        const float zc = zbuf[cur][ly][lx];
        const float zx = zbuf[cur][ly][lx + 1];
        const float zy = zbuf[cur][ly + 1][lx];
        const float zz = zbuf[nxt][ly][lx];
        float o0, o1, o2;
        dual_update(zc, zx, zy, zz, has_x, has_y, has_z, rbuf[cur][0][ly + 1][lx + 1],
                    rbuf[cur][1][ly + 1][lx + 1], rbuf[cur][2][ly + 1][lx + 1], pv0, pv1,
                    pv2, c, m, o0, o1, o2);
        p0[i] = pv0;
        p1[i] = pv1;
        p2[i] = pv2;
        ro0[i] = o0;
        ro1[i] = o1;
        ro2[i] = o2;
      }
      // rbuf[cur] and zbuf[cur] are rewritten as the next plane's "next"
      __syncthreads();
      i += own_ok ? sz : 0;
      ih += halo_ok ? sz : 0;
      cur = nxt;
    }
  }
}

}  // namespace tvfgp
