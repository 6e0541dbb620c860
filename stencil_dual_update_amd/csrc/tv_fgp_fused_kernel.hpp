// Default FGP kernel for gfx950: one fused pass, x-y tiles marching along z,
// z computed once per point and exchanged through LDS.
//
// The step ("TV solver: the FGP step on the GPU", section "What one step
// does") needs, at voxel i, z at i and at its three upper neighbours, and
// each z needs r at its point and at the three lower neighbours.  The page's
// plain fused kernel recomputes z four times per voxel; on gfx950 that costs
// more instructions and cache traffic than the 52 compulsory bytes per voxel
// can hide.  Here a workgroup owns a 64 x 8 (x, y) tile and walks `planes`
// consecutive z planes:
//   - at plane k it computes z(k+1) once for the tile and its upper x column
//     and upper y row (65 x 9 points) into a ring of three LDS planes, so one
//     barrier per plane suffices;
//   - the voxel's own z(k) and z(k+1), its own r and the r_z below are kept in
//     registers; z(i+e_x) and z(i+e_y) come from LDS;
//   - the b and r loads for plane k+2 are issued before plane k+1 is used, so
//     their latency overlaps the barrier and the dual update;
//   - p and r_out are written (and p read, see below) with non-temporal
//     hints: they are touched once per step, and the hint keeps L2 for the
//     neighbour reuse of r and b;
//   - tiles are ordered x fastest within a group of up to 16 tile columns,
//     then y within a band of rows, then z, then band, then group, and each
//     XCD takes a contiguous range.  Group width x band height is about 64
//     tiles, the number of tiles whose reads fit in one XCD's 4 MB L2, so the
//     tile above in z runs about 64 tiles later on the same XCD and finds the
//     plane it shares with this tile still in L2.  Measured on MI355X this
//     brings the HBM reads to within ~1% of the 7 compulsory volumes at 512^3;
//   - p is read with a streaming hint only when rows start on 128-byte
//     cache-line boundaries: with misaligned rows a streaming load makes the
//     two tiles sharing a line fetch it twice.
// Addresses are 32-bit byte offsets from the volume base (one scalar base and
// one vector offset per load) when every offset fits; otherwise 64-bit.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_device.hpp"

#pragma clang fp contract(off)

namespace tvfgp {

constexpr int kZxTileX = 64;  // one wave64 per tile row
constexpr int kZxTileY = 8;   // rows per tile (8 waves, 512 threads)
constexpr int kZxBlock = kZxTileX * kZxTileY;
constexpr int kZxPlanes = 4;  // z planes per tile
constexpr int kZxGroupMax = 16;  // tile columns per group in the tile order
constexpr int kZxReach = 64;     // tiles whose reads one XCD's L2 holds

template <typename I, typename Off>
struct ZxGeometry {
  I nx, ny, nz;
  Off sy4, sz4;  // byte strides of y and z
  I tiles_x, tiles_y, tiles_z;
  I ntiles;
  I planes;
  I group;  // tile columns per group
  I band;   // tile rows per band
};

template <typename Off>
__device__ __forceinline__ float ld(const float *__restrict__ base, Off off) {
  return *(const float *)((const char *)base + off);
}

template <typename Off>
__device__ __forceinline__ float ld_stream(const float *__restrict__ base,
                                           Off off) {
  return __builtin_nontemporal_load((const float *)((const char *)base + off));
}

template <typename Off>
__device__ __forceinline__ void st_stream(float *__restrict__ base, Off off,
                                          float v) {
  __builtin_nontemporal_store(v, (float *)((char *)base + off));
}

// Loads and stores of the dual volumes, whose element type S is float or
// _Float16.  Offsets are kept in bytes of a float volume (4 per element); a
// volume of S elements is addressed at offset * sizeof(S) / 4.  Values are
// widened to float on load (exact) and rounded to S on store (nearest, ties
// to even).
template <typename S, typename Off>
__device__ __forceinline__ const S *sptr(const S *base, Off off) {
  return (const S *)((const char *)base + off / (Off)(4 / sizeof(S)));
}
template <typename S, typename Off>
__device__ __forceinline__ float lds(const S *__restrict__ base, Off off) {
  return (float)*sptr(base, off);
}
template <typename S, typename Off>
__device__ __forceinline__ float lds_stream(const S *__restrict__ base, Off off) {
  return (float)__builtin_nontemporal_load(sptr(base, off));
}
template <typename S, typename Off>
__device__ __forceinline__ void sts_stream(S *__restrict__ base, Off off, float v) {
  __builtin_nontemporal_store((S)v, (S *)sptr((const S *)base, off));
}

// Tile t (after the XCD mapping) -> (tx, ty, tz).  Order, slowest first:
// group of tile columns, band of tile rows, z, row within the band, column
// within the group.  The last group and the last band may be narrower.
template <typename I, typename Off>
__device__ __forceinline__ void ordered_tile(I t, const ZxGeometry<I, Off> &g,
                                             I &tx, I &ty, I &tz) {
  const I per_group = g.group * g.tiles_y * g.tiles_z;
  const I grp = t / per_group;
  I rem = t % per_group;
  const I x_lo = grp * g.group;
  const I width = (g.tiles_x - x_lo < g.group) ? g.tiles_x - x_lo : g.group;
  const I per_band = width * g.band * g.tiles_z;
  const I bnd = rem / per_band;
  rem = rem % per_band;
  const I y_lo = bnd * g.band;
  const I height = (g.tiles_y - y_lo < g.band) ? g.tiles_y - y_lo : g.band;
  tz = rem / (width * height);
  rem = rem % (width * height);
  ty = y_lo + rem / width;
  tx = x_lo + rem % width;
}

template <typename I, typename Off, bool kStreamP, typename S>
__global__ __launch_bounds__(kZxBlock) void fused_zx_kernel(
    const float *__restrict__ b, S *__restrict__ p0, S *__restrict__ p1,
    S *__restrict__ p2, const S *__restrict__ ri0, const S *__restrict__ ri1,
    const S *__restrict__ ri2, S *__restrict__ ro0, S *__restrict__ ro1,
    S *__restrict__ ro2, float lam, float c,
    float m, ZxGeometry<I, Off> g) {
  constexpr int kW = kZxTileX + 1, kH = kZxTileY + 1;
  __shared__ float zring[3][kH][kW];
  const int lx = (int)(threadIdx.x % kZxTileX);
  const int ly = (int)(threadIdx.x / kZxTileX);
  // The thread's halo point: wave 0 takes the upper y row, lanes 0..7 of
  // wave 1 the upper x column; the other threads have none.
  int hxl = -1, hyl = -1;
  if (ly == 0) {
    hxl = lx;
    hyl = kZxTileY;
  } else if (ly == 1 && lx < kZxTileY) {
    hxl = kZxTileX;
    hyl = lx;
  }
  const Off sy4 = g.sy4, sz4 = g.sz4;
  const Off four = 4;

  for (I t = (I)blockIdx.x; t < g.ntiles; t += (I)gridDim.x) {
    I tx, ty, tz;
    ordered_tile<I, Off>(xcd_tile(t, g.ntiles), g, tx, ty, tz);
    const I x0 = tx * kZxTileX, y0 = ty * kZxTileY;
    const I z0 = tz * g.planes;
    const I z1 = (z0 + g.planes < g.nz) ? z0 + g.planes : g.nz;
    const I x = x0 + lx, y = y0 + ly;
    const I hx = x0 + hxl, hy = y0 + hyl;
    const bool own_ok = x < g.nx && y < g.ny;
    const bool halo_ok = hxl >= 0 && hx < g.nx && hy < g.ny;
    const bool has_x = x + 1 < g.nx, has_y = y + 1 < g.ny;
    const bool low_x = x > 0, low_y = y > 0;
    const bool hlow_x = hx > 0, hlow_y = hy > 0;
    const bool low_z = z0 > 0;
    // byte offsets of the column's first plane (0 for idle threads)
    const Off oi = own_ok ? ((Off)x + (Off)g.nx * (Off)y) * four + (Off)z0 * sz4 : 0;
    const Off oh = halo_ok ? ((Off)hx + (Off)g.nx * (Off)hy) * four + (Off)z0 * sz4 : 0;

    // z at plane z0, and the carried r of the column
    float r0c = 0.0f, r1c = 0.0f, r2c = 0.0f, r2h = 0.0f, zc = 0.0f;
    if (own_ok) {
      r0c = lds(ri0, oi);
      r1c = lds(ri1, oi);
      r2c = lds(ri2, oi);
      const float a = lds(ri0, low_x ? oi - four : oi);
      const float e = lds(ri1, low_y ? oi - sy4 : oi);
      const float f = lds(ri2, low_z ? oi - sz4 : oi);
      zc = primal_z(ld(b, oi), r0c, low_x ? a : 0.0f, r1c, low_y ? e : 0.0f,
                    r2c, low_z ? f : 0.0f, lam);
      zring[0][ly][lx] = zc;
    }
    if (halo_ok) {
      r2h = lds(ri2, oh);
      const float a = lds(ri0, hlow_x ? oh - four : oh);
      const float e = lds(ri1, hlow_y ? oh - sy4 : oh);
      const float f = lds(ri2, low_z ? oh - sz4 : oh);
      zring[0][hyl][hxl] =
          primal_z(ld(b, oh), lds(ri0, oh), hlow_x ? a : 0.0f, lds(ri1, oh),
                   hlow_y ? e : 0.0f, r2h, low_z ? f : 0.0f, lam);
    }

    // registers holding the loads of the next plane (own point and halo)
    float nb = 0.0f, n0 = 0.0f, n1 = 0.0f, n2 = 0.0f, n0l = 0.0f, n1l = 0.0f;
    float hb = 0.0f, h0 = 0.0f, h1 = 0.0f, h2 = 0.0f, h0l = 0.0f, h1l = 0.0f;
    auto load_plane = [&](I kp) {  // loads of plane kp (kp < nz)
      const Off dz = (Off)(kp - z0) * sz4;
      if (own_ok) {
        const Off j = oi + dz;
        nb = ld(b, j);
        n0 = lds(ri0, j);
        n1 = lds(ri1, j);
        n2 = lds(ri2, j);
        n0l = lds(ri0, low_x ? j - four : j);
        n1l = lds(ri1, low_y ? j - sy4 : j);
      }
      if (halo_ok) {
        const Off j = oh + dz;
        hb = ld(b, j);
        h0 = lds(ri0, j);
        h1 = lds(ri1, j);
        h2 = lds(ri2, j);
        h0l = lds(ri0, hlow_x ? j - four : j);
        h1l = lds(ri1, hlow_y ? j - sy4 : j);
      }
    };
    if (z0 + 1 < g.nz) load_plane(z0 + 1);

    int cur = 0;
    for (I k = z0; k < z1; ++k) {
      const int nxt = cur == 2 ? 0 : cur + 1;
      const bool has_z = k + 1 < g.nz;
      const Off ok = oi + (Off)(k - z0) * sz4;
      float pv0 = 0.0f, pv1 = 0.0f, pv2 = 0.0f;
      if (own_ok) {
        pv0 = kStreamP ? lds_stream(p0, ok) : lds(p0, ok);
        pv1 = kStreamP ? lds_stream(p1, ok) : lds(p1, ok);
        pv2 = kStreamP ? lds_stream(p2, ok) : lds(p2, ok);
      }
      // plane k+1 values in hand; start the loads of plane k+2
      const float cb = nb, c0 = n0, c1 = n1, c2 = n2, c0l = n0l, c1l = n1l;
      const float db = hb, d0 = h0, d1 = h1, d2 = h2, d0l = h0l, d1l = h1l;
      if (k + 1 < z1 && k + 2 < g.nz) load_plane(k + 2);

      float zz = 0.0f;
      if (has_z) {
        if (own_ok) {
          zz = primal_z(cb, c0, low_x ? c0l : 0.0f, c1, low_y ? c1l : 0.0f,
                        c2, r2c, lam);
          zring[nxt][ly][lx] = zz;
        }
        if (halo_ok) {
          zring[nxt][hyl][hxl] = primal_z(db, d0, hlow_x ? d0l : 0.0f, d1,
                                          hlow_y ? d1l : 0.0f, d2, r2h, lam);
          r2h = d2;
        }
      }
      // Ring of three planes: the slot written here was last read two planes
      // ago, before the previous barrier, so one barrier per plane is enough.
      __syncthreads();
      if (own_ok) {
        const float zx = zring[cur][ly][lx + 1];
        const float zy = zring[cur][ly + 1][lx];
        float o0, o1, o2;
        dual_update(zc, zx, zy, zz, has_x, has_y, has_z, r0c, r1c, r2c, pv0,
                    pv1, pv2, c, m, o0, o1, o2);
        sts_stream(p0, ok, pv0);
        sts_stream(p1, ok, pv1);
        sts_stream(p2, ok, pv2);
        sts_stream(ro0, ok, o0);
        sts_stream(ro1, ok, o1);
        sts_stream(ro2, ok, o2);
      }
      zc = zz;
      r0c = c0;
      r1c = c1;
      r2c = c2;
      cur = nxt;
    }
    __syncthreads();  // the next tile rewrites ring slot 0
  }
}

template <typename I, typename Off>
inline ZxGeometry<I, Off> zx_geometry(int64_t nx, int64_t ny, int64_t nz) {
  ZxGeometry<I, Off> g;
  g.nx = (I)nx;
  g.ny = (I)ny;
  g.nz = (I)nz;
  g.sy4 = (Off)nx * 4;
  g.sz4 = (Off)nx * (Off)ny * 4;
  g.tiles_x = (I)((nx + kZxTileX - 1) / kZxTileX);
  g.tiles_y = (I)((ny + kZxTileY - 1) / kZxTileY);
  g.planes = (I)kZxPlanes;
  g.tiles_z = (I)((nz + kZxPlanes - 1) / kZxPlanes);
  g.ntiles = g.tiles_x * g.tiles_y * g.tiles_z;
  g.group = g.tiles_x < (I)kZxGroupMax ? g.tiles_x : (I)kZxGroupMax;
  const I band = (I)kZxReach / g.group;
  g.band = band < 1 ? 1 : (band > 16 ? 16 : band);
  return g;
}

// Every byte offset the kernel forms stays below 2^32: the largest is about
// (nx*ny*(nz+1) + one tile of overhang) * 4.
inline bool fits_u32_offsets(int64_t nx, int64_t ny, int64_t nz) {
  const int64_t lim = int64_t(1) << 30;  // 2^32 bytes in floats
  const int64_t px = nx + kZxTileX + 1, py = ny + kZxTileY + 1, pz = nz + 1;
  if (px >= lim || py >= lim || pz >= lim) return false;
  if (px * py >= lim) return false;
  return px * py * pz < lim;
}

}  // namespace tvfgp
