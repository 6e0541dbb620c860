// FGP kernel with two x-adjacent voxels per lane.
//
// Same march as fused_zx_kernel (x-y tiles walking z, z computed once per
// point into a three-plane LDS ring, one barrier per plane, next plane
// prefetched, streaming stores), but each lane owns the voxel pair
// (2l, 2l+1) of its tile row, so a tile is 128 x 8 voxels and every load
// and store moves a pair: 8 bytes per lane for fp32 volumes, 4 bytes for
// binary16 ones.  Per voxel that halves the memory instructions the fused
// kernel issues (nine loads and six stores per pair instead of per voxel),
// which matters most for the binary16 dual, where one element per lane
// leaves each wave's requests too small to keep HBM busy.
//
// Within a pair the x differences need no memory: voxel 2l+1's lower x
// neighbour and voxel 2l's upper x neighbour are the other half of the pair.
// Voxel 2l's lower x neighbour of r (element 2l-1) is one scalar load.
//
// Pairs must be aligned: nx even (so every row and plane starts on an even
// element) and every volume aligned to two of its elements.  The caller
// checks this; other shapes take the one-voxel kernel.
//
// The eight plane steps of a tile are unrolled and every load is issued
// unconditionally, so the prefetched plane stays in flight until the step
// that uses it (a rolled loop rotates the prefetch registers with copies,
// which wait for the loads).  Measured at 512^3: binary16 0.751 -> 0.709
// ms/step, fp32 unchanged (1.29-1.34 vs 1.30).
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_device.hpp"
#include "tv_fgp_fused_kernel.hpp"

#pragma clang fp contract(off)

namespace tvfgp {

constexpr int kPairLanes = 64;                 // pairs per tile row (one wave)
constexpr int kPairTileX = 2 * kPairLanes;     // voxels per tile row
constexpr int kPairTileY = 8;                  // rows per tile (8 waves)
constexpr int kPairBlock = kPairLanes * kPairTileY;
constexpr int kPairPlanes = 8;
constexpr int kPairGroupMax = 8;   // tile columns per group in the tile order
constexpr int kPairReach = 32;     // tiles whose reads one XCD's L2 holds

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <typename S>
struct PairOf;
template <>
struct PairOf<float> {
  typedef f32x2 T;
};
template <>
struct PairOf<_Float16> {
  typedef f16x2 T;
};

// Pair loads and stores.  `off` is the byte offset of the pair's first
// element in a float volume (4 per element), as for the one-voxel kernel.
template <typename Off>
__device__ __forceinline__ f32x2 ldb2(const float *__restrict__ base, Off off) {
  return *(const f32x2 *)((const char *)base + off);
}
template <typename S, typename Off>
__device__ __forceinline__ f32x2 ld2(const S *__restrict__ base, Off off) {
  typedef typename PairOf<S>::T P;
  return __builtin_convertvector(*(const P *)sptr(base, off), f32x2);
}
template <typename S, typename Off>
__device__ __forceinline__ f32x2 ld2_stream(const S *__restrict__ base, Off off) {
  typedef typename PairOf<S>::T P;
  return __builtin_convertvector(__builtin_nontemporal_load((const P *)sptr(base, off)),
                                 f32x2);
}
template <typename S, typename Off>
__device__ __forceinline__ void st2_stream(S *__restrict__ base, Off off, f32x2 v) {
  typedef typename PairOf<S>::T P;
  __builtin_nontemporal_store(__builtin_convertvector(v, P),
                              (P *)sptr((const S *)base, off));
}

// z of a voxel pair from its b, r and lower-neighbour r values.  xl is r_x at
// the element before the pair; yl and zl are the r_y and r_z pairs one row
// and one plane below (each already 0 where that neighbour is outside).
__device__ __forceinline__ f32x2 primal_pair(f32x2 bv, f32x2 r0, float xl, f32x2 r1,
                                             f32x2 yl, f32x2 r2, f32x2 zl, float lam) {
  f32x2 z;
  z.x = primal_z(bv.x, r0.x, xl, r1.x, yl.x, r2.x, zl.x, lam);
  z.y = primal_z(bv.y, r0.y, r0.x, r1.y, yl.y, r2.y, zl.y, lam);
  return z;
}

template <typename I, typename Off, bool kStreamP, typename S>
__global__ __launch_bounds__(kPairBlock) void fused_pair_kernel(
    const float *__restrict__ b, S *__restrict__ p0, S *__restrict__ p1,
    S *__restrict__ p2, const S *__restrict__ ri0, const S *__restrict__ ri1,
    const S *__restrict__ ri2, S *__restrict__ ro0, S *__restrict__ ro1,
    S *__restrict__ ro2, float lam, float c, float m, ZxGeometry<I, Off> g) {
  // The ring holds the tile, its upper y row and the upper x pair column.
  constexpr int kW = kPairTileX + 2, kH = kPairTileY + 1;
  __shared__ __attribute__((aligned(16))) float zring[3][kH][kW];
  const int lx = (int)(threadIdx.x % kPairLanes);
  const int ly = (int)(threadIdx.x / kPairLanes);
  // The thread's halo pair: wave 0 takes the upper y row, lanes 0..7 of
  // wave 1 the pair just past the tile's last column; the others have none.
  int hxl = -1, hyl = -1;
  if (ly == 0) {
    hxl = lx;
    hyl = kPairTileY;
  } else if (ly == 1 && lx < kPairTileY) {
    hxl = kPairLanes;
    hyl = lx;
  }
  const Off sy4 = g.sy4, sz4 = g.sz4;
  const Off four = 4;
  const f32x2 zero2 = {0.0f, 0.0f};

  for (I t = (I)blockIdx.x; t < g.ntiles; t += (I)gridDim.x) {
    I tx, ty, tz;
    ordered_tile<I, Off>(xcd_tile(t, g.ntiles), g, tx, ty, tz);
    const I x0 = tx * kPairTileX, y0 = ty * kPairTileY;
    const I z0 = tz * g.planes;
    const I z1 = (z0 + g.planes < g.nz) ? z0 + g.planes : g.nz;
    // first voxel of the own pair and of the halo pair (nx is even, so the
    // second voxel is inside whenever the first is)
    const I x = x0 + 2 * lx, y = y0 + ly;
    const I hx = x0 + 2 * hxl, hy = y0 + hyl;
    const bool own_ok = x < g.nx && y < g.ny;
    const bool halo_ok = hxl >= 0 && hx < g.nx && hy < g.ny;
    const bool has_x2 = x + 2 < g.nx, has_y = y + 1 < g.ny;
    const bool low_x = x > 0, low_y = y > 0;
    const bool hlow_x = hx > 0, hlow_y = hy > 0;
    const bool low_z = z0 > 0;
    const Off oi = own_ok ? ((Off)x + (Off)g.nx * (Off)y) * four + (Off)z0 * sz4 : 0;
    const Off oh = halo_ok ? ((Off)hx + (Off)g.nx * (Off)hy) * four + (Off)z0 * sz4 : 0;

    // z at plane z0, and the carried r pairs of the column
    f32x2 r0c = zero2, r1c = zero2, r2c = zero2, r2h = zero2, zc = zero2;
    if (own_ok) {
      r0c = ld2(ri0, oi);
      r1c = ld2(ri1, oi);
      r2c = ld2(ri2, oi);
      const float a = lds(ri0, low_x ? oi - four : oi);
      const f32x2 e = ld2(ri1, low_y ? oi - sy4 : oi);
      const f32x2 f = ld2(ri2, low_z ? oi - sz4 : oi);
      zc = primal_pair(ldb2(b, oi), r0c, low_x ? a : 0.0f, r1c, low_y ? e : zero2, r2c,
                       low_z ? f : zero2, lam);
      *(f32x2 *)&zring[0][ly][2 * lx] = zc;
    }
    if (halo_ok) {
      r2h = ld2(ri2, oh);
      const float a = lds(ri0, hlow_x ? oh - four : oh);
      const f32x2 e = ld2(ri1, hlow_y ? oh - sy4 : oh);
      const f32x2 f = ld2(ri2, low_z ? oh - sz4 : oh);
      *(f32x2 *)&zring[0][hyl][2 * hxl] =
          primal_pair(ldb2(b, oh), ld2(ri0, oh), hlow_x ? a : 0.0f, ld2(ri1, oh),
                      hlow_y ? e : zero2, r2h, low_z ? f : zero2, lam);
    }

    // Loads of plane k+1, issued one plane ahead; the plane steps are
    // unrolled and the loads unconditional (a plane past the last one the
    // tile reads is replaced by that plane; threads outside the volume read
    // its first column, never used).
    const I last = z1 < g.nz - 1 ? z1 : g.nz - 1;
    const bool own_lx = own_ok && low_x, own_ly = own_ok && low_y;
    f32x2 nb, n0, n1, n2, n1l;
    f32x2 hb = zero2, h0 = zero2, h1 = zero2, h2 = zero2, h1l = zero2;
    float n0l, h0l = 0.0f;
    auto load_plane = [&](I kp) {
      const Off dz = (Off)((kp < last ? kp : last) - z0) * sz4;
      if (halo_ok) {
        const Off j = oh + dz;
        hb = ldb2(b, j);
        h0 = ld2(ri0, j);
        h1 = ld2(ri1, j);
        h2 = ld2(ri2, j);
        h0l = lds(ri0, hlow_x ? j - four : j);
        h1l = ld2(ri1, hlow_y ? j - sy4 : j);
      }
      const Off j = oi + dz;
      nb = ldb2(b, j);
      n0 = ld2(ri0, j);
      n1 = ld2(ri1, j);
      n2 = ld2(ri2, j);
      n0l = lds(ri0, own_lx ? j - four : j);
      n1l = ld2(ri1, own_ly ? j - sy4 : j);
    };
    load_plane(z0 + 1);

#pragma unroll
    for (int i = 0; i < kPairPlanes; ++i) {
      const I k = z0 + i;
      if (k >= z1) break;
      const int cur = i % 3, nxt = (i + 1) % 3;
      const bool has_z = k + 1 < g.nz;
      const Off ok = oi + (Off)i * sz4;
      const f32x2 pv0 = kStreamP ? ld2_stream(p0, ok) : ld2(p0, ok);
      const f32x2 pv1 = kStreamP ? ld2_stream(p1, ok) : ld2(p1, ok);
      const f32x2 pv2 = kStreamP ? ld2_stream(p2, ok) : ld2(p2, ok);
      const f32x2 cb = nb, c0 = n0, c1 = n1, c2 = n2, c1l = n1l;
      const f32x2 db = hb, d0 = h0, d1 = h1, d2 = h2, d1l = h1l;
      const float c0l = n0l, d0l = h0l;
      if (i + 1 < kPairPlanes) load_plane(k + 2);

      f32x2 zz = zero2;
      if (has_z) {
        if (own_ok) {
          zz = primal_pair(cb, c0, low_x ? c0l : 0.0f, c1, low_y ? c1l : zero2, c2, r2c,
                           lam);
          *(f32x2 *)&zring[nxt][ly][2 * lx] = zz;
        }
        if (halo_ok) {
          *(f32x2 *)&zring[nxt][hyl][2 * hxl] =
              primal_pair(db, d0, hlow_x ? d0l : 0.0f, d1, hlow_y ? d1l : zero2, d2, r2h,
                          lam);
          r2h = d2;
        }
      }
      __syncthreads();
      if (own_ok) {
        const float zx1 = zring[cur][ly][2 * lx + 2];
        const f32x2 zy = *(const f32x2 *)&zring[cur][ly + 1][2 * lx];
        float pa0 = pv0.x, pa1 = pv1.x, pa2 = pv2.x;
        float pb0 = pv0.y, pb1 = pv1.y, pb2 = pv2.y;
        float oa0, oa1, oa2, ob0, ob1, ob2;
        dual_update(zc.x, zc.y, zy.x, zz.x, true, has_y, has_z, r0c.x, r1c.x, r2c.x, pa0,
                    pa1, pa2, c, m, oa0, oa1, oa2);
        dual_update(zc.y, zx1, zy.y, zz.y, has_x2, has_y, has_z, r0c.y, r1c.y, r2c.y, pb0,
                    pb1, pb2, c, m, ob0, ob1, ob2);
        st2_stream(p0, ok, f32x2{pa0, pb0});
        st2_stream(p1, ok, f32x2{pa1, pb1});
        st2_stream(p2, ok, f32x2{pa2, pb2});
        st2_stream(ro0, ok, f32x2{oa0, ob0});
        st2_stream(ro1, ok, f32x2{oa1, ob1});
        st2_stream(ro2, ok, f32x2{oa2, ob2});
      }
      zc = zz;
      r0c = c0;
      r1c = c1;
      r2c = c2;
    }
    __syncthreads();  // the next tile rewrites ring slot 0
  }
}

template <typename I, typename Off>
inline ZxGeometry<I, Off> pair_geometry(int64_t nx, int64_t ny, int64_t nz) {
  ZxGeometry<I, Off> g;
  g.nx = (I)nx;
  g.ny = (I)ny;
  g.nz = (I)nz;
  g.sy4 = (Off)nx * 4;
  g.sz4 = (Off)nx * (Off)ny * 4;
  g.tiles_x = (I)((nx + kPairTileX - 1) / kPairTileX);
  g.tiles_y = (I)((ny + kPairTileY - 1) / kPairTileY);
  g.planes = (I)kPairPlanes;
  g.tiles_z = (I)((nz + kPairPlanes - 1) / kPairPlanes);
  g.ntiles = g.tiles_x * g.tiles_y * g.tiles_z;
  g.group = g.tiles_x < (I)kPairGroupMax ? g.tiles_x : (I)kPairGroupMax;
  const I band = (I)kPairReach / g.group;
  g.band = band < 1 ? 1 : (band > 16 ? 16 : band);
  return g;
}

// Every byte offset the pair kernel forms stays below 2^32.
inline bool pair_fits_u32_offsets(int64_t nx, int64_t ny, int64_t nz) {
  const int64_t lim = int64_t(1) << 30;  // 2^32 bytes in floats
  const int64_t px = nx + kPairTileX + 2, py = ny + kPairTileY + 1, pz = nz + 1;
  if (px >= lim || py >= lim || pz >= lim) return false;
  if (px * py >= lim) return false;
  return px * py * pz < lim;
}

// Shapes and pointers the pair kernel accepts: nx even and every volume
// aligned to two of its elements.
inline bool pair_eligible(int64_t nx, const void *b, const void *const *dual, int n_dual,
                          size_t elem) {
  if (nx % 2 != 0) return false;
  if ((uintptr_t)b % 8 != 0) return false;
  for (int k = 0; k < n_dual; ++k)
    if ((uintptr_t)dual[k] % (2 * elem) != 0) return false;
  return true;
}

}  // namespace tvfgp
