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
// The first pass walks the volume like the default step kernel: 64 x 8 x-y
// tiles marching 4 planes along z, z computed once per point (tile plus its
// upper x column and y row) into a ring of three LDS planes, z(i+e_x) and
// z(i+e_y) read from LDS.  The reduction is deterministic: a fixed number of
// workgroups each sum a fixed set of tiles in a fixed order into one partial
// triple, and a single workgroup adds the partials in a fixed order.
//
// When nx is even and b, p are aligned to two elements, gap_partial_pair_kernel
// does the first pass instead: two x-adjacent voxels per lane, 128 x 8 tiles
// of 24 planes, every load a pair, loads issued two planes ahead.  The
// reduction reads only b and p (16 bytes per voxel), so with one element per
// load and one plane of prefetch a wave has too few bytes in flight to cover
// HBM latency; pairs double them and the deeper prefetch doubles them again.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_device.hpp"
#include "tv_fgp_fused_kernel.hpp"
#include "tv_fgp_pair_kernel.hpp"

#pragma clang fp contract(off)

namespace tvfgp {

constexpr int kGapGrid = 1024;    // partial triples (upper bound)
constexpr int kGapPairGrid = 1024;  // the same for the pair kernel (<= kGapGrid)
// Planes per tile of the pair kernel: a multiple of 2 (load sets) and of 3
// (ring slots).  The prefetch drains at each tile's end, so long tiles pay
// off: at 512^3, 6 / 12 / 24 planes measured 0.58 / 0.50 / 0.47 ms.
constexpr int kGapPairPlanes = 24;
constexpr int kGapFinalBlock = 256;

// Square root of s for s = +0 or a finite s >= 2^-767: the compiler's
// sqrt() sequence (the v_rsq_f64 seed, a Goldschmidt step and two residual
// corrections, +0 passed through) without the rescaling of inputs below
// 2^-767, which is the identity above it; a sum of squares of floats is
// +0 or at least 2^-298.  The bits are those of sqrt().
__device__ __forceinline__ double sqrt_sum_of_squares(double s) {
  const double y = hw_rsq_estimate(s);
  double g = s * y;
  double h = y * 0.5;
  const double r = __builtin_fma(-h, g, 0.5);
  g = __builtin_fma(g, r, g);
  h = __builtin_fma(h, r, h);
  double d = __builtin_fma(-g, g, s);
  g = __builtin_fma(d, h, g);
  d = __builtin_fma(-g, g, s);
  g = __builtin_fma(d, h, g);
  return s == 0.0 ? s : g;
}

// Per-voxel contribution: |g|, |g| - g.p and (z - b)^2, in fp64 (the 1/2 of
// the fidelity term is applied to its total, an exact scaling).  A product
// of two floats is exact in fp64, so each multiply-add below rounds once,
// exactly as a multiply followed by an add: the terms are those of
// (dx dx + dy dy) + dz dz and (dx px + dy py) + dz pz.
__device__ __forceinline__ void gap_terms(float gx, float gy, float gz, float px,
                                          float py, float pz, float z, float b,
                                          double &norm, double &gap,
                                          double &fid) {
  const double dx = (double)gx, dy = (double)gy, dz = (double)gz;
  norm = sqrt_sum_of_squares(__builtin_fma(dz, dz, __builtin_fma(dx, dx, dy * dy)));
  const double dot =
      __builtin_fma(dz, (double)pz, __builtin_fma(dx, (double)px, dy * (double)py));
  gap = norm - dot;
  const double d = (double)z - (double)b;
  fid = d * d;
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

// Pass 1: workgroup w walks tiles w, w + gridDim.x, ... (64 x 8 x 4 voxels
// each) and writes the sum of its voxels' terms to partial[3w .. 3w+2].
template <typename I, typename Off>
__global__ __launch_bounds__(kZxBlock) void gap_partial_kernel(
    const float *__restrict__ b, const float *__restrict__ p0,
    const float *__restrict__ p1, const float *__restrict__ p2, float lam,
    ZxGeometry<I, Off> g, double *__restrict__ partial) {
  constexpr int kW = kZxTileX + 1, kH = kZxTileY + 1;
  __shared__ float zring[3][kH][kW];
  __shared__ double sh[3][kZxBlock];
  const int lx = (int)(threadIdx.x % kZxTileX);
  const int ly = (int)(threadIdx.x / kZxTileX);
  // halo z point: wave 0 the upper y row, lanes 0..7 of wave 1 the upper x column
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
  double s_norm = 0.0, s_gap = 0.0, s_fid = 0.0;

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
    const Off oi = own_ok ? ((Off)x + (Off)g.nx * (Off)y) * four + (Off)z0 * sz4 : 0;
    const Off oh = halo_ok ? ((Off)hx + (Off)g.nx * (Off)hy) * four + (Off)z0 * sz4 : 0;

    // z at plane z0; the own p and b of the column are carried
    float pc0 = 0.0f, pc1 = 0.0f, pc2 = 0.0f, bc = 0.0f, ph2 = 0.0f, zc = 0.0f;
    if (own_ok) {
      pc0 = ld(p0, oi);
      pc1 = ld(p1, oi);
      pc2 = ld(p2, oi);
      bc = ld(b, oi);
      const float a = ld(p0, low_x ? oi - four : oi);
      const float e = ld(p1, low_y ? oi - sy4 : oi);
      const float f = ld(p2, low_z ? oi - sz4 : oi);
      zc = primal_z(bc, pc0, low_x ? a : 0.0f, pc1, low_y ? e : 0.0f, pc2,
                    low_z ? f : 0.0f, lam);
      zring[0][ly][lx] = zc;
    }
    if (halo_ok) {
      ph2 = ld(p2, oh);
      const float a = ld(p0, hlow_x ? oh - four : oh);
      const float e = ld(p1, hlow_y ? oh - sy4 : oh);
      const float f = ld(p2, low_z ? oh - sz4 : oh);
      zring[0][hyl][hxl] = primal_z(ld(b, oh), ld(p0, oh), hlow_x ? a : 0.0f, ld(p1, oh),
                                    hlow_y ? e : 0.0f, ph2, low_z ? f : 0.0f, lam);
    }

    // loads of the next plane (own point and halo point)
    float nb = 0.0f, n0 = 0.0f, n1 = 0.0f, n2 = 0.0f, n0l = 0.0f, n1l = 0.0f;
    float hb = 0.0f, h0 = 0.0f, h1 = 0.0f, h2 = 0.0f, h0l = 0.0f, h1l = 0.0f;
    auto load_plane = [&](I kp) {
      const Off dz = (Off)(kp - z0) * sz4;
      if (own_ok) {
        const Off j = oi + dz;
        nb = ld(b, j);
        n0 = ld(p0, j);
        n1 = ld(p1, j);
        n2 = ld(p2, j);
        n0l = ld(p0, low_x ? j - four : j);
        n1l = ld(p1, low_y ? j - sy4 : j);
      }
      if (halo_ok) {
        const Off j = oh + dz;
        hb = ld(b, j);
        h0 = ld(p0, j);
        h1 = ld(p1, j);
        h2 = ld(p2, j);
        h0l = ld(p0, hlow_x ? j - four : j);
        h1l = ld(p1, hlow_y ? j - sy4 : j);
      }
    };
    if (z0 + 1 < g.nz) load_plane(z0 + 1);

    int cur = 0;
    for (I k = z0; k < z1; ++k) {
      const int nxt = cur == 2 ? 0 : cur + 1;
      const bool has_z = k + 1 < g.nz;
      const float cb = nb, c0 = n0, c1 = n1, c2 = n2, c0l = n0l, c1l = n1l;
      const float db = hb, d0 = h0, d1 = h1, d2 = h2, d0l = h0l, d1l = h1l;
      if (k + 1 < z1 && k + 2 < g.nz) load_plane(k + 2);
      float zz = 0.0f;
      if (has_z) {
        if (own_ok) {
          zz = primal_z(cb, c0, low_x ? c0l : 0.0f, c1, low_y ? c1l : 0.0f, c2, pc2, lam);
          zring[nxt][ly][lx] = zz;
        }
        if (halo_ok) {
          zring[nxt][hyl][hxl] = primal_z(db, d0, hlow_x ? d0l : 0.0f, d1,
                                          hlow_y ? d1l : 0.0f, d2, ph2, lam);
          ph2 = d2;
        }
      }
      // ring of three planes: one barrier per plane (as in the step kernel)
      __syncthreads();
      if (own_ok) {
        const float zx = zring[cur][ly][lx + 1];
        const float zy = zring[cur][ly + 1][lx];
        const float gx = has_x ? zc - zx : 0.0f;
        const float gy = has_y ? zc - zy : 0.0f;
        const float gz = has_z ? zc - zz : 0.0f;
        double n, gp, f;
        gap_terms(gx, gy, gz, pc0, pc1, pc2, zc, bc, n, gp, f);
        s_norm = s_norm + n;
        s_gap = s_gap + gp;
        s_fid = s_fid + f;
      }
      zc = zz;
      bc = cb;
      pc0 = c0;
      pc1 = c1;
      pc2 = c2;
      cur = nxt;
    }
    __syncthreads();  // the next tile rewrites ring slot 0
  }
  block_sum3<kZxBlock>(s_gap, s_norm, s_fid, sh);
  if (threadIdx.x == 0) {
    partial[3 * blockIdx.x + 0] = s_gap;
    partial[3 * blockIdx.x + 1] = s_norm;
    partial[3 * blockIdx.x + 2] = s_fid;
  }
}

// Pass 1 with two x-adjacent voxels per lane (nx even, b and p aligned to
// two elements): workgroup w walks tiles w, w + gridDim.x, ... of 128 x 8 x 24
// voxels.  Per voxel the same fp32 z and g and the same fp64 terms as
// gap_partial_kernel; a lane adds its first voxel's terms, then its second's.
template <typename I, typename Off>
__global__ __launch_bounds__(kPairBlock) void gap_partial_pair_kernel(
    const float *__restrict__ b, const float *__restrict__ p0,
    const float *__restrict__ p1, const float *__restrict__ p2, float lam,
    ZxGeometry<I, Off> g, double *__restrict__ partial) {
  constexpr int kW = kPairTileX + 2, kH = kPairTileY + 1;
  __shared__ __attribute__((aligned(16))) float zring[3][kH][kW];
  __shared__ double sh[3][kPairBlock];
  const int lx = (int)(threadIdx.x % kPairLanes);
  const int ly = (int)(threadIdx.x / kPairLanes);
  // halo pair: wave 0 the upper y row, lanes 0..7 of wave 1 the pair just
  // past the tile's last column
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
  double s_norm = 0.0, s_gap = 0.0, s_fid = 0.0;

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

    // z at plane z0; the own p and b pairs of the column are carried
    f32x2 pc0 = zero2, pc1 = zero2, pc2 = zero2, bc = zero2, ph2 = zero2, zc = zero2;
    if (own_ok) {
      pc0 = ld2(p0, oi);
      pc1 = ld2(p1, oi);
      pc2 = ld2(p2, oi);
      bc = ldb2(b, oi);
      const float a = lds(p0, low_x ? oi - four : oi);
      const f32x2 e = ld2(p1, low_y ? oi - sy4 : oi);
      const f32x2 f = ld2(p2, low_z ? oi - sz4 : oi);
      zc = primal_pair(bc, pc0, low_x ? a : 0.0f, pc1, low_y ? e : zero2, pc2,
                       low_z ? f : zero2, lam);
      *(f32x2 *)&zring[0][ly][2 * lx] = zc;
    }
    if (halo_ok) {
      ph2 = ld2(p2, oh);
      const float a = lds(p0, hlow_x ? oh - four : oh);
      const f32x2 e = ld2(p1, hlow_y ? oh - sy4 : oh);
      const f32x2 f = ld2(p2, low_z ? oh - sz4 : oh);
      *(f32x2 *)&zring[0][hyl][2 * hxl] =
          primal_pair(ldb2(b, oh), ld2(p0, oh), hlow_x ? a : 0.0f, ld2(p1, oh),
                      hlow_y ? e : zero2, ph2, low_z ? f : zero2, lam);
    }

    // Loads of the planes ahead, in two sets used on alternate planes: the
    // plane step that consumes a set refills it with the plane three ahead,
    // so every load has two plane steps to arrive.  The steps are unrolled
    // (ring slot and set are constants) and every refill is unconditional:
    // a plane past the last one the tile reads is replaced by that last
    // plane, and lanes outside the volume read elements of its first column,
    // which they never use.  So the wait for one set never has to cover the
    // other set's loads.
    struct Ahead {
      f32x2 b, p0, p1, p2, p1l, hb, h0, h1, h2, h1l;
      float p0l, h0l;
    };
    Ahead la[2];
    const bool own_lx = own_ok && low_x, own_ly = own_ok && low_y;
    const I last = z1 < g.nz - 1 ? z1 : g.nz - 1;  // last plane the tile reads
    auto load_plane = [&](Ahead &l, I kp) {  // loads of plane min(kp, last)
      const Off dz = (Off)((kp < last ? kp : last) - z0) * sz4;
      if (halo_ok) {
        const Off j = oh + dz;
        l.hb = ldb2(b, j);
        l.h0 = ld2(p0, j);
        l.h1 = ld2(p1, j);
        l.h2 = ld2(p2, j);
        l.h0l = lds(p0, hlow_x ? j - four : j);
        l.h1l = ld2(p1, hlow_y ? j - sy4 : j);
      }
      const Off j = oi + dz;
      l.b = ldb2(b, j);
      l.p0 = ld2(p0, j);
      l.p1 = ld2(p1, j);
      l.p2 = ld2(p2, j);
      l.p0l = lds(p0, own_lx ? j - four : j);
      l.p1l = ld2(p1, own_ly ? j - sy4 : j);
    };
    load_plane(la[0], z0 + 1);
    load_plane(la[1], z0 + 2);

#pragma unroll
    for (int i = 0; i < kGapPairPlanes; ++i) {
      Ahead &l = la[i % 2];  // plane k + 1
      const int cur = i % 3, nxt = (i + 1) % 3;
      const I k = z0 + i;
      const bool in = k < z1;
      const bool has_z = k + 1 < g.nz;
      f32x2 zz = zero2;
      if (in && has_z) {
        if (own_ok) {
          zz = primal_pair(l.b, l.p0, low_x ? l.p0l : 0.0f, l.p1, low_y ? l.p1l : zero2, l.p2,
                           pc2, lam);
          *(f32x2 *)&zring[nxt][ly][2 * lx] = zz;
        }
        if (halo_ok) {
          *(f32x2 *)&zring[nxt][hyl][2 * hxl] =
              primal_pair(l.hb, l.h0, hlow_x ? l.h0l : 0.0f, l.h1, hlow_y ? l.h1l : zero2,
                          l.h2, ph2, lam);
          ph2 = l.h2;
        }
      }
      const f32x2 cb = l.b, c0 = l.p0, c1 = l.p1, c2 = l.p2;
      if (i + 2 < kGapPairPlanes) load_plane(l, k + 3);
      // ring of three planes: one barrier per plane (as in the step kernel)
      __syncthreads();
      if (in && own_ok) {
        const float zx1 = zring[cur][ly][2 * lx + 2];
        const f32x2 zy = *(const f32x2 *)&zring[cur][ly + 1][2 * lx];
        double n, gp, f;
        // first voxel: its upper x neighbour is the pair's second voxel
        gap_terms(zc.x - zc.y, has_y ? zc.x - zy.x : 0.0f, has_z ? zc.x - zz.x : 0.0f,
                  pc0.x, pc1.x, pc2.x, zc.x, bc.x, n, gp, f);
        s_norm = s_norm + n;
        s_gap = s_gap + gp;
        s_fid = s_fid + f;
        gap_terms(has_x2 ? zc.y - zx1 : 0.0f, has_y ? zc.y - zy.y : 0.0f,
                  has_z ? zc.y - zz.y : 0.0f, pc0.y, pc1.y, pc2.y, zc.y, bc.y, n, gp, f);
        s_norm = s_norm + n;
        s_gap = s_gap + gp;
        s_fid = s_fid + f;
      }
      zc = zz;
      bc = cb;
      pc0 = c0;
      pc1 = c1;
      pc2 = c2;
    }
    __syncthreads();  // the next tile rewrites ring slot 0
  }
  block_sum3<kPairBlock>(s_gap, s_norm, s_fid, sh);
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
    out[2] = 0.5 * d;
  }
}

// Number of partial triples (= workgroups of pass 1) for these dimensions:
// gap_grid for gap_partial_kernel, gap_pair_grid (never larger) for the pair
// kernel.
inline int gap_grid(int64_t nx, int64_t ny, int64_t nz) {
  const int64_t tiles = ((nx + kZxTileX - 1) / kZxTileX) * ((ny + kZxTileY - 1) / kZxTileY) *
                        ((nz + kZxPlanes - 1) / kZxPlanes);
  return (int)(tiles < kGapGrid ? tiles : kGapGrid);
}

inline int gap_pair_grid(int64_t nx, int64_t ny, int64_t nz) {
  const int64_t tiles = ((nx + kPairTileX - 1) / kPairTileX) *
                        ((ny + kPairTileY - 1) / kPairTileY) *
                        ((nz + kGapPairPlanes - 1) / kGapPairPlanes);
  return (int)(tiles < kGapPairGrid ? tiles : kGapPairGrid);
}

// Tiles of the pair kernel: pair_geometry with kGapPairPlanes planes per tile.
template <typename I, typename Off>
inline ZxGeometry<I, Off> gap_pair_geometry(int64_t nx, int64_t ny, int64_t nz) {
  ZxGeometry<I, Off> g = pair_geometry<I, Off>(nx, ny, nz);
  g.planes = (I)kGapPairPlanes;
  g.tiles_z = (I)((nz + kGapPairPlanes - 1) / kGapPairPlanes);
  g.ntiles = g.tiles_x * g.tiles_y * g.tiles_z;
  return g;
}

}  // namespace tvfgp
