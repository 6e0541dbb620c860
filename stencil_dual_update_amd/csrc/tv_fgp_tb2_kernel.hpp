// Two FGP steps in one pass over HBM (temporal blocking along the z march).
//
// One step ("TV solver: the FGP step on the GPU", section "What one step
// does") makes the new r at a voxel depend on the old r within one voxel of
// it; two steps, within two.  So a workgroup that owns a 64 x 8 (x, y) tile
// and walks a slab of planes along z can run the first step on the tile
// grown by one voxel in x and y, keep that step's p' and r' on chip, and
// run the second step on the tile itself: b, p and r are read once and p,
// r written once per two steps, 52 compulsory bytes per voxel instead of
// 104.  The extra work is arithmetic on the halo (step one on 66 x 10 points,
// its primal on 67 x 11, the second primal on 65 x 9, per 64 x 8 outputs) and
// re-reads of neighbour data and of the planes around each slab; on MI355X
// most of those re-reads miss L2 (about 1.3 x the compulsory bytes in all),
// and the pass still takes 0.59 x the time of two one-step passes at 512^3.
// The dual may be stored as float or as binary16 (S).
//
// Every value is computed by the same device functions in the same order as
// the one-step kernels (primal_z, dual_update), so two launches of those and
// one launch of this give the same bits.
//
// Regions in tile coordinates (x, y), the tile being [0, 64) x [0, 8):
//   R0 = [-1, 65] x [-1, 9]   primal z0 of the input r       67 x 11
//   E1 = [-1, 64] x [-1, 8]   step one (p', r')              66 x 10
//   R1 = [ 0, 64] x [ 0, 8]   primal z1 of r'                65 x 9
// Thread t owns tile point (t % 64, t / 64); threads 0..224 also own one of
// the 225 points of R0 outside the tile.
//
// Iteration k of the z march (k runs from z0 - 4 to z1 - 1 for the slab
// [z0, z1); the first iterations only fill the pipeline):
//   phase 1: z1 at plane k+1 on R1 (from r' of planes k+1 and k);
//            z0 at plane k+3 on R0 (from the loads of plane k+3); then
//            the loads of plane k+4 go into the registers plane k+3 came in
//   barrier
//   phase 2: step two at plane k on the tile -> p_out, r_out;
//            step one at plane k+2 on E1 -> r' into LDS, own p', r' kept
//   barrier
// LDS rings of two planes hold z0, r'_z and z1; r'_x and r'_y need one.
// Each ring slot is rewritten only after the barrier that follows its last
// read.  The input p is read at halo points of neighbouring tiles, so the
// new p goes to a second buffer (p_out must not overlap p_in).
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_device.hpp"
#include "tv_fgp_fused_kernel.hpp"

#pragma clang fp contract(off)

namespace tvfgp {

constexpr int kTbTileX = 64;
constexpr int kTbTileY = 8;
constexpr int kTbBlock = kTbTileX * kTbTileY;
constexpr int kTbPlanes = 32;    // output planes per tile (most; see tb_planes)
constexpr int kTbGroupMax = 16;  // tile columns per group in the tile order
constexpr int kTbReach = 64;     // tiles whose reads one XCD's L2 holds
constexpr int kTbR0X = kTbTileX + 3, kTbR0Y = kTbTileY + 3;
constexpr int kTbE1X = kTbTileX + 2, kTbE1Y = kTbTileY + 2;
constexpr int kTbR1X = kTbTileX + 1, kTbR1Y = kTbTileY + 1;
constexpr int kTbHalo = kTbR0X * kTbR0Y - kTbTileX * kTbTileY;  // 225

// Tile coordinates of the h-th R0 point outside the tile: the rows y = -1, 8
// and 9 (x = -1..65), then the columns x = -1, 64 and 65 (y = 0..7).
__device__ __forceinline__ void tb_halo_point(int h, int &x, int &y) {
  if (h < 3 * kTbR0X) {
    const int row = h / kTbR0X;
    y = row == 0 ? -1 : kTbTileY - 1 + row;
    x = h % kTbR0X - 1;
  } else {
    const int c = h - 3 * kTbR0X;
    const int col = c / kTbTileY;
    y = c % kTbTileY;
    x = col == 0 ? -1 : kTbTileX - 1 + col;
  }
}

// One R0 point of the thread: where it is and the values it carries along z.
template <typename Off>
struct TbPoint {
  int lx, ly;               // tile coordinates
  bool ok;                  // inside the volume (x and y)
  bool e1, r1, own;         // member of E1, R1, the tile
  bool low_x, low_y, has_x, has_y;
  Off o;                    // byte offset of the column at plane 0
  float cb, c0, c1, c2, c0l, c1l;  // inputs of the first primal's next plane
  float nb, n0, n1, n2, n0l, n1l;  // binary16 pipeline: the plane after it
  float q0, q1, q2;                // r of plane k+2
  float bq, bqq;                   // b of planes k+2 and k+1
  float pp0, pp1, pp2;             // p_in of plane k+2
};

template <typename I, typename Off>
__device__ __forceinline__ void tb_init_point(TbPoint<Off> &pt, int lx, int ly, I x0, I y0,
                                              const ZxGeometry<I, Off> &g) {
  pt.lx = lx;
  pt.ly = ly;
  const I gx = x0 + lx, gy = y0 + ly;
  pt.ok = gx >= 0 && gy >= 0 && gx < g.nx && gy < g.ny;
  pt.e1 = lx >= -1 && lx <= kTbTileX && ly >= -1 && ly <= kTbTileY;
  pt.r1 = lx >= 0 && lx <= kTbTileX && ly >= 0 && ly <= kTbTileY;
  pt.own = lx >= 0 && lx < kTbTileX && ly >= 0 && ly < kTbTileY;
  // lower-neighbour flags only on points inside the volume, so that a load
  // at a point outside (clamped to the column offset 0) stays in bounds
  pt.low_x = pt.ok && gx > 0;
  pt.low_y = pt.ok && gy > 0;
  pt.has_x = gx + 1 < g.nx;
  pt.has_y = gy + 1 < g.ny;
  pt.o = pt.ok ? ((Off)gx + (Off)g.nx * (Off)gy) * (Off)4 : (Off)0;
  pt.cb = pt.c0 = pt.c1 = pt.c2 = pt.c0l = pt.c1l = 0.0f;
  pt.nb = pt.n0 = pt.n1 = pt.n2 = pt.n0l = pt.n1l = 0.0f;
  pt.q0 = pt.q1 = pt.q2 = 0.0f;
  pt.bq = pt.bqq = 0.0f;
  pt.pp0 = pt.pp1 = pt.pp2 = 0.0f;
}

// A value as it reads back after a store to an S volume (identity for float;
// for _Float16 the round to nearest, ties to even, widened again exactly).
template <typename S>
__device__ __forceinline__ float as_stored(float v) {
  return (float)(S)v;
}

// Loads of plane kp into the input registers of a point (caller checks
// 0 <= kp < nz).  The z march issues them once the first primal has used the
// previous plane's values, so they stay in flight across the barrier and the
// next plane's other work, and no register with a load in flight is copied.
// A point outside the volume has offset 0 and loads the plane's first voxel,
// which is in bounds; its values are never used.  S is the element type of
// the dual volumes (float, or _Float16: widened exactly).
template <typename S, typename Off>
__device__ __forceinline__ void tb_load(TbPoint<Off> &pt, Off kp_off, Off sy4,
                                        const float *__restrict__ b,
                                        const S *__restrict__ r0,
                                        const S *__restrict__ r1,
                                        const S *__restrict__ r2) {
  const Off four = 4;
  const Off j = pt.o + kp_off;
  pt.cb = ld(b, j);
  pt.c0 = lds(r0, j);
  pt.c1 = lds(r1, j);
  pt.c2 = lds(r2, j);
  pt.c0l = lds(r0, pt.low_x ? j - four : j);
  pt.c1l = lds(r1, pt.low_y ? j - sy4 : j);
}

// The same loads into the "n" registers, and the rotation that makes them
// current at the end of a plane: the two-step kernel's binary16 pipeline,
// which issues the next plane's loads at the top of the plane (measured 7%
// faster there than loading after the first primal, which the fp32
// instantiations do).
template <typename S, typename Off>
__device__ __forceinline__ void tb_load_next(TbPoint<Off> &pt, Off kp_off, Off sy4,
                                             const float *__restrict__ b,
                                             const S *__restrict__ r0,
                                             const S *__restrict__ r1,
                                             const S *__restrict__ r2) {
  const Off four = 4;
  const Off j = pt.o + kp_off;
  pt.nb = ld(b, j);
  pt.n0 = lds(r0, j);
  pt.n1 = lds(r1, j);
  pt.n2 = lds(r2, j);
  pt.n0l = lds(r0, pt.low_x ? j - four : j);
  pt.n1l = lds(r1, pt.low_y ? j - sy4 : j);
}

template <typename Off>
__device__ __forceinline__ void tb_rotate(TbPoint<Off> &pt) {
  pt.bqq = pt.bq;
  pt.bq = pt.cb;
  pt.q0 = pt.c0;
  pt.q1 = pt.c1;
  pt.q2 = pt.c2;
  pt.cb = pt.nb;
  pt.c0 = pt.n0;
  pt.c1 = pt.n1;
  pt.c2 = pt.n2;
  pt.c0l = pt.n0l;
  pt.c1l = pt.n1l;
}

// Six waves per SIMD (three workgroups per CU) measured ~9% faster than the
// five the unconstrained register allocation allows; the 32-bit-offset
// instantiations fit the cap (74 VGPRs) without spilling.
// S: element type of p and r (float, or _Float16 for the binary16 dual, where
// the first step's p' and r' are rounded to binary16 as a stored step's are).
template <typename I, typename Off, typename S>
__global__ __launch_bounds__(kTbBlock, 6) void tb2_kernel(
    const float *__restrict__ b, const S *__restrict__ pi0,
    const S *__restrict__ pi1, const S *__restrict__ pi2,
    S *__restrict__ po0, S *__restrict__ po1, S *__restrict__ po2,
    const S *__restrict__ ri0, const S *__restrict__ ri1,
    const S *__restrict__ ri2, S *__restrict__ ro0, S *__restrict__ ro1,
    S *__restrict__ ro2, float lam, float c, float m1, float m2,
    ZxGeometry<I, Off> g) {
  __shared__ float z0r[2][kTbR0Y][kTbR0X];    // z0 at (x+1, y+1)
  __shared__ float rxs[kTbE1Y][kTbE1X];       // r'_x at (x+1, y+1)
  __shared__ float rys[kTbE1Y][kTbE1X];       // r'_y
  __shared__ float rzs[2][kTbE1Y][kTbE1X];    // r'_z, two planes
  __shared__ float z1r[2][kTbR1Y][kTbR1X];    // z1 at (x, y)
  const int tid = (int)threadIdx.x;
  const bool has_halo = tid < kTbHalo;
  int hlx = 0, hly = 0;
  if (has_halo) tb_halo_point(tid, hlx, hly);
  // With binary16 storage the pass is bound by instruction issue, and the
  // halo waves (0-3) carry more work between barriers than waves 4-7, so
  // they issue first (0.7% at 512^3; with fp32 storage, which leaves issue
  // slots free, it cost 2%).  The branch is on a scalar, so the priority
  // instruction runs in those waves only.
  if (sizeof(S) == 2 && hw_wave_uniform(tid) < kTbHalo) hw_raise_priority();
  const Off sy4 = g.sy4, sz4 = g.sz4;

  for (I t = (I)blockIdx.x; t < g.ntiles; t += (I)gridDim.x) {
    I tx, ty, tz;
    ordered_tile<I, Off>(xcd_tile(t, g.ntiles), g, tx, ty, tz);
    const I x0 = tx * kTbTileX, y0 = ty * kTbTileY;
    const I z0 = tz * g.planes;
    const I z1 = (z0 + g.planes < g.nz) ? z0 + g.planes : g.nz;
    TbPoint<Off> own, hal;
    tb_init_point<I, Off>(own, tid % kTbTileX, tid / kTbTileX, x0, y0, g);
    tb_init_point<I, Off>(hal, hlx, hly, x0, y0, g);
    hal.ok = hal.ok && has_halo;
    // own p', r' of planes k and k+1 (step one at the thread's tile point)
    float pa0 = 0.0f, pa1 = 0.0f, pa2 = 0.0f, ra0 = 0.0f, ra1 = 0.0f, ra2 = 0.0f;
    float pb0 = 0.0f, pb1 = 0.0f, pb2 = 0.0f, rb0 = 0.0f, rb1 = 0.0f, rb2 = 0.0f;

    const I kstart = z0 - 4;
    // planes whose inputs the slab reads: [z0 - 1, z1 + 1] (and r_z of z0 - 2)
    const I lo_in = z0 - 1, hi_in = z1 + 1;
    auto input_plane = [&](I kp) { return kp >= 0 && kp < g.nz && kp >= lo_in && kp <= hi_in; };
    // before iteration kstart: r_z of plane z0 - 2 as the carried lower plane
    // and the inputs of plane z0 - 1 as "current"
    if (z0 - 2 >= 0) {
      const Off j = (Off)(z0 - 2) * sz4;
      own.q2 = lds(ri2, own.o + j);
      if (has_halo) hal.q2 = lds(ri2, hal.o + j);
    }
    if (input_plane(z0 - 1)) {
      tb_load<S, Off>(own, (Off)(z0 - 1) * sz4, sy4, b, ri0, ri1, ri2);
      if (has_halo) tb_load<S, Off>(hal, (Off)(z0 - 1) * sz4, sy4, b, ri0, ri1, ri2);
    }
    // fp32: the next plane's loads go into the registers of the plane the
    // first primal has just used, whose b and r are kept here for step one
    // in the next iteration; binary16: they go into the "n" registers at the
    // top of the plane and rotate in at its end
    constexpr bool kLateLoads = sizeof(S) == 4;
    float ot_b = 0.0f, ot_0 = 0.0f, ot_1 = 0.0f, ot_2 = 0.0f;
    float ht_b = 0.0f, ht_0 = 0.0f, ht_1 = 0.0f, ht_2 = 0.0f;

    for (I k = kstart; k < z1; ++k) {
      const I kd = k + 2;  // step-one plane
      const bool do_d = kd >= z0 - 1 && kd >= 0 && kd < g.nz && kd <= z1;
      const I kb = k + 3;  // z0 plane
      const bool do_b = input_plane(kb);
      const I kf = k + 1;  // z1 plane
      const bool do_f = k >= z0 - 1 && kf >= 0 && kf < g.nz;
      const bool do_h = k >= z0;
      // p_in of the step-one plane
      if (do_d) {
        const Off j = (Off)kd * sz4;
        own.pp0 = lds(pi0, own.o + j);
        own.pp1 = lds(pi1, own.o + j);
        own.pp2 = lds(pi2, own.o + j);
        // p is read at E1 points only: R0 points outside E1 feed the
        // first primal alone
        if (has_halo && hal.e1) {
          hal.pp0 = lds(pi0, hal.o + j);
          hal.pp1 = lds(pi1, hal.o + j);
          hal.pp2 = lds(pi2, hal.o + j);
        }
      }
      const I kl = k + 4;
      if (!kLateLoads && input_plane(kl)) {
        tb_load_next<S, Off>(own, (Off)kl * sz4, sy4, b, ri0, ri1, ri2);
        if (has_halo) tb_load_next<S, Off>(hal, (Off)kl * sz4, sy4, b, ri0, ri1, ri2);
      }

      // ---- phase 1: z1 of plane k+1 on R1, z0 of plane k+3 on R0
      auto phase_f = [&](TbPoint<Off> &pt) {
        const int x = pt.lx + 1, y = pt.ly + 1;
        const int s = (int)(kf & 1), sp = (int)((kf + 1) & 1);
        // every index is inside the arrays (x, y >= 1 on R1), so all reads
        // are unconditional and the boundary rule is a select
        const float rx = rxs[y][x], ry = rys[y][x], rz = rzs[s][y][x];
        const float rxm = rxs[y][x - 1], rym = rys[y - 1][x], rzm = rzs[sp][y][x];
        const float rxl = pt.low_x ? rxm : 0.0f;
        const float ryl = pt.low_y ? rym : 0.0f;
        const float rzl = kf > 0 ? rzm : 0.0f;
        z1r[s][pt.ly][pt.lx] = primal_z(pt.bqq, rx, rxl, ry, ryl, rz, rzl, lam);
      };
      auto phase_b = [&](TbPoint<Off> &pt) {
        z0r[kb & 1][pt.ly + 1][pt.lx + 1] =
            primal_z(pt.cb, pt.c0, pt.low_x ? pt.c0l : 0.0f, pt.c1,
                     pt.low_y ? pt.c1l : 0.0f, pt.c2, kb > 0 ? pt.q2 : 0.0f, lam);
      };
      if (do_f) {
        if (own.ok) phase_f(own);
        if (hal.ok && hal.r1) phase_f(hal);
      }
      if (do_b) {
        if (own.ok) phase_b(own);
        if (hal.ok) phase_b(hal);
      }
      if (kLateLoads) {
        // plane k+3 has been used; its b and r move aside and the loads of
        // plane k+4 take its registers
        ot_b = own.cb;
        ot_0 = own.c0;
        ot_1 = own.c1;
        ot_2 = own.c2;
        ht_b = hal.cb;
        ht_0 = hal.c0;
        ht_1 = hal.c1;
        ht_2 = hal.c2;
        if (input_plane(kl)) {
          tb_load<S, Off>(own, (Off)kl * sz4, sy4, b, ri0, ri1, ri2);
          if (has_halo) tb_load<S, Off>(hal, (Off)kl * sz4, sy4, b, ri0, ri1, ri2);
        }
      }
      __syncthreads();

      // ---- phase 2: step two at plane k (tile), step one at plane k+2 (E1)
      if (do_h && own.ok) {
        const int s = (int)(k & 1), sn = (int)((k + 1) & 1);
        const int x = own.lx, y = own.ly;
        const float zi = z1r[s][y][x], zx = z1r[s][y][x + 1], zy = z1r[s][y + 1][x];
        const float zz = z1r[sn][y][x];
        float o0, o1, o2;
        dual_update(zi, zx, zy, zz, own.has_x, own.has_y, k + 1 < g.nz, ra0, ra1, ra2,
                    pa0, pa1, pa2, c, m2, o0, o1, o2);
        const Off j = own.o + (Off)k * sz4;
        sts_stream(po0, j, pa0);
        sts_stream(po1, j, pa1);
        sts_stream(po2, j, pa2);
        sts_stream(ro0, j, o0);
        sts_stream(ro1, j, o1);
        sts_stream(ro2, j, o2);
      }
      pa0 = pb0;
      pa1 = pb1;
      pa2 = pb2;
      ra0 = rb0;
      ra1 = rb1;
      ra2 = rb2;
      auto phase_d = [&](TbPoint<Off> &pt, float &r0o, float &r1o, float &r2o) {
        const int x = pt.lx + 1, y = pt.ly + 1;
        const int s = (int)(kd & 1), sn = (int)((kd + 1) & 1);
        const float zi = z0r[s][y][x], zx = z0r[s][y][x + 1], zy = z0r[s][y + 1][x];
        const float zz = z0r[sn][y][x];
        dual_update(zi, zx, zy, zz, pt.has_x, pt.has_y, kd + 1 < g.nz, pt.q0, pt.q1, pt.q2,
                    pt.pp0, pt.pp1, pt.pp2, c, m1, r0o, r1o, r2o);
        // the second step sees the first step's p' and r' as stored
        pt.pp0 = as_stored<S>(pt.pp0);
        pt.pp1 = as_stored<S>(pt.pp1);
        pt.pp2 = as_stored<S>(pt.pp2);
        r0o = as_stored<S>(r0o);
        r1o = as_stored<S>(r1o);
        r2o = as_stored<S>(r2o);
        rxs[y][x] = r0o;
        rys[y][x] = r1o;
        rzs[s][y][x] = r2o;
      };
      if (do_d) {
        if (own.ok) {
          phase_d(own, rb0, rb1, rb2);
          pb0 = own.pp0;
          pb1 = own.pp1;
          pb2 = own.pp2;
        }
        if (hal.ok && hal.e1) {
          float h0, h1, h2;
          phase_d(hal, h0, h1, h2);
        }
      }
      __syncthreads();
      if (kLateLoads) {
        // b and r of plane k+3 become those of plane k+2 for the next step
        own.bqq = own.bq;
        own.bq = ot_b;
        own.q0 = ot_0;
        own.q1 = ot_1;
        own.q2 = ot_2;
        hal.bqq = hal.bq;
        hal.bq = ht_b;
        hal.q0 = ht_0;
        hal.q1 = ht_1;
        hal.q2 = ht_2;
      } else {
        tb_rotate(own);
        tb_rotate(hal);
      }
    }
  }
}

// Planes per slab: the largest of 32 and 16 that still gives at least 1536
// tiles (two per workgroup slot of the chip at three workgroups per CU), else
// 8.  A slab re-reads 4 planes and runs 4 pipeline-filling iterations, so
// long slabs pay off on large volumes; small volumes need the tiles to fill
// the chip.  Measured best at 512^3 (32), 256^3 (16) and 128^3 (8).
inline int64_t tb_planes(int64_t nx, int64_t ny, int64_t nz) {
  const int64_t txy = ((nx + kTbTileX - 1) / kTbTileX) * ((ny + kTbTileY - 1) / kTbTileY);
  for (int64_t p = kTbPlanes; p >= 16; p /= 2)
    if (txy * ((nz + p - 1) / p) >= 1536) return p;
  return 8;
}

// planes <= 0: tb_planes()
template <typename I, typename Off>
inline ZxGeometry<I, Off> tb_geometry(int64_t nx, int64_t ny, int64_t nz, int64_t planes = 0) {
  if (planes <= 0) planes = tb_planes(nx, ny, nz);
  ZxGeometry<I, Off> g;
  g.nx = (I)nx;
  g.ny = (I)ny;
  g.nz = (I)nz;
  g.sy4 = (Off)nx * 4;
  g.sz4 = (Off)nx * (Off)ny * 4;
  g.tiles_x = (I)((nx + kTbTileX - 1) / kTbTileX);
  g.tiles_y = (I)((ny + kTbTileY - 1) / kTbTileY);
  g.planes = (I)planes;
  g.tiles_z = (I)((nz + planes - 1) / planes);
  g.ntiles = g.tiles_x * g.tiles_y * g.tiles_z;
  g.group = g.tiles_x < (I)kTbGroupMax ? g.tiles_x : (I)kTbGroupMax;
  const I band = (I)kTbReach / g.group;
  g.band = band < 1 ? 1 : (band > 16 ? 16 : band);
  return g;
}

}  // namespace tvfgp
