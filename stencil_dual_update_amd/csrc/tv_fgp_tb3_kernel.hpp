// Three FGP steps in one pass over HBM (temporal blocking along the z march,
// one level deeper than tv_fgp_tb2_kernel.hpp).
//
// One step ("TV solver: the FGP step on the GPU", section "What one step
// does") makes the new r at a voxel depend on the old r within one voxel of
// it, so three steps depend on the old r within three.  A workgroup owns a
// 64 x 8 (x, y) tile and a slab of planes; it runs step one on the tile grown
// by two voxels in x and y, step two on the tile grown by one, step three on
// the tile, keeping the intermediate p and r on chip: b, p and r are read
// once and p, r written once per three steps.  On MI355X at 512^3 a launch
// takes 1.82-1.86 ms, 0.62 ms per step (two steps per pass: 0.75; one:
// 1.30); its HBM traffic is 1.21 x the compulsory bytes, moved at 4.5 TB/s.
// At two workgroups per CU it issues VALU instructions 63% of the time, and
// the unit that hands load data back to the waves spends 68% of the launch
// waiting for lines from the L1 and L2: the pass is bound by the latency of
// its loads at this occupancy, not by bandwidth.  Most of the traffic above
// the compulsory bytes is the y-halo rows: the tiles above and below run on
// the same XCD but drift apart by more planes than its L2 holds.
//
// Every value is computed by the same device functions in the same order as
// the one-step kernels (primal_z, dual_update), so three launches of those and
// one launch of this give the same bits; with binary16 storage the p and r of
// steps one and two are rounded as a stored step rounds them.
//
// Regions in tile coordinates (x, y), the tile being T = [0, 64) x [0, 8):
//   R0 = [-2, 66] x [-2, 10]  primal z0 of the input r     69 x 13
//   E1 = [-2, 65] x [-2,  9]  step one  -> p1, r1          68 x 12
//   R1 = [-1, 65] x [-1,  9]  primal z1 of r1              67 x 11
//   E2 = [-1, 64] x [-1,  8]  step two  -> p2, r2          66 x 10
//   R2 = [ 0, 64] x [ 0,  8]  primal z2 of r2              65 x  9
// Thread t owns tile point (t % 64, t / 64); threads 0..383 (waves 0-5) also
// own one of the 384 points of R0 outside the tile that a step reads (its
// corner (66, 10) is never read), so waves 6 and 7 carry no halo point.
//
// Iteration k of the z march (k from z0 - 7 to z1 - 1 for the slab [z0, z1)):
//   phase 1: z2 at plane k+1 on R2, z1 at plane k+3 on R1, z0 at plane k+5
//            on R0 (from the loads of plane k+5); then the loads of plane
//            k+6 go into the registers plane k+5 came in, so they are in
//            flight through phase 2 and the next phase 1 and no register
//            with a load in flight is ever copied
//   barrier
//   phase 2: step three at plane k on T -> p_out, r_out;
//            step two at plane k+2 on E2 -> r2 into LDS, p2 and r2 kept;
//            step one at plane k+4 on E1 -> r1 into LDS, p1 and r1 kept
//   barrier
// LDS rings of two planes hold z0, z1, z2 and the z components of r1 and r2;
// their x and y components need one plane.  Each slot is rewritten only after
// the barrier that follows its last read.  The input p is read at halo points
// of neighbouring tiles, so the new p goes to a second buffer.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_device.hpp"
#include "tv_fgp_fused_kernel.hpp"
#include "tv_fgp_tb2_kernel.hpp"

#pragma clang fp contract(off)

namespace tvfgp {

constexpr int kT3R0X = kTbTileX + 5, kT3R0Y = kTbTileY + 5;  // 69 x 13
constexpr int kT3E1X = kTbTileX + 4, kT3E1Y = kTbTileY + 4;  // 68 x 12
constexpr int kT3R1X = kTbTileX + 3, kT3R1Y = kTbTileY + 3;  // 67 x 11
constexpr int kT3E2X = kTbTileX + 2, kT3E2Y = kTbTileY + 2;  // 66 x 10
constexpr int kT3R2X = kTbTileX + 1, kT3R2Y = kTbTileY + 1;  // 65 x  9
constexpr int kT3Halo = kT3R0X * kT3R0Y - kTbTileX * kTbTileY - 1;  // 384

// Tile coordinates of the h-th R0 point outside the tile: the rows y = -2,
// -1, 8, 9, 10 (x = -2..66, the last row without x = 66), then the columns
// x = -2, -1, 64, 65, 66 (y = 0..7).
__device__ __forceinline__ void tb3_halo_point(int h, int &x, int &y) {
  if (h < 5 * kT3R0X - 1) {
    const int row = h / kT3R0X;
    y = row < 2 ? row - 2 : kTbTileY + row - 2;
    x = h % kT3R0X - 2;
  } else {
    const int c = h - (5 * kT3R0X - 1);
    const int col = c / kTbTileY;
    y = c % kTbTileY;
    x = col < 2 ? col - 2 : kTbTileX + col - 2;
  }
}

// Six floats carried from one plane step to the next as three 64-bit pairs
// (p0, p1), (p2, r0), (r1, r2): handing a set on is then three 64-bit
// register moves instead of six 32-bit ones.
struct Tb3Six {
  uint64_t a, b, c;
};

__device__ __forceinline__ uint64_t tb3_pair(float lo, float hi) {
  return (uint64_t)__builtin_bit_cast(uint32_t, lo) |
         ((uint64_t)__builtin_bit_cast(uint32_t, hi) << 32);
}
__device__ __forceinline__ float tb3_lo(uint64_t v) { return __builtin_bit_cast(float, (uint32_t)v); }
__device__ __forceinline__ float tb3_hi(uint64_t v) {
  return __builtin_bit_cast(float, (uint32_t)(v >> 32));
}
__device__ __forceinline__ Tb3Six tb3_six(float p0, float p1, float p2, float r0, float r1,
                                         float r2) {
  return Tb3Six{tb3_pair(p0, p1), tb3_pair(p2, r0), tb3_pair(r1, r2)};
}

// Region membership of a point and the state it carries beyond TbPoint.
struct Tb3Extra {
  bool e1, r1, e2, r2;
  float b2, b1;   // b of planes k+2 and k+1
  Tb3Six pr1a;    // step one's p1, r1 of plane k+2
  Tb3Six pr1b;    // ... of plane k+3
};

__device__ __forceinline__ void tb3_init_extra(Tb3Extra &e, int lx, int ly) {
  e.e1 = lx >= -2 && lx <= kTbTileX + 1 && ly >= -2 && ly <= kTbTileY + 1;
  e.r1 = lx >= -1 && lx <= kTbTileX + 1 && ly >= -1 && ly <= kTbTileY + 1;
  e.e2 = lx >= -1 && lx <= kTbTileX && ly >= -1 && ly <= kTbTileY;
  e.r2 = lx >= 0 && lx <= kTbTileX && ly >= 0 && ly <= kTbTileY;
  e.b2 = e.b1 = 0.0f;
  e.pr1a = e.pr1b = Tb3Six{0, 0, 0};
}

// LDS of a workgroup: the rings of the three primals and of the step-one and
// step-two r (z components two planes deep, x and y one plane).
struct Tb3Lds {
  float z0r[2][kT3R0Y][kT3R0X];    // z0 at (x+2, y+2)
  float r1x[kT3E1Y][kT3E1X];       // r1_x at (x+2, y+2)
  float r1y[kT3E1Y][kT3E1X];       // r1_y
  float r1z[2][kT3E1Y][kT3E1X];    // r1_z, two planes
  float z1r[2][kT3R1Y][kT3R1X];    // z1 at (x+1, y+1)
  float r2x[kT3E2Y][kT3E2X];       // r2_x at (x+1, y+1)
  float r2y[kT3E2Y][kT3E2X];       // r2_y
  float r2z[2][kT3E2Y][kT3E2X];    // r2_z, two planes
  float z2r[2][kT3R2Y][kT3R2X];    // z2 at (x, y)
};

// A tile whose R0 lies inside the volume with a voxel to spare on every x
// and y face: every point of it has lower and upper neighbours in x and y,
// so the boundary rules in x and y are the identity there.
template <typename I, typename Off>
__device__ __forceinline__ bool tb3_interior(I x0, I y0, const ZxGeometry<I, Off> &g) {
  return x0 >= 3 && y0 >= 3 && x0 + (kT3R0X - 2) < g.nx && y0 + (kT3R0Y - 2) < g.ny;
}

// The z march of one tile (x0, y0) over the planes [z0, z1).  kInterior:
// the tile passes tb3_interior, so the x and y boundary flags are constant
// true and their selects fold away.
template <bool kInterior, typename I, typename Off, typename S>
__device__ __forceinline__ void tb3_tile(
    Tb3Lds &L, const float *__restrict__ b, const S *__restrict__ pi0,
    const S *__restrict__ pi1, const S *__restrict__ pi2, S *__restrict__ po0,
    S *__restrict__ po1, S *__restrict__ po2, const S *__restrict__ ri0,
    const S *__restrict__ ri1, const S *__restrict__ ri2, S *__restrict__ ro0,
    S *__restrict__ ro1, S *__restrict__ ro2, float lam, float c, float m1, float m2,
    float m3, const ZxGeometry<I, Off> &g, int tid, bool has_halo, int hlx, int hly, I x0,
    I y0, I z0, I z1) {
  const Off sy4 = g.sy4, sz4 = g.sz4;
  TbPoint<Off> own, hal;
  tb_init_point<I, Off>(own, tid % kTbTileX, tid / kTbTileX, x0, y0, g);
  tb_init_point<I, Off>(hal, hlx, hly, x0, y0, g);
  hal.ok = hal.ok && has_halo;
  if constexpr (kInterior) {
    own.ok = true;
    own.low_x = own.low_y = own.has_x = own.has_y = true;
    hal.ok = has_halo;
    hal.low_x = hal.low_y = hal.has_x = hal.has_y = true;
  }
  Tb3Extra ox, hx;
  tb3_init_extra(ox, own.lx, own.ly);
  tb3_init_extra(hx, hal.lx, hal.ly);
  // own p2, r2 of planes k and k+1 (step two at the thread's tile point)
  Tb3Six pra{0, 0, 0}, prb{0, 0, 0};

  const I kstart = z0 - 7;
  // planes whose inputs the slab reads: [z0 - 2, z1 + 2] (and r_z of z0 - 3)
  const I lo_in = z0 - 2, hi_in = z1 + 2;
  auto input_plane = [&](I kp) { return kp >= 0 && kp < g.nz && kp >= lo_in && kp <= hi_in; };
  if (z0 - 3 >= 0) {
    const Off j = (Off)(z0 - 3) * sz4;
    own.q2 = lds(ri2, own.o + j);
    if (has_halo) hal.q2 = lds(ri2, hal.o + j);
  }
  if (input_plane(z0 - 2)) {
    tb_load<S, Off>(own, (Off)(z0 - 2) * sz4, sy4, b, ri0, ri1, ri2);
    if (has_halo) tb_load<S, Off>(hal, (Off)(z0 - 2) * sz4, sy4, b, ri0, ri1, ri2);
  }
  // b and r of plane k+5, kept after the loads of plane k+6 replace them
  float ot_b = 0.0f, ot_0 = 0.0f, ot_1 = 0.0f, ot_2 = 0.0f;
  float ht_b = 0.0f, ht_0 = 0.0f, ht_1 = 0.0f, ht_2 = 0.0f;

  for (I k = kstart; k < z1; ++k) {
    const I kd1 = k + 4;  // step-one plane
    const bool do_d1 = kd1 >= z0 - 2 && kd1 >= 0 && kd1 < g.nz && kd1 <= z1 + 1;
    const I kd2 = k + 2;  // step-two plane
    const bool do_d2 = kd2 >= z0 - 1 && kd2 >= 0 && kd2 < g.nz && kd2 <= z1;
    const I kb = k + 5;   // z0 plane
    const bool do_b = input_plane(kb);
    const I kf1 = k + 3;  // z1 plane
    const bool do_f1 = kf1 >= z0 - 1 && kf1 >= 0 && kf1 < g.nz && kf1 <= z1 + 1;
    const I kf2 = k + 1;  // z2 plane
    const bool do_f2 = kf2 >= z0 && kf2 < g.nz && kf2 <= z1;
    const bool do_h = k >= z0;
    // p_in of the step-one plane
    if (do_d1) {
      const Off j = (Off)kd1 * sz4;
      own.pp0 = lds(pi0, own.o + j);
      own.pp1 = lds(pi1, own.o + j);
      own.pp2 = lds(pi2, own.o + j);
      // p is read at E1 points only: R0 points outside E1 feed the first
      // primal alone
      if (has_halo && hx.e1) {
        hal.pp0 = lds(pi0, hal.o + j);
        hal.pp1 = lds(pi1, hal.o + j);
        hal.pp2 = lds(pi2, hal.o + j);
      }
    }
    const I kl = k + 6;

    // ---- phase 1: z2 of plane k+1 on R2, z1 of plane k+3 on R1, z0 of
    // plane k+5 on R0.  Every index is inside its array (the lower
    // neighbours of R2 lie in E2, those of R1 in E1), so the reads are
    // unconditional and the boundary rule is a select.
    auto phase_f2 = [&](TbPoint<Off> &pt, const Tb3Extra &e) {
      const int x = pt.lx + 1, y = pt.ly + 1;
      const int s = (int)(kf2 & 1), sp = (int)((kf2 + 1) & 1);
      const float rx = L.r2x[y][x], ry = L.r2y[y][x], rz = L.r2z[s][y][x];
      const float rxm = L.r2x[y][x - 1], rym = L.r2y[y - 1][x], rzm = L.r2z[sp][y][x];
      L.z2r[s][pt.ly][pt.lx] = primal_z(e.b1, rx, pt.low_x ? rxm : 0.0f, ry,
                                        pt.low_y ? rym : 0.0f, rz, kf2 > 0 ? rzm : 0.0f, lam);
    };
    auto phase_f1 = [&](TbPoint<Off> &pt) {
      const int x = pt.lx + 2, y = pt.ly + 2;
      const int s = (int)(kf1 & 1), sp = (int)((kf1 + 1) & 1);
      const float rx = L.r1x[y][x], ry = L.r1y[y][x], rz = L.r1z[s][y][x];
      const float rxm = L.r1x[y][x - 1], rym = L.r1y[y - 1][x], rzm = L.r1z[sp][y][x];
      L.z1r[s][pt.ly + 1][pt.lx + 1] =
          primal_z(pt.bqq, rx, pt.low_x ? rxm : 0.0f, ry, pt.low_y ? rym : 0.0f, rz,
                   kf1 > 0 ? rzm : 0.0f, lam);
    };
    auto phase_b = [&](TbPoint<Off> &pt) {
      L.z0r[kb & 1][pt.ly + 2][pt.lx + 2] =
          primal_z(pt.cb, pt.c0, pt.low_x ? pt.c0l : 0.0f, pt.c1,
                   pt.low_y ? pt.c1l : 0.0f, pt.c2, kb > 0 ? pt.q2 : 0.0f, lam);
    };
    if (do_f2) {
      if (own.ok) phase_f2(own, ox);
      if (hal.ok && hx.r2) phase_f2(hal, hx);
    }
    if (do_f1) {
      if (own.ok) phase_f1(own);
      if (hal.ok && hx.r1) phase_f1(hal);
    }
    if (do_b) {
      if (own.ok) phase_b(own);
      if (hal.ok) phase_b(hal);
    }
    // plane k+5's b and r are still needed (step one next iteration); the
    // registers take the loads of plane k+6
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
    __syncthreads();

    // ---- phase 2: step three at plane k (tile), step two at plane k+2
    // (E2), step one at plane k+4 (E1)
    if (do_h && own.ok) {
      const int s = (int)(k & 1), sn = (int)((k + 1) & 1);
      const int x = own.lx, y = own.ly;
      const float zi = L.z2r[s][y][x], zx = L.z2r[s][y][x + 1], zy = L.z2r[s][y + 1][x];
      const float zz = L.z2r[sn][y][x];
      float o0, o1, o2;
      float pa0 = tb3_lo(pra.a), pa1 = tb3_hi(pra.a), pa2 = tb3_lo(pra.b);
      dual_update(zi, zx, zy, zz, own.has_x, own.has_y, k + 1 < g.nz, tb3_hi(pra.b),
                  tb3_lo(pra.c), tb3_hi(pra.c), pa0, pa1, pa2, c, m3, o0, o1, o2);
      const Off j = own.o + (Off)k * sz4;
      sts_stream(po0, j, pa0);
      sts_stream(po1, j, pa1);
      sts_stream(po2, j, pa2);
      sts_stream(ro0, j, o0);
      sts_stream(ro1, j, o1);
      sts_stream(ro2, j, o2);
    }
    pra = prb;
    // step two at an E2 point from its step-one p1, r1 of plane k+2
    auto phase_d2 = [&](TbPoint<Off> &pt, Tb3Extra &e, Tb3Six &out) {
      const int x = pt.lx + 1, y = pt.ly + 1;
      const int s = (int)(kd2 & 1), sn = (int)((kd2 + 1) & 1);
      const float zi = L.z1r[s][y][x], zx = L.z1r[s][y][x + 1], zy = L.z1r[s][y + 1][x];
      const float zz = L.z1r[sn][y][x];
      float p0o = tb3_lo(e.pr1a.a), p1o = tb3_hi(e.pr1a.a), p2o = tb3_lo(e.pr1a.b);
      float r0o, r1o, r2o;
      dual_update(zi, zx, zy, zz, pt.has_x, pt.has_y, kd2 + 1 < g.nz, tb3_hi(e.pr1a.b),
                  tb3_lo(e.pr1a.c), tb3_hi(e.pr1a.c), p0o, p1o, p2o, c, m2, r0o, r1o, r2o);
      p0o = as_stored<S>(p0o);
      p1o = as_stored<S>(p1o);
      p2o = as_stored<S>(p2o);
      r0o = as_stored<S>(r0o);
      r1o = as_stored<S>(r1o);
      r2o = as_stored<S>(r2o);
      L.r2x[y][x] = r0o;
      L.r2y[y][x] = r1o;
      L.r2z[s][y][x] = r2o;
      out = tb3_six(p0o, p1o, p2o, r0o, r1o, r2o);
    };
    if (do_d2) {
      if (own.ok) phase_d2(own, ox, prb);
      if (hal.ok && hx.e2) {
        Tb3Six unused;
        phase_d2(hal, hx, unused);
      }
    }
    ox.pr1a = ox.pr1b;
    hx.pr1a = hx.pr1b;
    // step one at an E1 point from the input r and p of plane k+4
    auto phase_d1 = [&](TbPoint<Off> &pt, Tb3Extra &e) {
      const int x = pt.lx + 2, y = pt.ly + 2;
      const int s = (int)(kd1 & 1), sn = (int)((kd1 + 1) & 1);
      const float zi = L.z0r[s][y][x], zx = L.z0r[s][y][x + 1], zy = L.z0r[s][y + 1][x];
      const float zz = L.z0r[sn][y][x];
      float r0o, r1o, r2o;
      dual_update(zi, zx, zy, zz, pt.has_x, pt.has_y, kd1 + 1 < g.nz, pt.q0, pt.q1, pt.q2,
                  pt.pp0, pt.pp1, pt.pp2, c, m1, r0o, r1o, r2o);
      r0o = as_stored<S>(r0o);
      r1o = as_stored<S>(r1o);
      r2o = as_stored<S>(r2o);
      e.pr1b = tb3_six(as_stored<S>(pt.pp0), as_stored<S>(pt.pp1), as_stored<S>(pt.pp2), r0o,
                       r1o, r2o);
      L.r1x[y][x] = r0o;
      L.r1y[y][x] = r1o;
      L.r1z[s][y][x] = r2o;
    };
    if (do_d1) {
      if (own.ok) phase_d1(own, ox);
      if (hal.ok && hx.e1) phase_d1(hal, hx);
    }
    __syncthreads();
    ox.b1 = ox.b2;
    ox.b2 = own.bqq;
    hx.b1 = hx.b2;
    hx.b2 = hal.bqq;
    // b and r of plane k+5 move down a plane; the loads of plane k+6 are
    // already in place, so no register with a load in flight is copied
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
  }
}

// Four waves per SIMD (two workgroups per CU): the carried state of three
// levels takes 125 VGPRs; capping at six waves spilled 53 and ran 2.8x slower.
template <typename I, typename Off, typename S>
__global__ __launch_bounds__(kTbBlock, 4) void tb3_kernel(
    const float *__restrict__ b, const S *__restrict__ pi0,
    const S *__restrict__ pi1, const S *__restrict__ pi2,
    S *__restrict__ po0, S *__restrict__ po1, S *__restrict__ po2,
    const S *__restrict__ ri0, const S *__restrict__ ri1,
    const S *__restrict__ ri2, S *__restrict__ ro0, S *__restrict__ ro1,
    S *__restrict__ ro2, float lam, float c, float m1, float m2, float m3,
    ZxGeometry<I, Off> g) {
  __shared__ Tb3Lds L;
  const int tid = (int)threadIdx.x;
  const bool has_halo = tid < kT3Halo;
  int hlx = 0, hly = 0;
  if (has_halo) tb3_halo_point(tid, hlx, hly);
  // The halo waves (0-5) carry more work between barriers than waves 6 and
  // 7, so they issue first (1% at 512^3).  The branch is on a scalar, so the
  // priority instruction runs in those waves only.
  if (hw_wave_uniform(tid) < kT3Halo) hw_raise_priority();

  for (I t = (I)blockIdx.x; t < g.ntiles; t += (I)gridDim.x) {
    I tx, ty, tz;
    ordered_tile<I, Off>(xcd_tile(t, g.ntiles), g, tx, ty, tz);
    const I x0 = tx * kTbTileX, y0 = ty * kTbTileY;
    const I z0 = tz * g.planes;
    const I z1 = (z0 + g.planes < g.nz) ? z0 + g.planes : g.nz;
    if (tb3_interior<I, Off>(x0, y0, g))
      tb3_tile<true, I, Off, S>(L, b, pi0, pi1, pi2, po0, po1, po2, ri0, ri1, ri2, ro0, ro1,
                                ro2, lam, c, m1, m2, m3, g, tid, has_halo, hlx, hly, x0, y0,
                                z0, z1);
    else
      tb3_tile<false, I, Off, S>(L, b, pi0, pi1, pi2, po0, po1, po2, ri0, ri1, ri2, ro0, ro1,
                                 ro2, lam, c, m1, m2, m3, g, tid, has_halo, hlx, hly, x0, y0,
                                 z0, z1);
  }
}

// Planes per slab, of 96, 64, 32, 16 and 8: the one with the least estimated
// pass time (the longer on a tie).  A workgroup slot runs its tiles one after
// another, a tile taking its planes + 7 plane steps (seven fill the pipeline).
// When one slab layer's tiles fill the `slots` resident workgroups, the
// layers run one after another and the pass takes about the sum over layers
// of ceil(tiles per layer / slots) x (layer planes + 7); otherwise several
// layers run side by side and it takes about ceil(tiles / slots) x (slab
// planes + 7).  Long slabs re-read fewer planes and fill the pipeline less
// often; short ones fill the chip when a layer has few tiles.  Measured per
// three-step launch against the rule it replaced (the longest slab giving at
// least 1024 tiles): 256^3 0.26 against 0.29 ms (64 against 32 planes),
// 320^3 0.49 against 0.55 (64 against 32), 384^3 0.88 against 0.94 (32
// against 96), 512 x 512 x 70 0.27 against 0.30 (one 70-plane slab against
// 64 + 6); 448^3, 512^3 and 1000 x 777 x 301 keep 96 planes.
inline int64_t tb3_planes(int64_t nx, int64_t ny, int64_t nz, int64_t slots = 512) {
  const int64_t txy = ((nx + kTbTileX - 1) / kTbTileX) * ((ny + kTbTileY - 1) / kTbTileY);
  const int64_t choices[5] = {96, 64, 32, 16, 8};
  int64_t best = 8, best_t = -1;
  for (int i = 0; i < 5; ++i) {
    const int64_t c = choices[i];
    const int64_t layers = (nz + c - 1) / c;
    int64_t t;
    if (txy >= slots) {
      const int64_t last = nz - (layers - 1) * c;
      t = ((txy + slots - 1) / slots) * ((layers - 1) * (c + 7) + last + 7);
    } else {
      t = ((txy * layers + slots - 1) / slots) * ((c < nz ? c : nz) + 7);
    }
    if (best_t < 0 || t < best_t) {
      best_t = t;
      best = c;
    }
  }
  return best;
}

}  // namespace tvfgp
