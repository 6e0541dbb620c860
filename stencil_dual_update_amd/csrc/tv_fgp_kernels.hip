// Dispatch of all FGP variants and the launchers of the ablation kernels
// (tv_fgp_ablation_kernels.hpp).  The default kernel is launched from
// tv_fgp_fused.hip, the LDS march from tv_fgp_lds.hip.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_ablation_kernels.hpp"
#include "tv_fgp_launch.hpp"

namespace tvfgp {

namespace {

template <typename I>
int launch_step_t(const StepArgs &a) {
  hipStream_t s = (hipStream_t)a.stream;
  const dim3 block(kBlock);
  switch (a.variant) {
    case kVariantFused:
      return launch_fused_zx(a);
    case kVariantRegMarch: {
      const Geometry<I> g = make_geometry<I>(a.nx, a.ny, a.nz, a.planes);
      fused_march_kernel<I><<<grid_for(g.ntiles), block, 0, s>>>(
          a.b, a.p[0], a.p[1], a.p[2], a.r_in[0], a.r_in[1], a.r_in[2],
          a.r_out[0], a.r_out[1], a.r_out[2], a.lam, a.c, a.m, g);
      break;
    }
    case kVariantPoint: {
      const Geometry<I> g = make_geometry<I>(a.nx, a.ny, a.nz, 1);
      fused_point_kernel<I><<<grid_for(g.ntiles), block, 0, s>>>(
          a.b, a.p[0], a.p[1], a.p[2], a.r_in[0], a.r_in[1], a.r_in[2],
          a.r_out[0], a.r_out[1], a.r_out[2], a.lam, a.c, a.m, g);
      break;
    }
    case kVariantTwoKernel: {
      const Geometry<I> g = make_geometry<I>(a.nx, a.ny, a.nz, a.planes);
      primal_kernel<I><<<grid_for(g.ntiles), block, 0, s>>>(
          a.b, a.r_in[0], a.r_in[1], a.r_in[2], a.z_ws, a.lam, g);
      if (hipGetLastError() != hipSuccess) return kLaunchFailed;
      dual_kernel<I><<<grid_for(g.ntiles), block, 0, s>>>(
          a.z_ws, a.p[0], a.p[1], a.p[2], a.r_in[0], a.r_in[1], a.r_in[2],
          a.r_out[0], a.r_out[1], a.r_out[2], a.c, a.m, g);
      break;
    }
    case kVariantLdsMarch:
      return launch_lds_march(a);
    case kVariantPair:
      return launch_fused_pair(a);
    case kVariantTb2:  // a single step: the fused kernel
    case kVariantTb3:
      return launch_fused_zx(a);
    case kVariantCube:
    case kVariantCube32x8x2:
    case kVariantCube64x8x1:
    case kVariantCube8x8x8:
    case kVariantCube32x4x4:
      return launch_cube(a);
    default:
      return kLaunchFailed;
  }
  return hipGetLastError() == hipSuccess ? 0 : kLaunchFailed;
}

template <typename I>
int launch_primal_t(const PrimalArgs &a) {
  const Geometry<I> g = make_geometry<I>(a.nx, a.ny, a.nz, a.planes);
  primal_kernel<I><<<grid_for(g.ntiles), dim3(kBlock), 0,
                     (hipStream_t)a.stream>>>(a.b, a.p[0], a.p[1], a.p[2],
                                              a.z, a.lam, g);
  return hipGetLastError() == hipSuccess ? 0 : kLaunchFailed;
}

template <typename I>
int launch_primal_h_t(const PrimalArgsH &a) {
  const Geometry<I> g = make_geometry<I>(a.nx, a.ny, a.nz, kDefaultPlanes);
  primal_kernel<I, _Float16><<<grid_for(g.ntiles), dim3(kBlock), 0,
                               (hipStream_t)a.stream>>>(
      a.b, (const _Float16 *)a.p[0], (const _Float16 *)a.p[1],
      (const _Float16 *)a.p[2], a.z, a.lam, g);
  return hipGetLastError() == hipSuccess ? 0 : kLaunchFailed;
}

}  // namespace

int launch_primal_h(const PrimalArgsH &a) {
  return fits_int32(a.nx, a.ny, a.nz) ? launch_primal_h_t<int32_t>(a)
                                      : launch_primal_h_t<int64_t>(a);
}

int launch_step(const StepArgs &a) {
  return fits_int32(a.nx, a.ny, a.nz) ? launch_step_t<int32_t>(a)
                                      : launch_step_t<int64_t>(a);
}

int launch_primal(const PrimalArgs &a) {
  return fits_int32(a.nx, a.ny, a.nz) ? launch_primal_t<int32_t>(a)
                                      : launch_primal_t<int64_t>(a);
}

}  // namespace tvfgp
