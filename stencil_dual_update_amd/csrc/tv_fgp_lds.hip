// Launcher of the LDS z-marching ablation (tv_fgp_lds_kernel.hpp).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_ablation_kernels.hpp"
#include "tv_fgp_launch.hpp"
#include "tv_fgp_lds_kernel.hpp"

namespace tvfgp {

namespace {

template <typename I>
int launch_lds_t(const StepArgs &a) {
  const Geometry<I> g = make_geometry<I>(a.nx, a.ny, a.nz, a.planes);
  lds_march_kernel<I><<<grid_for(g.ntiles), dim3(kBlock), 0,
                        (hipStream_t)a.stream>>>(
      a.b, a.p[0], a.p[1], a.p[2], a.r_in[0], a.r_in[1], a.r_in[2],
      a.r_out[0], a.r_out[1], a.r_out[2], a.lam, a.c, a.m, g);
  return hipGetLastError() == hipSuccess ? 0 : kLaunchFailed;
}

}  // namespace

int launch_lds_march(const StepArgs &a) {
  return fits_int32(a.nx, a.ny, a.nz) ? launch_lds_t<int32_t>(a)
                                      : launch_lds_t<int64_t>(a);
}

}  // namespace tvfgp
