// Launcher of the two-steps-per-pass FGP kernel (tv_fgp_tb2_kernel.hpp).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_launch.hpp"
#include "tv_fgp_tb2_kernel.hpp"

namespace tvfgp {

namespace {

template <typename I, typename Off>
int launch_tb2_t(const Step2Args &a) {
  const ZxGeometry<I, Off> g = tb_geometry<I, Off>(a.nx, a.ny, a.nz);
  tb2_kernel<I, Off><<<dim3(grid_for(g.ntiles)), dim3(kTbBlock), 0, (hipStream_t)a.stream>>>(
      a.b, a.p_in[0], a.p_in[1], a.p_in[2], a.p_out[0], a.p_out[1], a.p_out[2], a.r_in[0],
      a.r_in[1], a.r_in[2], a.r_out[0], a.r_out[1], a.r_out[2], a.lam, a.c, a.m1, a.m2, g);
  return hipGetLastError() == hipSuccess ? 0 : kLaunchFailed;
}

}  // namespace

int launch_tb2(const Step2Args &a) {
  return fits_u32_offsets(a.nx, a.ny, a.nz) ? launch_tb2_t<int32_t, uint32_t>(a)
                                            : launch_tb2_t<int64_t, uint64_t>(a);
}

}  // namespace tvfgp
