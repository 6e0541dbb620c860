// Launcher of the duality-gap reduction (tv_fgp_gap_kernel.hpp).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_fused_kernel.hpp"
#include "tv_fgp_gap_kernel.hpp"
#include "tv_fgp_launch.hpp"

namespace tvfgp {

namespace {

template <typename I, typename Off>
int launch_gap_t(const GapArgs &a) {
  const ZxGeometry<I, Off> g = zx_geometry<I, Off>(a.nx, a.ny, a.nz);
  const int grid = gap_grid(a.nx, a.ny, a.nz);
  hipStream_t s = (hipStream_t)a.stream;
  gap_partial_kernel<I, Off><<<dim3(grid), dim3(kZxBlock), 0, s>>>(
      a.b, a.p[0], a.p[1], a.p[2], a.lam, g, a.partial);
  if (hipGetLastError() != hipSuccess) return kLaunchFailed;
  gap_final_kernel<<<dim3(1), dim3(kGapFinalBlock), 0, s>>>(
      a.partial, grid, (double)a.lam, a.out);
  return hipGetLastError() == hipSuccess ? 0 : kLaunchFailed;
}

}  // namespace

int gap_partial_count(int64_t nx, int64_t ny, int64_t nz) {
  return gap_grid(nx, ny, nz);
}

int launch_duality_gap(const GapArgs &a) {
  return fits_u32_offsets(a.nx, a.ny, a.nz) ? launch_gap_t<int32_t, uint32_t>(a)
                                            : launch_gap_t<int64_t, uint64_t>(a);
}

}  // namespace tvfgp
