// Launcher of the duality-gap reduction (tv_fgp_gap_kernel.hpp).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_fused_kernel.hpp"
#include "tv_fgp_gap_kernel.hpp"
#include "tv_fgp_launch.hpp"
#include "tv_fgp_pair_kernel.hpp"

namespace tvfgp {

namespace {

int launch_gap_final(const GapArgs &a, int grid) {
  gap_final_kernel<<<dim3(1), dim3(kGapFinalBlock), 0, (hipStream_t)a.stream>>>(
      a.partial, grid, (double)a.lam, a.out);
  return hipGetLastError() == hipSuccess ? 0 : kLaunchFailed;
}

template <typename I, typename Off>
int launch_gap_t(const GapArgs &a) {
  const ZxGeometry<I, Off> g = zx_geometry<I, Off>(a.nx, a.ny, a.nz);
  const int grid = gap_grid(a.nx, a.ny, a.nz);
  gap_partial_kernel<I, Off><<<dim3(grid), dim3(kZxBlock), 0, (hipStream_t)a.stream>>>(
      a.b, a.p[0], a.p[1], a.p[2], a.lam, g, a.partial);
  if (hipGetLastError() != hipSuccess) return kLaunchFailed;
  return launch_gap_final(a, grid);
}

template <typename I, typename Off>
int launch_gap_pair_t(const GapArgs &a) {
  const ZxGeometry<I, Off> g = gap_pair_geometry<I, Off>(a.nx, a.ny, a.nz);
  const int grid = gap_pair_grid(a.nx, a.ny, a.nz);
  gap_partial_pair_kernel<I, Off><<<dim3(grid), dim3(kPairBlock), 0, (hipStream_t)a.stream>>>(
      a.b, a.p[0], a.p[1], a.p[2], a.lam, g, a.partial);
  if (hipGetLastError() != hipSuccess) return kLaunchFailed;
  return launch_gap_final(a, grid);
}

}  // namespace

// Enough partial triples for either first pass (the pair kernel's tiles are
// larger, so its grid is never the larger one).
int gap_partial_count(int64_t nx, int64_t ny, int64_t nz) {
  return gap_grid(nx, ny, nz);
}

int launch_duality_gap(const GapArgs &a) {
  const void *dual[3] = {a.p[0], a.p[1], a.p[2]};
  if (pair_eligible(a.nx, a.b, dual, 3, sizeof(float)))
    return pair_fits_u32_offsets(a.nx, a.ny, a.nz) ? launch_gap_pair_t<int32_t, uint32_t>(a)
                                                   : launch_gap_pair_t<int64_t, uint64_t>(a);
  return fits_u32_offsets(a.nx, a.ny, a.nz) ? launch_gap_t<int32_t, uint32_t>(a)
                                            : launch_gap_t<int64_t, uint64_t>(a);
}

}  // namespace tvfgp
