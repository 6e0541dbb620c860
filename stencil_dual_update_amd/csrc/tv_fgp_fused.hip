// Launcher of the default FGP kernel (tv_fgp_fused_kernel.hpp).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_fused_kernel.hpp"
#include "tv_fgp_launch.hpp"

namespace tvfgp {

namespace {

// Rows (and therefore planes) of p start on 128-byte boundaries.
inline bool rows_line_aligned(const StepArgs &a) {
  if ((a.nx * 4) % 128 != 0) return false;
  for (int k = 0; k < 3; ++k)
    if (((uintptr_t)a.p[k]) % 128 != 0) return false;
  return true;
}

template <typename I, typename Off>
int launch_zx(const StepArgs &a) {
  const ZxGeometry<I, Off> g = zx_geometry<I, Off>(a.nx, a.ny, a.nz);
  const dim3 grid(grid_for(g.ntiles)), block(kZxBlock);
  hipStream_t s = (hipStream_t)a.stream;
  if (rows_line_aligned(a))
    fused_zx_kernel<I, Off, true, float><<<grid, block, 0, s>>>(
        a.b, a.p[0], a.p[1], a.p[2], a.r_in[0], a.r_in[1], a.r_in[2],
        a.r_out[0], a.r_out[1], a.r_out[2], a.lam, a.c, a.m, g);
  else
    fused_zx_kernel<I, Off, false, float><<<grid, block, 0, s>>>(
        a.b, a.p[0], a.p[1], a.p[2], a.r_in[0], a.r_in[1], a.r_in[2],
        a.r_out[0], a.r_out[1], a.r_out[2], a.lam, a.c, a.m, g);
  return hipGetLastError() == hipSuccess ? 0 : kLaunchFailed;
}

using half_t = _Float16;

inline bool rows_line_aligned_h(const StepArgsH &a) {
  if ((a.nx * 2) % 128 != 0) return false;
  for (int k = 0; k < 3; ++k)
    if (((uintptr_t)a.p[k]) % 128 != 0) return false;
  return true;
}

template <typename I, typename Off>
int launch_zx_h(const StepArgsH &a) {
  const ZxGeometry<I, Off> g = zx_geometry<I, Off>(a.nx, a.ny, a.nz);
  const dim3 grid(grid_for(g.ntiles)), block(kZxBlock);
  hipStream_t s = (hipStream_t)a.stream;
  half_t *p0 = (half_t *)a.p[0], *p1 = (half_t *)a.p[1], *p2 = (half_t *)a.p[2];
  const half_t *r0 = (const half_t *)a.r_in[0], *r1 = (const half_t *)a.r_in[1],
               *r2 = (const half_t *)a.r_in[2];
  half_t *o0 = (half_t *)a.r_out[0], *o1 = (half_t *)a.r_out[1], *o2 = (half_t *)a.r_out[2];
  if (rows_line_aligned_h(a))
    fused_zx_kernel<I, Off, true, half_t><<<grid, block, 0, s>>>(
        a.b, p0, p1, p2, r0, r1, r2, o0, o1, o2, a.lam, a.c, a.m, g);
  else
    fused_zx_kernel<I, Off, false, half_t><<<grid, block, 0, s>>>(
        a.b, p0, p1, p2, r0, r1, r2, o0, o1, o2, a.lam, a.c, a.m, g);
  return hipGetLastError() == hipSuccess ? 0 : kLaunchFailed;
}

}  // namespace

int launch_fused_zx_h(const StepArgsH &a) {
  return fits_u32_offsets(a.nx, a.ny, a.nz)
             ? launch_zx_h<int32_t, uint32_t>(a)
             : launch_zx_h<int64_t, uint64_t>(a);
}

int launch_fused_zx(const StepArgs &a) {
  return fits_u32_offsets(a.nx, a.ny, a.nz)
             ? launch_zx<int32_t, uint32_t>(a)
             : launch_zx<int64_t, uint64_t>(a);
}

}  // namespace tvfgp
