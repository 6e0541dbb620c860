// Launchers of the cube-tiled ablation kernel (tv_fgp_cube_kernel.hpp) for
// the cube shapes of the tile-shape sweep.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_cube_kernel.hpp"
#include "tv_fgp_launch.hpp"

namespace tvfgp {

namespace {

template <typename I, int TX, int TY, int TZ>
int launch_cube_t(const StepArgs &a) {
  const CubeGeometry<I> g = cube_geometry<I, TX, TY, TZ>(a.nx, a.ny, a.nz);
  cube_kernel<I, TX, TY, TZ><<<dim3(grid_for(g.ntiles)), dim3(kCubeBlock), 0,
                               (hipStream_t)a.stream>>>(
      a.b, a.p[0], a.p[1], a.p[2], a.r_in[0], a.r_in[1], a.r_in[2], a.r_out[0], a.r_out[1],
      a.r_out[2], a.lam, a.c, a.m, g);
  return hipGetLastError() == hipSuccess ? 0 : kLaunchFailed;
}

template <int TX, int TY, int TZ>
int launch_cube_shape(const StepArgs &a) {
  return cube_fits_int32(a.nx, a.ny, a.nz) ? launch_cube_t<int32_t, TX, TY, TZ>(a)
                                           : launch_cube_t<int64_t, TX, TY, TZ>(a);
}

}  // namespace

int launch_cube(const StepArgs &a) {
  switch (a.variant) {
    case kVariantCube: return launch_cube_shape<16, 8, 4>(a);
    case kVariantCube32x8x2: return launch_cube_shape<32, 8, 2>(a);
    case kVariantCube64x8x1: return launch_cube_shape<64, 8, 1>(a);
    case kVariantCube8x8x8: return launch_cube_shape<8, 8, 8>(a);
    case kVariantCube32x4x4: return launch_cube_shape<32, 4, 4>(a);
    default: return kLaunchFailed;
  }
}

}  // namespace tvfgp
