// Launcher of the LDS z-marching ablation (tv_fgp_lds_kernel.hpp).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_ablation_kernels.hpp"
#include "tv_fgp_launch.hpp"
#include "tv_fgp_lds_kernel.hpp"

namespace tvfgp {

namespace {

template <typename I, int TX, int TY>
int launch_lds_t(const StepArgs &a) {
  const Geometry<I> g = march_geometry<I>(a.nx, a.ny, a.nz, a.planes, TX, TY);
  lds_march_kernel<I, TX, TY><<<grid_for(g.ntiles), dim3(TX * TY), 0, (hipStream_t)a.stream>>>(
      a.b, a.p[0], a.p[1], a.p[2], a.r_in[0], a.r_in[1], a.r_in[2], a.r_out[0], a.r_out[1],
      a.r_out[2], a.lam, a.c, a.m, g);
  return hipGetLastError() == hipSuccess ? 0 : kLaunchFailed;
}

template <int TX, int TY>
int launch_lds_shape(const StepArgs &a) {
  return fits_int32(a.nx, a.ny, a.nz) ? launch_lds_t<int32_t, TX, TY>(a)
                                      : launch_lds_t<int64_t, TX, TY>(a);
}

}  // namespace

int launch_lds_march(const StepArgs &a) { return launch_lds_shape<kTileX, kTileY>(a); }

bool march_shape_supported(int tile_x, int tile_y) {
  return (tile_x == 32 && (tile_y == 4 || tile_y == 8 || tile_y == 16)) ||
         (tile_x == 64 && (tile_y == 4 || tile_y == 8));
}

int launch_lds_march_shape(const StepArgs &a, int tile_x, int tile_y) {
  if (tile_x == 32 && tile_y == 4) return launch_lds_shape<32, 4>(a);
  if (tile_x == 32 && tile_y == 8) return launch_lds_shape<32, 8>(a);
  if (tile_x == 32 && tile_y == 16) return launch_lds_shape<32, 16>(a);
  if (tile_x == 64 && tile_y == 4) return launch_lds_shape<64, 4>(a);
  if (tile_x == 64 && tile_y == 8) return launch_lds_shape<64, 8>(a);
  return kLaunchFailed;
}

}  // namespace tvfgp
