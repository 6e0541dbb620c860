// Launchers of the two-steps-per-pass FGP kernel (tv_fgp_tb2_kernel.hpp) for
// fp32 and binary16 dual volumes.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_launch.hpp"
#include "tv_fgp_tb2_kernel.hpp"

namespace tvfgp {

namespace {

template <typename I, typename Off, typename S>
int launch_tb2_t(const float *b, const S *const pi[3], S *const po[3], const S *const ri[3],
                 S *const ro[3], float lam, float c, float m1, float m2, int64_t nx,
                 int64_t ny, int64_t nz, void *stream) {
  const ZxGeometry<I, Off> g = tb_geometry<I, Off>(nx, ny, nz);
  tb2_kernel<I, Off, S><<<dim3(grid_for(g.ntiles)), dim3(kTbBlock), 0, (hipStream_t)stream>>>(
      b, pi[0], pi[1], pi[2], po[0], po[1], po[2], ri[0], ri[1], ri[2], ro[0], ro[1], ro[2], lam,
      c, m1, m2, g);
  return hipGetLastError() == hipSuccess ? 0 : kLaunchFailed;
}

template <typename S>
int launch_tb2_s(const float *b, const S *const pi[3], S *const po[3], const S *const ri[3],
                 S *const ro[3], float lam, float c, float m1, float m2, int64_t nx,
                 int64_t ny, int64_t nz, void *stream) {
  return fits_u32_offsets(nx, ny, nz)
             ? launch_tb2_t<int32_t, uint32_t, S>(b, pi, po, ri, ro, lam, c, m1, m2, nx, ny, nz,
                                                  stream)
             : launch_tb2_t<int64_t, uint64_t, S>(b, pi, po, ri, ro, lam, c, m1, m2, nx, ny, nz,
                                                  stream);
}

}  // namespace

int launch_tb2(const Step2Args &a) {
  return launch_tb2_s<float>(a.b, a.p_in, a.p_out, a.r_in, a.r_out, a.lam, a.c, a.m1, a.m2,
                             a.nx, a.ny, a.nz, a.stream);
}

int launch_tb2_h(const Step2ArgsH &a) {
  typedef _Float16 half_t;
  const half_t *const pi[3] = {(const half_t *)a.p_in[0], (const half_t *)a.p_in[1],
                               (const half_t *)a.p_in[2]};
  half_t *const po[3] = {(half_t *)a.p_out[0], (half_t *)a.p_out[1], (half_t *)a.p_out[2]};
  const half_t *const ri[3] = {(const half_t *)a.r_in[0], (const half_t *)a.r_in[1],
                               (const half_t *)a.r_in[2]};
  half_t *const ro[3] = {(half_t *)a.r_out[0], (half_t *)a.r_out[1], (half_t *)a.r_out[2]};
  return launch_tb2_s<half_t>(a.b, pi, po, ri, ro, a.lam, a.c, a.m1, a.m2, a.nx, a.ny, a.nz,
                              a.stream);
}

}  // namespace tvfgp
