// Launchers of the two-voxels-per-lane FGP kernel (tv_fgp_pair_kernel.hpp),
// for fp32 and binary16 dual volumes.  Shapes the pair kernel does not take
// (odd nx, volumes not aligned to two elements) go to the one-voxel kernel.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_launch.hpp"
#include "tv_fgp_pair_kernel.hpp"

namespace tvfgp {

namespace {

// Rows (and therefore planes) of the p volumes start on 128-byte lines.
inline bool rows_on_lines(int64_t nx, size_t elem, void *const *p) {
  if ((nx * (int64_t)elem) % 128 != 0) return false;
  for (int k = 0; k < 3; ++k)
    if (((uintptr_t)p[k]) % 128 != 0) return false;
  return true;
}

template <typename I, typename Off, typename S>
int launch_pair_t(const float *b, S *const p[3], const S *const ri[3], S *const ro[3],
                  float lam, float c, float m, int64_t nx, int64_t ny, int64_t nz,
                  void *stream) {
  const ZxGeometry<I, Off> g = pair_geometry<I, Off>(nx, ny, nz);
  const dim3 grid(grid_for(g.ntiles)), block(kPairBlock);
  hipStream_t s = (hipStream_t)stream;
  if (rows_on_lines(nx, sizeof(S), (void *const *)p))
    fused_pair_kernel<I, Off, true, S><<<grid, block, 0, s>>>(
        b, p[0], p[1], p[2], ri[0], ri[1], ri[2], ro[0], ro[1], ro[2], lam, c, m, g);
  else
    fused_pair_kernel<I, Off, false, S><<<grid, block, 0, s>>>(
        b, p[0], p[1], p[2], ri[0], ri[1], ri[2], ro[0], ro[1], ro[2], lam, c, m, g);
  return hipGetLastError() == hipSuccess ? 0 : kLaunchFailed;
}

template <typename S>
int launch_pair(const float *b, S *const p[3], const S *const ri[3], S *const ro[3],
                float lam, float c, float m, int64_t nx, int64_t ny, int64_t nz,
                void *stream) {
  return pair_fits_u32_offsets(nx, ny, nz)
             ? launch_pair_t<int32_t, uint32_t, S>(b, p, ri, ro, lam, c, m, nx, ny, nz, stream)
             : launch_pair_t<int64_t, uint64_t, S>(b, p, ri, ro, lam, c, m, nx, ny, nz,
                                                   stream);
}

template <typename T>
bool eligible(int64_t nx, const float *b, T *const p[3], const T *const ri[3],
              T *const ro[3], size_t elem) {
  const void *dual[9] = {p[0], p[1], p[2], ri[0], ri[1], ri[2], ro[0], ro[1], ro[2]};
  return pair_eligible(nx, b, dual, 9, elem);
}

}  // namespace

int launch_fused_pair(const StepArgs &a) {
  if (!eligible(a.nx, a.b, a.p, a.r_in, a.r_out, sizeof(float))) return launch_fused_zx(a);
  return launch_pair<float>(a.b, a.p, a.r_in, a.r_out, a.lam, a.c, a.m, a.nx, a.ny, a.nz,
                            a.stream);
}

int launch_fused_pair_h(const StepArgsH &a) {
  if (!eligible(a.nx, a.b, a.p, a.r_in, a.r_out, 2)) return launch_fused_zx_h(a);
  typedef _Float16 half_t;
  half_t *const p[3] = {(half_t *)a.p[0], (half_t *)a.p[1], (half_t *)a.p[2]};
  const half_t *const ri[3] = {(const half_t *)a.r_in[0], (const half_t *)a.r_in[1],
                               (const half_t *)a.r_in[2]};
  half_t *const ro[3] = {(half_t *)a.r_out[0], (half_t *)a.r_out[1], (half_t *)a.r_out[2]};
  return launch_pair<half_t>(a.b, p, ri, ro, a.lam, a.c, a.m, a.nx, a.ny, a.nz, a.stream);
}

}  // namespace tvfgp
