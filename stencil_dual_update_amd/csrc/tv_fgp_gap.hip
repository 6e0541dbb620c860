// Launcher of the duality-gap reduction (tv_fgp_gap_kernel.hpp).
#include <hip/hip_runtime.h>

#include <mutex>
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

// Partial triples of the allocation-free gap (launch_duality_gap_static):
// one per first-pass workgroup, at most kGapGrid of them, 24 KiB.  Each GPU
// the library runs on holds its own copy until the process ends.  In host
// code the name stands for a host-side handle, not a device address: kernels
// get the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) double scratch[3 * kGapGrid];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
double *scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// Device address of `scratch` on the current device, looked up once per
// device; nullptr if the runtime fails.
double *scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_ptr[dev] == nullptr) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return nullptr;
    scratch_ptr[dev] = (double *)ptr;
  }
  return scratch_ptr[dev];
}

}  // namespace

size_t gap_static_capacity_bytes() { return sizeof(scratch); }

int launch_duality_gap_static(const GapArgs &a) {
  if ((size_t)gap_partial_count(a.nx, a.ny, a.nz) * 3 * sizeof(double) > sizeof(scratch))
    return kLaunchFailed;
  double *partial = scratch_on_current_device();
  if (partial == nullptr) return kLaunchFailed;
  GapArgs s = a;
  s.partial = partial;  // every partial is written by pass 1 before pass 2 reads it
  return launch_duality_gap(s);
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
