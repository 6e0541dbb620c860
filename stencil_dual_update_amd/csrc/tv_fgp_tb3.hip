// Launcher of the three-steps-per-pass FGP kernel (tv_fgp_tb3_kernel.hpp).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <mutex>

#include "tv_fgp_launch.hpp"
#include "tv_fgp_tb3_kernel.hpp"

namespace tvfgp {

namespace {

// Resident workgroups of the three-step kernel on the current device: two per
// CU (its registers allow four waves per SIMD); 512 on MI355X.  Looked up once
// per device.
int64_t tb3_slots() {
  constexpr int kMaxDevices = 64;
  static int64_t slots[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 512;
  std::lock_guard<std::mutex> lock(mu);
  if (slots[dev] == 0) {
    int cus = 0;
    slots[dev] = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) ==
                             hipSuccess && cus > 0
                     ? 2 * (int64_t)cus
                     : 512;
  }
  return slots[dev];
}

template <typename I, typename Off>
int launch_tb3_t(const Step3Args &a) {
  const ZxGeometry<I, Off> g =
      tb_geometry<I, Off>(a.nx, a.ny, a.nz, tb3_planes(a.nx, a.ny, a.nz, tb3_slots()));
  tb3_kernel<I, Off, float><<<dim3(grid_for(g.ntiles)), dim3(kTbBlock), 0,
                              (hipStream_t)a.stream>>>(
      a.b, a.p_in[0], a.p_in[1], a.p_in[2], a.p_out[0], a.p_out[1], a.p_out[2], a.r_in[0],
      a.r_in[1], a.r_in[2], a.r_out[0], a.r_out[1], a.r_out[2], a.lam, a.c, a.m1, a.m2, a.m3,
      g);
  return hipGetLastError() == hipSuccess ? 0 : kLaunchFailed;
}

}  // namespace

int launch_tb3(const Step3Args &a) {
  return fits_u32_offsets(a.nx, a.ny, a.nz) ? launch_tb3_t<int32_t, uint32_t>(a)
                                            : launch_tb3_t<int64_t, uint64_t>(a);
}

}  // namespace tvfgp
