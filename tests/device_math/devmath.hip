// Test kernels for the correctly rounded square root and quotients of the
// dual update (tv_fgp_device.hpp) and the duality gap's double square root
// (tv_fgp_gap_kernel.hpp) on the GPU.  Each writes what it computes
// with plain vector stores; the Python test compares it with the host's IEEE
// results.  Test infrastructure only, built next to this file as
// libdevmath.so.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_device.hpp"
#include "tv_fgp_gap_kernel.hpp"

namespace {

constexpr int kBlock = 256;

// out[i] = sqrt_above_one(x) for the float x with bit pattern lo + i
__global__ void sqrt_kernel(uint32_t lo, int64_t count, float *out) {
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * kBlock)
    out[i] = tvfgp::sqrt_above_one(__builtin_bit_cast(float, (uint32_t)(lo + (uint32_t)i)));
}

// out[i] = recip_refined(d) for the float d with bit pattern lo + i
__global__ void recip_kernel(uint32_t lo, int64_t count, float *out) {
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * kBlock)
    out[i] = tvfgp::recip_refined(__builtin_bit_cast(float, (uint32_t)(lo + (uint32_t)i)));
}

// out[i] = div_by_refined(n[i], d[i], recip_refined(d[i]))
__global__ void div_kernel(const float *n, const float *d, int64_t count, float *out) {
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * kBlock)
    out[i] = tvfgp::div_by_refined(n[i], d[i], tvfgp::recip_refined(d[i]));
}

// out[i] = sqrt_sum_of_squares(s[i]), ref[i] = sqrt(s[i]) (the compiler's)
__global__ void sqrt64_kernel(const double *s, int64_t count, double *out, double *ref) {
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * kBlock) {
    out[i] = tvfgp::sqrt_sum_of_squares(s[i]);
    ref[i] = __builtin_sqrt(s[i]);
  }
}

unsigned grid(int64_t count) {
  const int64_t g = (count + kBlock - 1) / kBlock;
  return (unsigned)(g < 65536 ? (g < 1 ? 1 : g) : 65536);
}

}  // namespace

// Each returns 0, or the HIP error of the launch.  out, n and d are device
// arrays of count floats (s, out and ref of count doubles); the work is
// enqueued on the null stream.
extern "C" int devmath_sqrt(uint32_t lo, int64_t count, float *out) {
  sqrt_kernel<<<grid(count), kBlock>>>(lo, count, out);
  return (int)hipGetLastError();
}

extern "C" int devmath_recip(uint32_t lo, int64_t count, float *out) {
  recip_kernel<<<grid(count), kBlock>>>(lo, count, out);
  return (int)hipGetLastError();
}

extern "C" int devmath_div(const float *n, const float *d, int64_t count, float *out) {
  div_kernel<<<grid(count), kBlock>>>(n, d, count, out);
  return (int)hipGetLastError();
}

extern "C" int devmath_sqrt64(const double *s, int64_t count, double *out, double *ref) {
  sqrt64_kernel<<<grid(count), kBlock>>>(s, count, out, ref);
  return (int)hipGetLastError();
}
