// Bandwidth probe for the traffic of one FGP step.
//
// The page "TV solver: the FGP step on the GPU" (section "Profiler counters"
// and its closing paragraph) prices a fused step by the bytes it moves: 13
// volumes, the 7 it reads (b, p, r) and the 6 it writes (p, r).  This kernel
// moves exactly that mix as a plain linear stream, with none of the step's
// arithmetic and none of its neighbour reads: 16-byte loads of the seven
// inputs and non-temporal 16-byte stores of the six outputs, each thread
// taking one 4-float group of every volume.  Its time is the ceiling a step
// kernel of the same traffic can reach on the part.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_launch.hpp"

namespace tvfgp {

namespace {

constexpr int kProbeBlock = 256;

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Probe13 {
  const f32x4 *s[7];
  f32x4 *d[6];
};

// d_k = s_k + s_6 for k < 6, so that every input is consumed.
__global__ __launch_bounds__(kProbeBlock) void stream13_kernel(Probe13 v, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * kProbeBlock + threadIdx.x;
  if (i >= n4) return;
  const f32x4 a0 = v.s[0][i], a1 = v.s[1][i], a2 = v.s[2][i], a3 = v.s[3][i];
  const f32x4 a4 = v.s[4][i], a5 = v.s[5][i], a6 = v.s[6][i];
  __builtin_nontemporal_store(a0 + a6, &v.d[0][i]);
  __builtin_nontemporal_store(a1 + a6, &v.d[1][i]);
  __builtin_nontemporal_store(a2 + a6, &v.d[2][i]);
  __builtin_nontemporal_store(a3 + a6, &v.d[3][i]);
  __builtin_nontemporal_store(a4 + a6, &v.d[4][i]);
  __builtin_nontemporal_store(a5 + a6, &v.d[5][i]);
}

struct Tail13 {
  const float *s[7];
  float *d[6];
};

// The last n % 4 elements, one thread each.
__global__ void stream13_tail(Tail13 v, int64_t start, int64_t n) {
  const int64_t i = start + (int64_t)threadIdx.x;
  if (i >= n) return;
  for (int k = 0; k < 6; ++k) v.d[k][i] = v.s[k][i] + v.s[6][i];
}

}  // namespace

int launch_stream13(const float *const src[7], float *const dst[6], int64_t n, void *stream) {
  const int64_t n4 = n / 4;
  hipStream_t s = (hipStream_t)stream;
  if (n4 > 0) {
    Probe13 v;
    for (int k = 0; k < 7; ++k) v.s[k] = (const f32x4 *)src[k];
    for (int k = 0; k < 6; ++k) v.d[k] = (f32x4 *)dst[k];
    const int64_t grid = (n4 + kProbeBlock - 1) / kProbeBlock;
    if (grid > 0x7fffffff) return kLaunchFailed;
    stream13_kernel<<<dim3((unsigned)grid), dim3(kProbeBlock), 0, s>>>(v, n4);
    if (hipGetLastError() != hipSuccess) return kLaunchFailed;
  }
  if (n % 4 != 0) {
    Tail13 t;
    for (int k = 0; k < 7; ++k) t.s[k] = src[k];
    for (int k = 0; k < 6; ++k) t.d[k] = dst[k];
    stream13_tail<<<dim3(1), dim3(4), 0, s>>>(t, 4 * n4, n);
    if (hipGetLastError() != hipSuccess) return kLaunchFailed;
  }
  return 0;
}

}  // namespace tvfgp
