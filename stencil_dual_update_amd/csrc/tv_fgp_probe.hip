// Bandwidth probes for the traffic of one FGP step.
//
// The page "TV solver: the FGP step on the GPU" (section "Profiler counters"
// and its closing paragraph) prices a fused step by the bytes it moves: 13
// volumes, the 7 it reads (b, p, r) and the 6 it writes (p, r).  The main
// probe moves exactly that mix as a plain linear stream, with none of the
// step's arithmetic and none of its neighbour reads: each thread takes one
// 4-float group of every volume, with non-temporal 16-byte loads and stores
// (the fastest of the linear forms measured on MI355X: plain loads, plain
// stores, 512-thread blocks, grid-stride loops and two or four groups per
// thread were all slower).  Its time is the ceiling a step kernel of the same
// traffic can reach on the part.  Three more shapes give the part's rates for
// reading only (7 volumes), writing only (6) and a one-to-one copy.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tv_fgp_launch.hpp"

namespace tvfgp {

namespace {

constexpr int kProbeBlock = 256;

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct ProbeVols {
  const f32x4 *s[7];
  f32x4 *d[6];
};

__device__ __forceinline__ f32x4 ld_nt(const f32x4 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt(f32x4 v, f32x4 *p) { __builtin_nontemporal_store(v, p); }
// Marks a value as used without storing it (an empty asm statement that
// takes it as an operand), so that the read-only shape's loads are kept.
__device__ __forceinline__ void keep(float v) { asm volatile("" : : "v"(v)); }

// NS sources, ND destinations: (7, 6) d_k = s_k + s_6; (1, 1) d_0 = s_0;
// (0, 6) d_k = k; (7, 0) the seven are summed and the sum dropped.
template <int NS, int ND>
__global__ __launch_bounds__(kProbeBlock) void stream_kernel(ProbeVols v, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * kProbeBlock + threadIdx.x;
  if (i >= n4) return;
  if constexpr (NS == 7 && ND == 6) {
    f32x4 a[7];
#pragma unroll
    for (int k = 0; k < 7; ++k) a[k] = ld_nt(&v.s[k][i]);
#pragma unroll
    for (int k = 0; k < 6; ++k) st_nt(a[k] + a[6], &v.d[k][i]);
  } else if constexpr (NS == 1 && ND == 1) {
    st_nt(ld_nt(&v.s[0][i]), &v.d[0][i]);
  } else if constexpr (NS == 0 && ND == 6) {
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      const float f = (float)k;
      st_nt(f32x4{f, f, f, f}, &v.d[k][i]);
    }
  } else {
    static_assert(NS == 7 && ND == 0, "probe shapes: (7, 6), (1, 1), (0, 6), (7, 0)");
    f32x4 s = ld_nt(&v.s[0][i]);
#pragma unroll
    for (int k = 1; k < 7; ++k) s += ld_nt(&v.s[k][i]);
    keep(s.x);
    keep(s.y);
    keep(s.z);
    keep(s.w);
  }
}

struct TailVols {
  const float *s[7];
  float *d[6];
};

// The last n % 4 elements, one thread each, with the same rule.
__global__ void stream_tail(TailVols v, int ns, int nd, int64_t start, int64_t n) {
  const int64_t i = start + (int64_t)threadIdx.x;
  if (i >= n) return;
  if (ns == 7 && nd == 6) {
    for (int k = 0; k < 6; ++k) v.d[k][i] = v.s[k][i] + v.s[6][i];
  } else if (ns == 1 && nd == 1) {
    v.d[0][i] = v.s[0][i];
  } else if (ns == 0 && nd == 6) {
    for (int k = 0; k < 6; ++k) v.d[k][i] = (float)k;
  } else {
    float s = 0.0f;
    for (int k = 0; k < 7; ++k) s += v.s[k][i];
    keep(s);
  }
}

template <int NS, int ND>
int launch_shape(const ProbeVols &v, int64_t n4, hipStream_t s) {
  const int64_t grid = (n4 + kProbeBlock - 1) / kProbeBlock;
  if (grid > 0x7fffffff) return kLaunchFailed;
  stream_kernel<NS, ND><<<dim3((unsigned)grid), dim3(kProbeBlock), 0, s>>>(v, n4);
  return hipGetLastError() == hipSuccess ? 0 : kLaunchFailed;
}

}  // namespace

bool stream_shape_supported(int n_src, int n_dst) {
  return (n_src == 7 && n_dst == 6) || (n_src == 1 && n_dst == 1) ||
         (n_src == 0 && n_dst == 6) || (n_src == 7 && n_dst == 0);
}

int launch_stream(const float *const *src, int n_src, float *const *dst, int n_dst, int64_t n,
                  void *stream) {
  if (!stream_shape_supported(n_src, n_dst)) return kLaunchFailed;
  const int64_t n4 = n / 4;
  hipStream_t s = (hipStream_t)stream;
  if (n4 > 0) {
    ProbeVols v = {};
    for (int k = 0; k < n_src; ++k) v.s[k] = (const f32x4 *)src[k];
    for (int k = 0; k < n_dst; ++k) v.d[k] = (f32x4 *)dst[k];
    int st;
    if (n_src == 7 && n_dst == 6)
      st = launch_shape<7, 6>(v, n4, s);
    else if (n_src == 1)
      st = launch_shape<1, 1>(v, n4, s);
    else if (n_src == 0)
      st = launch_shape<0, 6>(v, n4, s);
    else
      st = launch_shape<7, 0>(v, n4, s);
    if (st != 0) return st;
  }
  if (n % 4 != 0) {
    TailVols t = {};
    for (int k = 0; k < n_src; ++k) t.s[k] = src[k];
    for (int k = 0; k < n_dst; ++k) t.d[k] = dst[k];
    stream_tail<<<dim3(1), dim3(4), 0, s>>>(t, n_src, n_dst, 4 * n4, n);
    if (hipGetLastError() != hipSuccess) return kLaunchFailed;
  }
  return 0;
}

int launch_stream13(const float *const src[7], float *const dst[6], int64_t n, void *stream) {
  return launch_stream(src, 7, dst, 6, n, stream);
}

}  // namespace tvfgp
