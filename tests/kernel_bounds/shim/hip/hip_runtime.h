// Host stand-in for the few HIP names the kernel headers use, so the kernel
// sources compile as ordinary C++ for the CPU bounds check.  Test
// infrastructure only; the library itself is built with hipcc for gfx950.
#pragma once

#include <math.h>
#include <stdint.h>

#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __shared__ static
#define __launch_bounds__(...)

struct EmulDim3 {
  unsigned x, y, z;
};

extern thread_local EmulDim3 threadIdx, blockIdx, gridDim, blockDim;

// Threads run one after another, so a barrier has nothing to wait for; LDS
// contents are then meaningless, but every address a thread forms is the
// one it forms on the GPU, which is what the check is about.
inline void __syncthreads() {}
