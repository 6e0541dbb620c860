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

#ifdef TVFGP_EMUL_THREADS
// Functional emulation: every thread of a workgroup is an OS thread and the
// barrier is a real one (func.cpp), so LDS exchanges behave as on the GPU.
void emul_syncthreads();
inline void __syncthreads() { emul_syncthreads(); }
#else
// Bounds check: threads run one after another, so a barrier has nothing to
// wait for; LDS contents are then meaningless, but every address a thread
// forms is the one it forms on the GPU, which is what the check is about.
inline void __syncthreads() {}
#endif
