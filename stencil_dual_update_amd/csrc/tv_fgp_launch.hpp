// Internal interface between the C-ABI layer (argument checks, momentum
// schedule, buffer ping-pong) and the kernel launchers.  Arguments reaching
// a launcher have been validated: pointers non-null, aligned and disjoint,
// dimensions >= 1, parameters finite.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace tvfgp {

constexpr int kVariantFused = 0;
constexpr int kVariantLdsMarch = 1;
constexpr int kVariantTwoKernel = 2;
constexpr int kVariantPoint = 3;
constexpr int kVariantRegMarch = 4;
constexpr int kVariantPair = 5;
constexpr int kVariantTb2 = 6;
constexpr int kVariantCube = 7;  // 16 x 8 x 4 cubes, then other cube shapes
constexpr int kVariantCube32x8x2 = 8;
constexpr int kVariantCube64x8x1 = 9;
constexpr int kVariantCube8x8x8 = 10;
constexpr int kVariantCube32x4x4 = 11;
constexpr int kVariantTb3 = 12;
constexpr int kNumVariants = 13;

constexpr int kLaunchFailed = -1;

// Planes along z that one thread (or one tile) walks in the marching
// ablation kernels (the default kernel fixes its own tile shape).
constexpr int64_t kDefaultPlanes = 8;

struct StepArgs {
  const float *b;
  float *p[3];
  const float *r_in[3];
  float *r_out[3];
  float *z_ws;       // two-kernel variant only
  float lam;         // lambda
  float c;           // 1 / (12 lambda), rounded in fp32
  float m;           // momentum coefficient
  int64_t nx, ny, nz;
  int64_t planes;    // planes per tile along z
  int variant;
  void *stream;      // hipStream_t
};

// Two consecutive steps in one pass (momentum m1, then m2): p is read from
// p_in and written to p_out, r from r_in to r_out.
struct Step2Args {
  const float *b;
  const float *p_in[3];
  float *p_out[3];
  const float *r_in[3];
  float *r_out[3];
  float lam, c, m1, m2;
  int64_t nx, ny, nz;
  void *stream;
};

// Step2Args with the dual stored as binary16.
struct Step2ArgsH {
  const float *b;
  const uint16_t *p_in[3];
  uint16_t *p_out[3];
  const uint16_t *r_in[3];
  uint16_t *r_out[3];
  float lam, c, m1, m2;
  int64_t nx, ny, nz;
  void *stream;
};

// Three steps in one pass: p_in -> p_out (separate buffers), r_in -> r_out,
// momentum m1, m2, m3 for the three steps.
struct Step3Args {
  const float *b;
  const float *p_in[3];
  float *p_out[3];
  const float *r_in[3];
  float *r_out[3];
  float lam, c, m1, m2, m3;
  int64_t nx, ny, nz;
  void *stream;
};

struct PrimalArgs {
  const float *b;
  const float *p[3];
  float *z;
  float lam;
  int64_t nx, ny, nz;
  int64_t planes;
  void *stream;
};

// Step with the dual stored as binary16 (default kernel only).  The 16-bit
// pointers hold IEEE binary16 values.
struct StepArgsH {
  const float *b;
  uint16_t *p[3];
  const uint16_t *r_in[3];
  uint16_t *r_out[3];
  float lam, c, m;
  int64_t nx, ny, nz;
  void *stream;
};

struct PrimalArgsH {
  const float *b;
  const uint16_t *p[3];
  float *z;
  float lam;
  int64_t nx, ny, nz;
  void *stream;
};

struct GapArgs {
  const float *b;
  const float *p[3];
  float lam;
  int64_t nx, ny, nz;
  double *out;      // 3 doubles, device
  double *partial;  // 3 * gap_partial_count(...) doubles, device
  void *stream;
};

// Enqueue one step / one read-out.  Return 0, or kLaunchFailed when the HIP
// runtime reports an error after a launch.
int launch_step(const StepArgs &a);
int launch_primal(const PrimalArgs &a);
int launch_lds_march(const StepArgs &a);
int launch_fused_zx(const StepArgs &a);
int launch_fused_zx_h(const StepArgsH &a);
// Two voxels per lane where nx is even and the volumes are aligned to two
// elements; otherwise the one-voxel kernel above.
int launch_fused_pair(const StepArgs &a);
int launch_fused_pair_h(const StepArgsH &a);
int launch_tb2(const Step2Args &a);
int launch_tb2_h(const Step2ArgsH &a);
int launch_tb3(const Step3Args &a);
// LDS z-march with a tile of tile_x x tile_y (32 x 4, 32 x 8, 32 x 16,
// 64 x 4, 64 x 8) and a.planes planes per tile.
bool march_shape_supported(int tile_x, int tile_y);
int launch_lds_march_shape(const StepArgs &a, int tile_x, int tile_y);
// Cube-tiled ablation, shape chosen by a.variant (kVariantCube...).
int launch_cube(const StepArgs &a);
int launch_primal_h(const PrimalArgsH &a);
// Duality gap of p (two kernels: partial sums, then their fixed-order sum).
int launch_duality_gap(const GapArgs &a);
// Partial triples the gap reduction writes for these dimensions.
int gap_partial_count(int64_t nx, int64_t ny, int64_t nz);
// launch_duality_gap with a.partial ignored: the partial sums go to a static
// device array of the library (gap_static_capacity_bytes bytes per device),
// so nothing is allocated.  Calls that overlap on one device race on it.
int launch_duality_gap_static(const GapArgs &a);
size_t gap_static_capacity_bytes();
// Bandwidth probe: dst[k][i] = src[k][i] + src[6][i] for k < 6 over n
// elements (the 7-read / 6-write traffic of one step as a linear stream).
// The volumes must be 16-byte aligned.
int launch_stream13(const float *const src[7], float *const dst[6], int64_t n, void *stream);
bool stream_shape_supported(int n_src, int n_dst);
int launch_stream(const float *const *src, int n_src, float *const *dst, int n_dst, int64_t n,
                  void *stream);

}  // namespace tvfgp
