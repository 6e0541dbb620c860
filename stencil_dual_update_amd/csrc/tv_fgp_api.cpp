// C-ABI layer of the FGP library: argument checks, the FISTA momentum
// schedule, the r ping-pong of the inner loop, and dispatch to the kernel
// launchers.  Everything here is host code; nothing allocates, synchronises
// or touches device memory, and a call that fails validation enqueues
// nothing.
#include "tv_fgp.h"

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "tv_fgp_launch.hpp"

namespace {

// Bytes one volume occupies, or 0 when the dimensions are invalid or the
// size overflows.
size_t volume_bytes(int64_t nx, int64_t ny, int64_t nz) {
  if (nx < 1 || ny < 1 || nz < 1) return 0;
  const uint64_t lim = (uint64_t)INT64_MAX / sizeof(float);
  const uint64_t ux = (uint64_t)nx, uy = (uint64_t)ny, uz = (uint64_t)nz;
  if (ux > lim / uy) return 0;
  const uint64_t nxy = ux * uy;
  if (nxy > lim / uz) return 0;
  return (size_t)(nxy * uz * sizeof(float));
}

struct Buf {
  const void *ptr;
  bool written;
};

// Every buffer must be non-null and 4-byte aligned, and a written buffer may
// not overlap any other buffer.  All buffers span `bytes`.
int check_buffers(const Buf *bufs, int count, size_t bytes) {
  for (int k = 0; k < count; ++k)
    if (bufs[k].ptr == nullptr) return TV_ERR_NULL;
  for (int k = 0; k < count; ++k)
    if (((uintptr_t)bufs[k].ptr & (sizeof(float) - 1)) != 0) return TV_ERR_ALIGN;
  for (int k = 0; k < count; ++k) {
    const uintptr_t a = (uintptr_t)bufs[k].ptr;
    if (a > UINTPTR_MAX - bytes) return TV_ERR_DIMS;
    for (int l = k + 1; l < count; ++l) {
      if (!bufs[k].written && !bufs[l].written) continue;
      const uintptr_t c = (uintptr_t)bufs[l].ptr;
      if (a < c + bytes && c < a + bytes) return TV_ERR_ALIAS;
    }
  }
  return TV_OK;
}

int check_lambda(float lambda, float *c_out) {
  if (!isfinite(lambda) || !(lambda > 0.0f)) return TV_ERR_PARAM;
  const float twelve_lam = 12.0f * lambda;
  const float c = 1.0f / twelve_lam;
  if (!isfinite(twelve_lam) || !isfinite(c)) return TV_ERR_PARAM;
  *c_out = c;
  return TV_OK;
}

bool known_variant(int v) { return v >= 0 && v < tvfgp::kNumVariants; }

tvfgp::StepArgs make_step(const float *b, float *const p[3],
                          const float *const r_in[3], float *const r_out[3],
                          float lambda, float c, float m, int64_t nx,
                          int64_t ny, int64_t nz, int variant, float *z_ws,
                          void *stream) {
  tvfgp::StepArgs a;
  a.b = b;
  for (int k = 0; k < 3; ++k) {
    a.p[k] = p[k];
    a.r_in[k] = r_in[k];
    a.r_out[k] = r_out[k];
  }
  a.z_ws = z_ws;
  a.lam = lambda;
  a.c = c;
  a.m = m;
  a.nx = nx;
  a.ny = ny;
  a.nz = nz;
  a.planes = tvfgp::kDefaultPlanes;
  a.variant = variant;
  a.stream = stream;
  return a;
}

// Shared checks of a step: variant, dimensions, lambda, m, buffers.
int check_step(const float *b, float *const p[3], const float *const r_in[3],
               float *const r_out[3], float lambda, float m, int64_t nx,
               int64_t ny, int64_t nz, int variant, const float *z_ws,
               float *c_out) {
  if (!known_variant(variant)) return TV_ERR_VARIANT;
  if (p == nullptr || r_in == nullptr || r_out == nullptr) return TV_ERR_NULL;
  const size_t bytes = volume_bytes(nx, ny, nz);
  if (bytes == 0) return TV_ERR_DIMS;
  int st = check_lambda(lambda, c_out);
  if (st != TV_OK) return st;
  if (!isfinite(m)) return TV_ERR_PARAM;
  const bool two = variant == tvfgp::kVariantTwoKernel;
  if (two && z_ws == nullptr) return TV_ERR_WORKSPACE;
  Buf bufs[11] = {{b, false},        {p[0], true},     {p[1], true},
                  {p[2], true},      {r_in[0], false}, {r_in[1], false},
                  {r_in[2], false},  {r_out[0], true}, {r_out[1], true},
                  {r_out[2], true},  {z_ws, true}};
  return check_buffers(bufs, two ? 11 : 10, bytes);
}

int launch_status(int rc) { return rc == 0 ? TV_OK : TV_ERR_LAUNCH; }

}  // namespace

extern "C" {

float tv_fgp_momentum(int k) {
  if (k < 1) return 0.0f;
  // FISTA sequence: t_1 = 1, t_{k+1} = (1 + sqrt(1 + 4 t_k^2)) / 2,
  // m_k = (t_k - 1) / t_{k+1}; double precision, rounded once.
  double t = 1.0;
  double t_next = (1.0 + sqrt(1.0 + 4.0 * t * t)) / 2.0;
  for (int s = 2; s <= k; ++s) {
    t = t_next;
    t_next = (1.0 + sqrt(1.0 + 4.0 * t * t)) / 2.0;
  }
  return (float)((t - 1.0) / t_next);
}

int tv_fgp_step_ex(const float *b, float *const p[3],
                   const float *const r_in[3], float *const r_out[3],
                   float lambda, float m, int64_t nx, int64_t ny, int64_t nz,
                   int variant, float *z_ws, void *stream) {
  float c = 0.0f;
  const int st =
      check_step(b, p, r_in, r_out, lambda, m, nx, ny, nz, variant, z_ws, &c);
  if (st != TV_OK) return st;
  return launch_status(tvfgp::launch_step(
      make_step(b, p, r_in, r_out, lambda, c, m, nx, ny, nz, variant, z_ws,
                stream)));
}

int tv_fgp_step(const float *b, float *const p[3], const float *const r_in[3],
                float *const r_out[3], float lambda, float m, int64_t nx,
                int64_t ny, int64_t nz, void *stream) {
  return tv_fgp_step_ex(b, p, r_in, r_out, lambda, m, nx, ny, nz,
                        tvfgp::kVariantFused, nullptr, stream);
}

int tv_fgp_run(const float *b, float *const p[3], float *const r_a[3],
               float *const r_b[3], float lambda, int n_outer, int n_inner,
               int64_t nx, int64_t ny, int64_t nz, int variant, float *z_ws,
               void *stream, int *r_final) {
  if (r_final) *r_final = 0;
  if (!known_variant(variant)) return TV_ERR_VARIANT;
  if (p == nullptr || r_a == nullptr || r_b == nullptr) return TV_ERR_NULL;
  const size_t bytes = volume_bytes(nx, ny, nz);
  if (bytes == 0) return TV_ERR_DIMS;
  if (n_outer < 0 || n_inner < 0) return TV_ERR_PARAM;
  float c = 0.0f;
  int st = check_lambda(lambda, &c);
  if (st != TV_OK) return st;
  const bool two = variant == tvfgp::kVariantTwoKernel;
  if (two && z_ws == nullptr) return TV_ERR_WORKSPACE;
  Buf bufs[11] = {{b, false},     {p[0], true},   {p[1], true},  {p[2], true},
                  {r_a[0], true}, {r_a[1], true}, {r_a[2], true}, {r_b[0], true},
                  {r_b[1], true}, {r_b[2], true}, {z_ws, true}};
  st = check_buffers(bufs, two ? 11 : 10, bytes);
  if (st != TV_OK) return st;

  const float *cur_in[3] = {r_a[0], r_a[1], r_a[2]};
  float *cur_out[3] = {r_b[0], r_b[1], r_b[2]};
  int where = 0;
  for (int o = 0; o < n_outer; ++o) {
    double t = 1.0;
    for (int k = 1; k <= n_inner; ++k) {
      const double t_next = (1.0 + sqrt(1.0 + 4.0 * t * t)) / 2.0;
      const float m = (float)((t - 1.0) / t_next);
      t = t_next;
      const int rc = tvfgp::launch_step(make_step(b, p, cur_in, cur_out, lambda,
                                                  c, m, nx, ny, nz, variant,
                                                  z_ws, stream));
      if (rc != 0) return TV_ERR_LAUNCH;
      where ^= 1;
      float *const *next_in = where ? r_b : r_a;
      float *const *next_out = where ? r_a : r_b;
      for (int a = 0; a < 3; ++a) {
        cur_in[a] = next_in[a];
        cur_out[a] = next_out[a];
      }
      if (r_final) *r_final = where;
    }
  }
  return TV_OK;
}

int tv_primal(const float *b, const float *const p[3], float *z, float lambda,
              int64_t nx, int64_t ny, int64_t nz, void *stream) {
  if (p == nullptr) return TV_ERR_NULL;
  const size_t bytes = volume_bytes(nx, ny, nz);
  if (bytes == 0) return TV_ERR_DIMS;
  float c = 0.0f;
  int st = check_lambda(lambda, &c);
  if (st != TV_OK) return st;
  Buf bufs[5] = {{b, false}, {p[0], false}, {p[1], false}, {p[2], false},
                 {z, true}};
  st = check_buffers(bufs, 5, bytes);
  if (st != TV_OK) return st;
  tvfgp::PrimalArgs a;
  a.b = b;
  for (int k = 0; k < 3; ++k) a.p[k] = p[k];
  a.z = z;
  a.lam = lambda;
  a.nx = nx;
  a.ny = ny;
  a.nz = nz;
  a.planes = tvfgp::kDefaultPlanes;
  a.stream = stream;
  return launch_status(tvfgp::launch_primal(a));
}

size_t tv_fgp_workspace_bytes(int variant, int64_t nx, int64_t ny, int64_t nz) {
  if (!known_variant(variant)) return 0;
  if (variant != tvfgp::kVariantTwoKernel) return 0;
  return volume_bytes(nx, ny, nz);
}

const char *tv_fgp_status_string(int status) {
  switch (status) {
    case TV_OK: return "ok";
    case TV_ERR_NULL: return "a required pointer is NULL";
    case TV_ERR_DIMS: return "invalid dimensions (< 1 or size overflow)";
    case TV_ERR_ALIAS: return "a written buffer overlaps another buffer";
    case TV_ERR_PARAM: return "invalid parameter (lambda, m or step count)";
    case TV_ERR_WORKSPACE: return "the two-kernel variant needs a z workspace";
    case TV_ERR_VARIANT: return "unknown variant";
    case TV_ERR_LAUNCH: return "the HIP runtime reported a launch error";
    case TV_ERR_ALIGN: return "a pointer is not 4-byte aligned";
    default: return "unknown status";
  }
}

const char *tv_fgp_variant_name(int variant) {
  switch (variant) {
    case tvfgp::kVariantFused: return "fused";
    case tvfgp::kVariantLdsMarch: return "lds_march";
    case tvfgp::kVariantTwoKernel: return "two_kernel";
    case tvfgp::kVariantPoint: return "point";
    case tvfgp::kVariantRegMarch: return "reg_march";
    default: return nullptr;
  }
}

}  // extern "C"
