// C-ABI layer of the FGP library: argument checks, the FISTA momentum
// schedule, the r ping-pong of the inner loop, the convergence-checked solve
// loop, and dispatch to the kernel launchers.  Host code only.  A call that
// fails validation enqueues nothing; only tv_fgp_solve synchronises.
#include "tv_fgp.h"

#include <hip/hip_runtime.h>
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
  size_t bytes;
  size_t align;
  bool written;
};

// Every buffer must be non-null and aligned, and a written buffer may not
// overlap any other buffer.
int check_buffers(const Buf *bufs, int count) {
  for (int k = 0; k < count; ++k)
    if (bufs[k].ptr == nullptr) return TV_ERR_NULL;
  for (int k = 0; k < count; ++k)
    if (((uintptr_t)bufs[k].ptr & (bufs[k].align - 1)) != 0) return TV_ERR_ALIGN;
  for (int k = 0; k < count; ++k) {
    const uintptr_t a = (uintptr_t)bufs[k].ptr;
    if (a > UINTPTR_MAX - bufs[k].bytes) return TV_ERR_DIMS;
    for (int l = k + 1; l < count; ++l) {
      if (!bufs[k].written && !bufs[l].written) continue;
      const uintptr_t c = (uintptr_t)bufs[l].ptr;
      if (a < c + bufs[l].bytes && c < a + bufs[k].bytes) return TV_ERR_ALIAS;
    }
  }
  return TV_OK;
}

Buf vol(const void *p, size_t bytes, bool written) {
  return Buf{p, bytes, sizeof(float), written};
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

int launch_status(int rc) { return rc == 0 ? TV_OK : TV_ERR_LAUNCH; }

// Inner loop of the multi-step-per-pass kernels, for fp32 (T = float) and
// binary16 (T = uint16_t) duals.  The n_outer x n_inner steps run as one
// sequence cut into passes of up to max_group (2 or 3) steps: pass3(p_in,
// p_out, r_in, r_out, m1, m2, m3), pass2(..., m1, m2), each with p
// alternating between the caller's p and the workspace p_ws, and a single
// step single(p, r_in, r_out, m) in place when one step is left.  The
// momentum of a step is m_k for its position k in its outer iteration (the
// sequence restarts at each outer iteration, and p and r carry over), so a
// pass may span two outer iterations and the result is the same as step by
// step.  Threes end in twos rather than a single step where they can
// (200 = 66 x 3 + 2, 10 = 3 + 3 + 2 + 2).  If p ends in the workspace it is
// copied back, unless p_where is given: then *p_where is set to 1 (p is in
// the workspace) or 0.  `where` (0: r_a holds r, 1: r_b) flips after every
// launch.  The callables return 0 on success.
template <typename T, typename Pass3, typename Pass2, typename Single>
int enqueue_grouped(T *const p[3], T *p_ws, T *const r_a[3], T *const r_b[3], int n_outer,
                    int n_inner, size_t vol_bytes, void *stream, int *where, int max_group,
                    Pass3 pass3, Pass2 pass2, Single single, int *p_where = nullptr) {
  const size_t n = vol_bytes / sizeof(T);
  T *const ws[3] = {p_ws, p_ws + n, p_ws + 2 * n};
  T *const *cur = p;
  T *const *alt = ws;
  const int64_t total = (int64_t)n_outer * n_inner;
  double t = 1.0;
  int k_in = 0;  // steps already taken in the current outer iteration
  for (int64_t s = 0; s < total;) {
    const int64_t left = total - s;
    int todo;
    if (max_group >= 3 && (left >= 5 || left == 3))
      todo = 3;
    else
      todo = left >= 2 ? 2 : 1;
    float m[3] = {0.0f, 0.0f, 0.0f};
    for (int q = 0; q < todo; ++q) {
      if (k_in == 0) t = 1.0;  // momentum restarts with each outer iteration
      const double t_next = (1.0 + sqrt(1.0 + 4.0 * t * t)) / 2.0;
      m[q] = (float)((t - 1.0) / t_next);
      t = t_next;
      if (++k_in == n_inner) k_in = 0;
    }
    T *const *in = *where ? r_b : r_a;
    T *const *out = *where ? r_a : r_b;
    int rc;
    if (todo == 1) {
      rc = single(cur, in, out, m[0]);
    } else {
      rc = todo == 3 ? pass3(cur, alt, in, out, m[0], m[1], m[2])
                     : pass2(cur, alt, in, out, m[0], m[1]);
      T *const *tmp = cur;
      cur = alt;
      alt = tmp;
    }
    if (rc != 0) return TV_ERR_LAUNCH;
    *where ^= 1;
    s += todo;
  }
  if (p_where != nullptr) {
    *p_where = cur != p ? 1 : 0;
    return TV_OK;
  }
  if (cur != p) {
    for (int q = 0; q < 3; ++q)
      if (hipMemcpyAsync(p[q], cur[q], vol_bytes, hipMemcpyDeviceToDevice,
                         (hipStream_t)stream) != hipSuccess)
        return TV_ERR_LAUNCH;
  }
  return TV_OK;
}

// enqueue_grouped with passes of at most two steps.
template <typename T, typename Pass, typename Single>
int enqueue_pairs(T *const p[3], T *p_ws, T *const r_a[3], T *const r_b[3], int n_outer,
                  int n_inner, size_t vol_bytes, void *stream, int *where, Pass pass,
                  Single single, int *p_where = nullptr) {
  auto no_pass3 = [](T *const *, T *const *, T *const *, T *const *, float, float, float) {
    return (int)tvfgp::kLaunchFailed;
  };
  return enqueue_grouped<T>(p, p_ws, r_a, r_b, n_outer, n_inner, vol_bytes, stream, where, 2,
                            no_pass3, pass, single, p_where);
}

int enqueue_steps_tb2(const float *b, float *const p[3], float *const r_a[3],
                      float *const r_b[3], float lambda, float c, int n_outer,
                      int n_inner, int64_t nx, int64_t ny, int64_t nz,
                      float *p_ws, size_t bytes, void *stream, int *where, int *p_where) {
  auto pass = [&](float *const *pi, float *const *po, float *const *ri, float *const *ro,
                  float m1, float m2) {
    tvfgp::Step2Args a;
    a.b = b;
    for (int q = 0; q < 3; ++q) {
      a.p_in[q] = pi[q];
      a.p_out[q] = po[q];
      a.r_in[q] = ri[q];
      a.r_out[q] = ro[q];
    }
    a.lam = lambda;
    a.c = c;
    a.m1 = m1;
    a.m2 = m2;
    a.nx = nx;
    a.ny = ny;
    a.nz = nz;
    a.stream = stream;
    return tvfgp::launch_tb2(a);
  };
  auto single = [&](float *const *pc, float *const *ri, float *const *ro, float m) {
    const float *cin[3] = {ri[0], ri[1], ri[2]};
    return tvfgp::launch_step(make_step(b, pc, cin, ro, lambda, c, m, nx, ny, nz,
                                        tvfgp::kVariantFused, nullptr, stream));
  };
  return enqueue_pairs<float>(p, p_ws, r_a, r_b, n_outer, n_inner, bytes, stream, where, pass,
                              single, p_where);
}

int enqueue_steps_tb3(const float *b, float *const p[3], float *const r_a[3],
                      float *const r_b[3], float lambda, float c, int n_outer,
                      int n_inner, int64_t nx, int64_t ny, int64_t nz,
                      float *p_ws, size_t bytes, void *stream, int *where, int *p_where) {
  auto pass3 = [&](float *const *pi, float *const *po, float *const *ri, float *const *ro,
                   float m1, float m2, float m3) {
    tvfgp::Step3Args a;
    a.b = b;
    for (int q = 0; q < 3; ++q) {
      a.p_in[q] = pi[q];
      a.p_out[q] = po[q];
      a.r_in[q] = ri[q];
      a.r_out[q] = ro[q];
    }
    a.lam = lambda;
    a.c = c;
    a.m1 = m1;
    a.m2 = m2;
    a.m3 = m3;
    a.nx = nx;
    a.ny = ny;
    a.nz = nz;
    a.stream = stream;
    return tvfgp::launch_tb3(a);
  };
  auto pass2 = [&](float *const *pi, float *const *po, float *const *ri, float *const *ro,
                   float m1, float m2) {
    tvfgp::Step2Args a;
    a.b = b;
    for (int q = 0; q < 3; ++q) {
      a.p_in[q] = pi[q];
      a.p_out[q] = po[q];
      a.r_in[q] = ri[q];
      a.r_out[q] = ro[q];
    }
    a.lam = lambda;
    a.c = c;
    a.m1 = m1;
    a.m2 = m2;
    a.nx = nx;
    a.ny = ny;
    a.nz = nz;
    a.stream = stream;
    return tvfgp::launch_tb2(a);
  };
  auto single = [&](float *const *pc, float *const *ri, float *const *ro, float m) {
    const float *cin[3] = {ri[0], ri[1], ri[2]};
    return tvfgp::launch_step(make_step(b, pc, cin, ro, lambda, c, m, nx, ny, nz,
                                        tvfgp::kVariantFused, nullptr, stream));
  };
  return enqueue_grouped<float>(p, p_ws, r_a, r_b, n_outer, n_inner, bytes, stream, where, 3,
                                pass3, pass2, single, p_where);
}

// Enqueue n_outer x n_inner steps; `where` (0: r_a holds r, 1: r_b) is
// updated after every step, so the caller learns where the last r is.  With
// p_where given, the multi-step variants leave p where their last pass put
// it and report it (1: the workspace) instead of copying it back.
int enqueue_steps(const float *b, float *const p[3], float *const r_a[3],
                  float *const r_b[3], float lambda, float c, int n_outer,
                  int n_inner, int64_t nx, int64_t ny, int64_t nz, int variant,
                  float *z_ws, void *stream, int *where, int *p_where = nullptr) {
  if (p_where != nullptr) *p_where = 0;
  if (variant == tvfgp::kVariantTb2)
    return enqueue_steps_tb2(b, p, r_a, r_b, lambda, c, n_outer, n_inner, nx, ny, nz, z_ws,
                             volume_bytes(nx, ny, nz), stream, where, p_where);
  if (variant == tvfgp::kVariantTb3)
    return enqueue_steps_tb3(b, p, r_a, r_b, lambda, c, n_outer, n_inner, nx, ny, nz, z_ws,
                             volume_bytes(nx, ny, nz), stream, where, p_where);
  for (int o = 0; o < n_outer; ++o) {
    double t = 1.0;
    for (int k = 1; k <= n_inner; ++k) {
      const double t_next = (1.0 + sqrt(1.0 + 4.0 * t * t)) / 2.0;
      const float m = (float)((t - 1.0) / t_next);
      t = t_next;
      float *const *in = *where ? r_b : r_a;
      float *const *out = *where ? r_a : r_b;
      const float *cin[3] = {in[0], in[1], in[2]};
      const int rc = tvfgp::launch_step(make_step(b, p, cin, out, lambda, c, m,
                                                  nx, ny, nz, variant, z_ws,
                                                  stream));
      if (rc != 0) return TV_ERR_LAUNCH;
      *where ^= 1;
    }
  }
  return TV_OK;
}

// Workspace a run of `variant` needs for volumes of `bytes`: the two-kernel
// variant's z, the two-steps-per-pass variant's second p (three volumes).
size_t run_workspace_bytes(int variant, size_t bytes) {
  if (variant == tvfgp::kVariantTwoKernel) return bytes;
  if (variant == tvfgp::kVariantTb2 || variant == tvfgp::kVariantTb3) return 3 * bytes;
  return 0;
}

size_t gap_ws_bytes(int64_t nx, int64_t ny, int64_t nz) {
  return (size_t)tvfgp::gap_partial_count(nx, ny, nz) * 3 * sizeof(double);
}

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
  if (!known_variant(variant)) return TV_ERR_VARIANT;
  if (p == nullptr || r_in == nullptr || r_out == nullptr) return TV_ERR_NULL;
  const size_t bytes = volume_bytes(nx, ny, nz);
  if (bytes == 0) return TV_ERR_DIMS;
  float c = 0.0f;
  int st = check_lambda(lambda, &c);
  if (st != TV_OK) return st;
  if (!isfinite(m)) return TV_ERR_PARAM;
  const bool two = variant == tvfgp::kVariantTwoKernel;
  if (two && z_ws == nullptr) return TV_ERR_WORKSPACE;
  const Buf bufs[11] = {vol(b, bytes, false),        vol(p[0], bytes, true),
                        vol(p[1], bytes, true),      vol(p[2], bytes, true),
                        vol(r_in[0], bytes, false),  vol(r_in[1], bytes, false),
                        vol(r_in[2], bytes, false),  vol(r_out[0], bytes, true),
                        vol(r_out[1], bytes, true),  vol(r_out[2], bytes, true),
                        vol(z_ws, bytes, true)};
  st = check_buffers(bufs, two ? 11 : 10);
  if (st != TV_OK) return st;
  return launch_status(tvfgp::launch_step(make_step(
      b, p, r_in, r_out, lambda, c, m, nx, ny, nz, variant, z_ws, stream)));
}

int tv_fgp_step_march(const float *b, float *const p[3], const float *const r_in[3],
                      float *const r_out[3], float lambda, float m, int64_t nx, int64_t ny,
                      int64_t nz, int tile_x, int tile_y, int planes, void *stream) {
  if (!tvfgp::march_shape_supported(tile_x, tile_y) || planes < 1 || planes > 1024)
    return TV_ERR_PARAM;
  if (p == nullptr || r_in == nullptr || r_out == nullptr) return TV_ERR_NULL;
  const size_t bytes = volume_bytes(nx, ny, nz);
  if (bytes == 0) return TV_ERR_DIMS;
  float c = 0.0f;
  int st = check_lambda(lambda, &c);
  if (st != TV_OK) return st;
  if (!isfinite(m)) return TV_ERR_PARAM;
  const Buf bufs[10] = {vol(b, bytes, false),        vol(p[0], bytes, true),
                        vol(p[1], bytes, true),      vol(p[2], bytes, true),
                        vol(r_in[0], bytes, false),  vol(r_in[1], bytes, false),
                        vol(r_in[2], bytes, false),  vol(r_out[0], bytes, true),
                        vol(r_out[1], bytes, true),  vol(r_out[2], bytes, true)};
  st = check_buffers(bufs, 10);
  if (st != TV_OK) return st;
  tvfgp::StepArgs a = make_step(b, p, r_in, r_out, lambda, c, m, nx, ny, nz,
                                tvfgp::kVariantLdsMarch, nullptr, stream);
  a.planes = planes;
  return launch_status(tvfgp::launch_lds_march_shape(a, tile_x, tile_y));
}

int tv_fgp_step(const float *b, float *const p[3], const float *const r_in[3],
                float *const r_out[3], float lambda, float m, int64_t nx,
                int64_t ny, int64_t nz, void *stream) {
  return tv_fgp_step_ex(b, p, r_in, r_out, lambda, m, nx, ny, nz,
                        tvfgp::kVariantFused, nullptr, stream);
}

// Checks shared by tv_fgp_run and tv_fgp_solve for the step buffers.
static int check_run(const float *b, float *const p[3], float *const r_a[3],
                     float *const r_b[3], float lambda, int64_t nx, int64_t ny,
                     int64_t nz, int variant, float *z_ws, float *c_out,
                     size_t *bytes_out) {
  if (!known_variant(variant)) return TV_ERR_VARIANT;
  if (p == nullptr || r_a == nullptr || r_b == nullptr) return TV_ERR_NULL;
  const size_t bytes = volume_bytes(nx, ny, nz);
  if (bytes == 0) return TV_ERR_DIMS;
  int st = check_lambda(lambda, c_out);
  if (st != TV_OK) return st;
  const size_t ws = run_workspace_bytes(variant, bytes);
  if (ws != 0 && z_ws == nullptr) return TV_ERR_WORKSPACE;
  const Buf bufs[11] = {vol(b, bytes, false),     vol(p[0], bytes, true),
                        vol(p[1], bytes, true),   vol(p[2], bytes, true),
                        vol(r_a[0], bytes, true), vol(r_a[1], bytes, true),
                        vol(r_a[2], bytes, true), vol(r_b[0], bytes, true),
                        vol(r_b[1], bytes, true), vol(r_b[2], bytes, true),
                        vol(z_ws, ws, true)};
  *bytes_out = bytes;
  return check_buffers(bufs, ws != 0 ? 11 : 10);
}

int tv_fgp_run(const float *b, float *const p[3], float *const r_a[3],
               float *const r_b[3], float lambda, int n_outer, int n_inner,
               int64_t nx, int64_t ny, int64_t nz, int variant, float *z_ws,
               void *stream, int *r_final) {
  if (r_final) *r_final = 0;
  float c = 0.0f;
  size_t bytes = 0;
  int st = check_run(b, p, r_a, r_b, lambda, nx, ny, nz, variant, z_ws, &c, &bytes);
  if (st != TV_OK) return st;
  if (n_outer < 0 || n_inner < 0) return TV_ERR_PARAM;
  int where = 0;
  st = enqueue_steps(b, p, r_a, r_b, lambda, c, n_outer, n_inner, nx, ny, nz,
                     variant, z_ws, stream, &where);
  if (r_final) *r_final = where;
  return st;
}

int tv_fgp_run_pp(const float *b, float *const p[3], float *const r_a[3],
                  float *const r_b[3], float lambda, int n_outer, int n_inner, int64_t nx,
                  int64_t ny, int64_t nz, int variant, float *z_ws, void *stream,
                  int *r_final, int *p_final) {
  if (r_final) *r_final = 0;
  if (p_final) *p_final = 0;
  if (p_final == nullptr) return TV_ERR_NULL;
  float c = 0.0f;
  size_t bytes = 0;
  int st = check_run(b, p, r_a, r_b, lambda, nx, ny, nz, variant, z_ws, &c, &bytes);
  if (st != TV_OK) return st;
  if (n_outer < 0 || n_inner < 0) return TV_ERR_PARAM;
  int where = 0;
  st = enqueue_steps(b, p, r_a, r_b, lambda, c, n_outer, n_inner, nx, ny, nz, variant, z_ws,
                     stream, &where, p_final);
  if (r_final) *r_final = where;
  return st;
}

int tv_fgp_step2(const float *b, const float *const p_in[3], float *const p_out[3],
                 const float *const r_in[3], float *const r_out[3], float lambda,
                 float m1, float m2, int64_t nx, int64_t ny, int64_t nz, void *stream) {
  if (p_in == nullptr || p_out == nullptr || r_in == nullptr || r_out == nullptr)
    return TV_ERR_NULL;
  const size_t bytes = volume_bytes(nx, ny, nz);
  if (bytes == 0) return TV_ERR_DIMS;
  float c = 0.0f;
  int st = check_lambda(lambda, &c);
  if (st != TV_OK) return st;
  if (!isfinite(m1) || !isfinite(m2)) return TV_ERR_PARAM;
  const Buf bufs[13] = {vol(b, bytes, false),        vol(p_in[0], bytes, false),
                        vol(p_in[1], bytes, false),  vol(p_in[2], bytes, false),
                        vol(p_out[0], bytes, true),  vol(p_out[1], bytes, true),
                        vol(p_out[2], bytes, true),  vol(r_in[0], bytes, false),
                        vol(r_in[1], bytes, false),  vol(r_in[2], bytes, false),
                        vol(r_out[0], bytes, true),  vol(r_out[1], bytes, true),
                        vol(r_out[2], bytes, true)};
  st = check_buffers(bufs, 13);
  if (st != TV_OK) return st;
  tvfgp::Step2Args a;
  a.b = b;
  for (int q = 0; q < 3; ++q) {
    a.p_in[q] = p_in[q];
    a.p_out[q] = p_out[q];
    a.r_in[q] = r_in[q];
    a.r_out[q] = r_out[q];
  }
  a.lam = lambda;
  a.c = c;
  a.m1 = m1;
  a.m2 = m2;
  a.nx = nx;
  a.ny = ny;
  a.nz = nz;
  a.stream = stream;
  return launch_status(tvfgp::launch_tb2(a));
}

int tv_fgp_step3(const float *b, const float *const p_in[3], float *const p_out[3],
                 const float *const r_in[3], float *const r_out[3], float lambda,
                 float m1, float m2, float m3, int64_t nx, int64_t ny, int64_t nz,
                 void *stream) {
  if (p_in == nullptr || p_out == nullptr || r_in == nullptr || r_out == nullptr)
    return TV_ERR_NULL;
  const size_t bytes = volume_bytes(nx, ny, nz);
  if (bytes == 0) return TV_ERR_DIMS;
  float c = 0.0f;
  int st = check_lambda(lambda, &c);
  if (st != TV_OK) return st;
  if (!isfinite(m1) || !isfinite(m2) || !isfinite(m3)) return TV_ERR_PARAM;
  const Buf bufs[13] = {vol(b, bytes, false),        vol(p_in[0], bytes, false),
                        vol(p_in[1], bytes, false),  vol(p_in[2], bytes, false),
                        vol(p_out[0], bytes, true),  vol(p_out[1], bytes, true),
                        vol(p_out[2], bytes, true),  vol(r_in[0], bytes, false),
                        vol(r_in[1], bytes, false),  vol(r_in[2], bytes, false),
                        vol(r_out[0], bytes, true),  vol(r_out[1], bytes, true),
                        vol(r_out[2], bytes, true)};
  st = check_buffers(bufs, 13);
  if (st != TV_OK) return st;
  tvfgp::Step3Args a;
  a.b = b;
  for (int q = 0; q < 3; ++q) {
    a.p_in[q] = p_in[q];
    a.p_out[q] = p_out[q];
    a.r_in[q] = r_in[q];
    a.r_out[q] = r_out[q];
  }
  a.lam = lambda;
  a.c = c;
  a.m1 = m1;
  a.m2 = m2;
  a.m3 = m3;
  a.nx = nx;
  a.ny = ny;
  a.nz = nz;
  a.stream = stream;
  return launch_status(tvfgp::launch_tb3(a));
}

int tv_primal(const float *b, const float *const p[3], float *z, float lambda,
              int64_t nx, int64_t ny, int64_t nz, void *stream) {
  if (p == nullptr) return TV_ERR_NULL;
  const size_t bytes = volume_bytes(nx, ny, nz);
  if (bytes == 0) return TV_ERR_DIMS;
  float c = 0.0f;
  int st = check_lambda(lambda, &c);
  if (st != TV_OK) return st;
  const Buf bufs[5] = {vol(b, bytes, false), vol(p[0], bytes, false),
                       vol(p[1], bytes, false), vol(p[2], bytes, false),
                       vol(z, bytes, true)};
  st = check_buffers(bufs, 5);
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

// ---------------------------------------------------------------------------
// dual stored as binary16

static Buf hvol(const void *p, size_t half_bytes, bool written) {
  return Buf{p, half_bytes, sizeof(uint16_t), written};
}

int tv_fgp_step_h(const float *b, uint16_t *const p[3],
                  const uint16_t *const r_in[3], uint16_t *const r_out[3],
                  float lambda, float m, int64_t nx, int64_t ny, int64_t nz,
                  void *stream) {
  if (p == nullptr || r_in == nullptr || r_out == nullptr) return TV_ERR_NULL;
  const size_t bytes = volume_bytes(nx, ny, nz);
  if (bytes == 0) return TV_ERR_DIMS;
  float c = 0.0f;
  int st = check_lambda(lambda, &c);
  if (st != TV_OK) return st;
  if (!isfinite(m)) return TV_ERR_PARAM;
  const size_t hb = bytes / 2;
  const Buf bufs[10] = {vol(b, bytes, false),      hvol(p[0], hb, true),
                        hvol(p[1], hb, true),      hvol(p[2], hb, true),
                        hvol(r_in[0], hb, false),  hvol(r_in[1], hb, false),
                        hvol(r_in[2], hb, false),  hvol(r_out[0], hb, true),
                        hvol(r_out[1], hb, true),  hvol(r_out[2], hb, true)};
  st = check_buffers(bufs, 10);
  if (st != TV_OK) return st;
  tvfgp::StepArgsH h;
  h.b = b;
  for (int k = 0; k < 3; ++k) {
    h.p[k] = p[k];
    h.r_in[k] = r_in[k];
    h.r_out[k] = r_out[k];
  }
  h.lam = lambda;
  h.c = c;
  h.m = m;
  h.nx = nx;
  h.ny = ny;
  h.nz = nz;
  h.stream = stream;
  return launch_status(tvfgp::launch_fused_pair_h(h));
}

int tv_fgp_run_h(const float *b, uint16_t *const p[3], uint16_t *const r_a[3],
                 uint16_t *const r_b[3], float lambda, int n_outer, int n_inner,
                 int64_t nx, int64_t ny, int64_t nz, void *stream, int *r_final) {
  if (r_final) *r_final = 0;
  if (p == nullptr || r_a == nullptr || r_b == nullptr) return TV_ERR_NULL;
  const size_t bytes = volume_bytes(nx, ny, nz);
  if (bytes == 0) return TV_ERR_DIMS;
  float c = 0.0f;
  int st = check_lambda(lambda, &c);
  if (st != TV_OK) return st;
  if (n_outer < 0 || n_inner < 0) return TV_ERR_PARAM;
  const size_t hb = bytes / 2;
  const Buf bufs[10] = {vol(b, bytes, false),   hvol(p[0], hb, true),
                        hvol(p[1], hb, true),   hvol(p[2], hb, true),
                        hvol(r_a[0], hb, true), hvol(r_a[1], hb, true),
                        hvol(r_a[2], hb, true), hvol(r_b[0], hb, true),
                        hvol(r_b[1], hb, true), hvol(r_b[2], hb, true)};
  st = check_buffers(bufs, 10);
  if (st != TV_OK) return st;
  tvfgp::StepArgsH h;
  h.b = b;
  for (int k = 0; k < 3; ++k) h.p[k] = p[k];
  h.lam = lambda;
  h.c = c;
  h.nx = nx;
  h.ny = ny;
  h.nz = nz;
  h.stream = stream;
  int where = 0;
  for (int o = 0; o < n_outer; ++o) {
    double t = 1.0;
    for (int k = 1; k <= n_inner; ++k) {
      const double t_next = (1.0 + sqrt(1.0 + 4.0 * t * t)) / 2.0;
      h.m = (float)((t - 1.0) / t_next);
      t = t_next;
      uint16_t *const *in = where ? r_b : r_a;
      uint16_t *const *out = where ? r_a : r_b;
      for (int a = 0; a < 3; ++a) {
        h.r_in[a] = in[a];
        h.r_out[a] = out[a];
      }
      if (tvfgp::launch_fused_pair_h(h) != 0) return TV_ERR_LAUNCH;
      where ^= 1;
      if (r_final) *r_final = where;
    }
  }
  return TV_OK;
}

int tv_fgp_step2_h(const float *b, const uint16_t *const p_in[3], uint16_t *const p_out[3],
                   const uint16_t *const r_in[3], uint16_t *const r_out[3], float lambda,
                   float m1, float m2, int64_t nx, int64_t ny, int64_t nz, void *stream) {
  if (p_in == nullptr || p_out == nullptr || r_in == nullptr || r_out == nullptr)
    return TV_ERR_NULL;
  const size_t bytes = volume_bytes(nx, ny, nz);
  if (bytes == 0) return TV_ERR_DIMS;
  float c = 0.0f;
  int st = check_lambda(lambda, &c);
  if (st != TV_OK) return st;
  if (!isfinite(m1) || !isfinite(m2)) return TV_ERR_PARAM;
  const size_t hb = bytes / 2;
  const Buf bufs[13] = {vol(b, bytes, false),       hvol(p_in[0], hb, false),
                        hvol(p_in[1], hb, false),   hvol(p_in[2], hb, false),
                        hvol(p_out[0], hb, true),   hvol(p_out[1], hb, true),
                        hvol(p_out[2], hb, true),   hvol(r_in[0], hb, false),
                        hvol(r_in[1], hb, false),   hvol(r_in[2], hb, false),
                        hvol(r_out[0], hb, true),   hvol(r_out[1], hb, true),
                        hvol(r_out[2], hb, true)};
  st = check_buffers(bufs, 13);
  if (st != TV_OK) return st;
  tvfgp::Step2ArgsH a;
  a.b = b;
  for (int q = 0; q < 3; ++q) {
    a.p_in[q] = p_in[q];
    a.p_out[q] = p_out[q];
    a.r_in[q] = r_in[q];
    a.r_out[q] = r_out[q];
  }
  a.lam = lambda;
  a.c = c;
  a.m1 = m1;
  a.m2 = m2;
  a.nx = nx;
  a.ny = ny;
  a.nz = nz;
  a.stream = stream;
  return launch_status(tvfgp::launch_tb2_h(a));
}

int tv_fgp_run2_h(const float *b, uint16_t *const p[3], uint16_t *p_ws,
                  uint16_t *const r_a[3], uint16_t *const r_b[3], float lambda, int n_outer,
                  int n_inner, int64_t nx, int64_t ny, int64_t nz, void *stream,
                  int *r_final) {
  if (r_final) *r_final = 0;
  if (p == nullptr || r_a == nullptr || r_b == nullptr || p_ws == nullptr)
    return TV_ERR_NULL;
  const size_t bytes = volume_bytes(nx, ny, nz);
  if (bytes == 0) return TV_ERR_DIMS;
  float c = 0.0f;
  int st = check_lambda(lambda, &c);
  if (st != TV_OK) return st;
  if (n_outer < 0 || n_inner < 0) return TV_ERR_PARAM;
  const size_t hb = bytes / 2;
  const Buf bufs[11] = {vol(b, bytes, false),   hvol(p[0], hb, true),
                        hvol(p[1], hb, true),   hvol(p[2], hb, true),
                        hvol(r_a[0], hb, true), hvol(r_a[1], hb, true),
                        hvol(r_a[2], hb, true), hvol(r_b[0], hb, true),
                        hvol(r_b[1], hb, true), hvol(r_b[2], hb, true),
                        hvol(p_ws, 3 * hb, true)};
  st = check_buffers(bufs, 11);
  if (st != TV_OK) return st;
  auto pass = [&](uint16_t *const *pi, uint16_t *const *po, uint16_t *const *ri,
                  uint16_t *const *ro, float m1, float m2) {
    tvfgp::Step2ArgsH a;
    a.b = b;
    for (int q = 0; q < 3; ++q) {
      a.p_in[q] = pi[q];
      a.p_out[q] = po[q];
      a.r_in[q] = ri[q];
      a.r_out[q] = ro[q];
    }
    a.lam = lambda;
    a.c = c;
    a.m1 = m1;
    a.m2 = m2;
    a.nx = nx;
    a.ny = ny;
    a.nz = nz;
    a.stream = stream;
    return tvfgp::launch_tb2_h(a);
  };
  auto single = [&](uint16_t *const *pc, uint16_t *const *ri, uint16_t *const *ro, float m) {
    tvfgp::StepArgsH h;
    h.b = b;
    for (int q = 0; q < 3; ++q) {
      h.p[q] = pc[q];
      h.r_in[q] = ri[q];
      h.r_out[q] = ro[q];
    }
    h.lam = lambda;
    h.c = c;
    h.m = m;
    h.nx = nx;
    h.ny = ny;
    h.nz = nz;
    h.stream = stream;
    return tvfgp::launch_fused_pair_h(h);
  };
  int where = 0;
  st = enqueue_pairs<uint16_t>(p, p_ws, r_a, r_b, n_outer, n_inner, hb, stream, &where, pass,
                               single);
  if (r_final) *r_final = where;
  return st;
}

int tv_primal_h(const float *b, const uint16_t *const p[3], float *z, float lambda,
                int64_t nx, int64_t ny, int64_t nz, void *stream) {
  if (p == nullptr) return TV_ERR_NULL;
  const size_t bytes = volume_bytes(nx, ny, nz);
  if (bytes == 0) return TV_ERR_DIMS;
  float c = 0.0f;
  int st = check_lambda(lambda, &c);
  if (st != TV_OK) return st;
  const size_t hb = bytes / 2;
  const Buf bufs[5] = {vol(b, bytes, false), hvol(p[0], hb, false),
                       hvol(p[1], hb, false), hvol(p[2], hb, false),
                       vol(z, bytes, true)};
  st = check_buffers(bufs, 5);
  if (st != TV_OK) return st;
  tvfgp::PrimalArgsH a;
  a.b = b;
  for (int k = 0; k < 3; ++k) a.p[k] = p[k];
  a.z = z;
  a.lam = lambda;
  a.nx = nx;
  a.ny = ny;
  a.nz = nz;
  a.stream = stream;
  return launch_status(tvfgp::launch_primal_h(a));
}

size_t tv_fgp_gap_workspace_bytes(int64_t nx, int64_t ny, int64_t nz) {
  if (volume_bytes(nx, ny, nz) == 0) return 0;
  return gap_ws_bytes(nx, ny, nz);
}

// Checks of the gap buffers; bytes of one volume in *bytes_out.
static int check_gap(const float *b, const float *const p[3], float lambda,
                     int64_t nx, int64_t ny, int64_t nz, double *out,
                     void *workspace, size_t workspace_bytes,
                     const Buf *extra, int n_extra) {
  if (p == nullptr) return TV_ERR_NULL;
  const size_t bytes = volume_bytes(nx, ny, nz);
  if (bytes == 0) return TV_ERR_DIMS;
  float c = 0.0f;
  int st = check_lambda(lambda, &c);
  if (st != TV_OK) return st;
  const size_t ws = gap_ws_bytes(nx, ny, nz);
  if (workspace == nullptr || out == nullptr) return TV_ERR_NULL;
  if (workspace_bytes < ws) return TV_ERR_WORKSPACE;
  Buf bufs[16];
  int n = 0;
  bufs[n++] = vol(b, bytes, false);
  for (int k = 0; k < 3; ++k) bufs[n++] = vol(p[k], bytes, false);
  bufs[n++] = Buf{out, 3 * sizeof(double), sizeof(double), true};
  bufs[n++] = Buf{workspace, ws, sizeof(double), true};
  for (int k = 0; k < n_extra; ++k) bufs[n++] = extra[k];
  return check_buffers(bufs, n);
}

int tv_fgp_duality_gap(const float *b, const float *const p[3], float lambda,
                       int64_t nx, int64_t ny, int64_t nz, double *out,
                       void *workspace, size_t workspace_bytes, void *stream) {
  const int st = check_gap(b, p, lambda, nx, ny, nz, out, workspace,
                           workspace_bytes, nullptr, 0);
  if (st != TV_OK) return st;
  tvfgp::GapArgs a;
  a.b = b;
  for (int k = 0; k < 3; ++k) a.p[k] = p[k];
  a.lam = lambda;
  a.nx = nx;
  a.ny = ny;
  a.nz = nz;
  a.out = out;
  a.partial = (double *)workspace;
  a.stream = stream;
  return launch_status(tvfgp::launch_duality_gap(a));
}

int tv_fgp_duality_gap_noalloc(const float *b, const float *const p[3], float lambda,
                               int64_t nx, int64_t ny, int64_t nz, double *out,
                               void *stream) {
  if (p == nullptr || out == nullptr) return TV_ERR_NULL;
  const size_t bytes = volume_bytes(nx, ny, nz);
  if (bytes == 0) return TV_ERR_DIMS;
  float c = 0.0f;
  int st = check_lambda(lambda, &c);
  if (st != TV_OK) return st;
  if (gap_ws_bytes(nx, ny, nz) > tvfgp::gap_static_capacity_bytes()) return TV_ERR_WORKSPACE;
  const Buf bufs[5] = {vol(b, bytes, false), vol(p[0], bytes, false), vol(p[1], bytes, false),
                       vol(p[2], bytes, false), Buf{out, 3 * sizeof(double), sizeof(double), true}};
  st = check_buffers(bufs, 5);
  if (st != TV_OK) return st;
  tvfgp::GapArgs a;
  a.b = b;
  for (int k = 0; k < 3; ++k) a.p[k] = p[k];
  a.lam = lambda;
  a.nx = nx;
  a.ny = ny;
  a.nz = nz;
  a.out = out;
  a.partial = nullptr;
  a.stream = stream;
  return launch_status(tvfgp::launch_duality_gap_static(a));
}

int tv_fgp_solve(const float *b, float *const p[3], float *const r_a[3],
                 float *const r_b[3], float lambda, int max_outer, int n_inner,
                 double tol, int64_t nx, int64_t ny, int64_t nz, int variant,
                 float *z_ws, void *gap_ws, size_t gap_ws_bytes_given,
                 double *gap_dev, void *stream, int *r_final, int *outer_done,
                 double gap_host[3]) {
  if (r_final) *r_final = 0;
  if (outer_done) *outer_done = 0;
  float c = 0.0f;
  size_t bytes = 0;
  int st = check_run(b, p, r_a, r_b, lambda, nx, ny, nz, variant, z_ws, &c, &bytes);
  if (st != TV_OK) return st;
  if (max_outer < 0 || n_inner < 0 || isnan(tol)) return TV_ERR_PARAM;
  if (gap_host == nullptr) return TV_ERR_NULL;
  // the gap buffers may not overlap anything the steps write
  Buf extra[7];
  int n_extra = 0;
  for (int k = 0; k < 3; ++k) {
    extra[n_extra++] = vol(r_a[k], bytes, true);
    extra[n_extra++] = vol(r_b[k], bytes, true);
  }
  const size_t ws = run_workspace_bytes(variant, bytes);
  if (ws != 0) extra[n_extra++] = vol(z_ws, ws, true);
  st = check_gap(b, p, lambda, nx, ny, nz, gap_dev, gap_ws, gap_ws_bytes_given,
                 extra, n_extra);
  if (st != TV_OK) return st;

  tvfgp::GapArgs g;
  g.b = b;
  for (int k = 0; k < 3; ++k) g.p[k] = p[k];
  g.lam = lambda;
  g.nx = nx;
  g.ny = ny;
  g.nz = nz;
  g.out = gap_dev;
  g.partial = (double *)gap_ws;
  g.stream = stream;
  hipStream_t s = (hipStream_t)stream;
  int where = 0;
  int done = 0;
  for (;;) {
    if (tvfgp::launch_duality_gap(g) != 0) return TV_ERR_LAUNCH;
    if (hipMemcpyAsync(gap_host, gap_dev, 3 * sizeof(double),
                       hipMemcpyDeviceToHost, s) != hipSuccess)
      return TV_ERR_LAUNCH;
    if (hipStreamSynchronize(s) != hipSuccess) return TV_ERR_LAUNCH;
    const double primal = gap_host[2] + (double)lambda * gap_host[1];
    if (done >= max_outer || gap_host[0] <= tol * primal) break;
    st = enqueue_steps(b, p, r_a, r_b, lambda, c, 1, n_inner, nx, ny, nz,
                       variant, z_ws, stream, &where);
    if (st != TV_OK) return st;
    ++done;
    if (r_final) *r_final = where;
    if (outer_done) *outer_done = done;
  }
  return TV_OK;
}

int tv_fgp_stream_probe(const float *const src[7], float *const dst[6], int64_t n,
                        void *stream) {
  if (src == nullptr || dst == nullptr) return TV_ERR_NULL;
  const size_t bytes = volume_bytes(n, 1, 1);
  if (bytes == 0) return TV_ERR_DIMS;
  Buf bufs[13];
  for (int k = 0; k < 7; ++k) bufs[k] = Buf{src[k], bytes, 16, false};
  for (int k = 0; k < 6; ++k) bufs[7 + k] = Buf{dst[k], bytes, 16, true};
  const int st = check_buffers(bufs, 13);
  if (st != TV_OK) return st;
  return launch_status(tvfgp::launch_stream13(src, dst, n, stream));
}

int tv_fgp_stream_probe_ex(const float *const *src, int n_src, float *const *dst, int n_dst,
                           int64_t n, void *stream) {
  if (!tvfgp::stream_shape_supported(n_src, n_dst)) return TV_ERR_PARAM;
  if ((n_src > 0 && src == nullptr) || (n_dst > 0 && dst == nullptr)) return TV_ERR_NULL;
  const size_t bytes = volume_bytes(n, 1, 1);
  if (bytes == 0) return TV_ERR_DIMS;
  Buf bufs[13];
  int count = 0;
  for (int k = 0; k < n_src; ++k) bufs[count++] = Buf{src[k], bytes, 16, false};
  for (int k = 0; k < n_dst; ++k) bufs[count++] = Buf{dst[k], bytes, 16, true};
  const int st = check_buffers(bufs, count);
  if (st != TV_OK) return st;
  return launch_status(tvfgp::launch_stream(src, n_src, dst, n_dst, n, stream));
}

size_t tv_fgp_workspace_bytes(int variant, int64_t nx, int64_t ny, int64_t nz) {
  if (!known_variant(variant)) return 0;
  return run_workspace_bytes(variant, volume_bytes(nx, ny, nz));
}

const char *tv_fgp_status_string(int status) {
  switch (status) {
    case TV_OK: return "ok";
    case TV_ERR_NULL: return "a required pointer is NULL";
    case TV_ERR_DIMS: return "invalid dimensions (< 1 or size overflow)";
    case TV_ERR_ALIAS: return "a written buffer overlaps another buffer";
    case TV_ERR_PARAM: return "invalid parameter (lambda, m, tolerance or step count)";
    case TV_ERR_WORKSPACE: return "missing or too small workspace";
    case TV_ERR_VARIANT: return "unknown variant";
    case TV_ERR_LAUNCH: return "the HIP runtime reported an error";
    case TV_ERR_ALIGN: return "a pointer is not aligned to its element size";
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
    case tvfgp::kVariantPair: return "pair";
    case tvfgp::kVariantTb2: return "tb2";
    case tvfgp::kVariantTb3: return "tb3";
    case tvfgp::kVariantCube: return "cube";
    case tvfgp::kVariantCube32x8x2: return "cube_32x8x2";
    case tvfgp::kVariantCube64x8x1: return "cube_64x8x1";
    case tvfgp::kVariantCube8x8x8: return "cube_8x8x8";
    case tvfgp::kVariantCube32x4x4: return "cube_32x4x4";
    default: return nullptr;
  }
}

}  // extern "C"
