/*
 * The C ABI used from plain C, without Python or torch (test infrastructure).
 *
 * Reads b (n floats), p and r (3n floats each) from <dir>, allocates device
 * buffers with the HIP runtime, runs tv_fgp_run (variant from argv),
 * tv_primal and tv_fgp_duality_gap through include/tv_fgp.h, and writes p, r
 * (the buffer r_final names) and z back to <dir>/{p,r,z}_out.bin and the gap
 * triple to <dir>/gap_out.bin (3 doubles).  The caller compares them with
 * the CPU oracle.  Every HIP and library status is checked; any failure
 * prints the call and exits non-zero.
 *
 * usage: fgp_abi_c <dir> <nx> <ny> <nz> <lambda> <n_outer> <n_inner> <variant>
 */
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tv_fgp.h"

#define HIP_OK(call)                                                        \
  do {                                                                      \
    hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));     \
      exit(3);                                                              \
    }                                                                       \
  } while (0)

static float *read_floats(const char *dir, const char *name, size_t n) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "rb");
  float *v = (float *)malloc(n * sizeof(float));
  if (!f || !v || fread(v, sizeof(float), n, f) != n) {
    fprintf(stderr, "cannot read %s\n", path);
    exit(2);
  }
  fclose(f);
  return v;
}

static void write_floats(const char *dir, const char *name, const float *v, size_t n) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "wb");
  if (!f || fwrite(v, sizeof(float), n, f) != n) {
    fprintf(stderr, "cannot write %s\n", path);
    exit(2);
  }
  fclose(f);
}

int main(int argc, char **argv) {
  if (argc != 9) {
    fprintf(stderr, "usage: fgp_abi_c dir nx ny nz lambda n_outer n_inner variant\n");
    return 2;
  }
  const char *dir = argv[1];
  const int64_t nx = atoll(argv[2]), ny = atoll(argv[3]), nz = atoll(argv[4]);
  const float lambda = strtof(argv[5], NULL);
  const int n_outer = atoi(argv[6]), n_inner = atoi(argv[7]), variant = atoi(argv[8]);
  const size_t n = (size_t)(nx * ny * nz), bytes = n * sizeof(float);
  float *hb = read_floats(dir, "b.bin", n);
  float *hp = read_floats(dir, "p.bin", 3 * n);
  float *hr = read_floats(dir, "r.bin", 3 * n);

  float *b, *p, *ra, *rb, *z, *ws = NULL;
  HIP_OK(hipMalloc((void **)&b, bytes));
  HIP_OK(hipMalloc((void **)&p, 3 * bytes));
  HIP_OK(hipMalloc((void **)&ra, 3 * bytes));
  HIP_OK(hipMalloc((void **)&rb, 3 * bytes));
  HIP_OK(hipMalloc((void **)&z, bytes));
  const size_t ws_bytes = tv_fgp_workspace_bytes(variant, nx, ny, nz);
  if (ws_bytes) HIP_OK(hipMalloc((void **)&ws, ws_bytes));
  HIP_OK(hipMemcpy(b, hb, bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(p, hp, 3 * bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(ra, hr, 3 * bytes, hipMemcpyHostToDevice));

  float *const P[3] = {p, p + n, p + 2 * n};
  float *const RA[3] = {ra, ra + n, ra + 2 * n};
  float *const RB[3] = {rb, rb + n, rb + 2 * n};
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  int r_final = -1;
  int st = tv_fgp_run(b, P, RA, RB, lambda, n_outer, n_inner, nx, ny, nz, variant, ws,
                      (void *)stream, &r_final);
  if (st != TV_OK) {
    fprintf(stderr, "tv_fgp_run: %s\n", tv_fgp_status_string(st));
    return 4;
  }
  st = tv_primal(b, (const float *const *)P, z, lambda, nx, ny, nz, (void *)stream);
  if (st != TV_OK) {
    fprintf(stderr, "tv_primal: %s\n", tv_fgp_status_string(st));
    return 4;
  }
  const size_t gap_ws_bytes = tv_fgp_gap_workspace_bytes(nx, ny, nz);
  void *gap_ws = NULL;
  double *gap_dev = NULL, gap[3];
  HIP_OK(hipMalloc(&gap_ws, gap_ws_bytes));
  HIP_OK(hipMalloc((void **)&gap_dev, 3 * sizeof(double)));
  st = tv_fgp_duality_gap(b, (const float *const *)P, lambda, nx, ny, nz, gap_dev, gap_ws,
                          gap_ws_bytes, (void *)stream);
  if (st != TV_OK) {
    fprintf(stderr, "tv_fgp_duality_gap: %s\n", tv_fgp_status_string(st));
    return 4;
  }
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(gap, gap_dev, 3 * sizeof(double), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hp, p, 3 * bytes, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hr, r_final ? rb : ra, 3 * bytes, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hb, z, bytes, hipMemcpyDeviceToHost));
  write_floats(dir, "p_out.bin", hp, 3 * n);
  write_floats(dir, "r_out.bin", hr, 3 * n);
  write_floats(dir, "z_out.bin", hb, n);
  {
    char path[4096];
    snprintf(path, sizeof path, "%s/gap_out.bin", dir);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(gap, sizeof(double), 3, f) != 3) {
      fprintf(stderr, "cannot write %s\n", path);
      exit(2);
    }
    fclose(f);
  }
  HIP_OK(hipStreamDestroy(stream));
  HIP_OK(hipFree(b));
  HIP_OK(hipFree(p));
  HIP_OK(hipFree(ra));
  HIP_OK(hipFree(rb));
  HIP_OK(hipFree(z));
  if (ws) HIP_OK(hipFree(ws));
  HIP_OK(hipFree(gap_ws));
  HIP_OK(hipFree(gap_dev));
  printf("ok %s r_final=%d\n", tv_fgp_variant_name(variant), r_final);
  return 0;
}
