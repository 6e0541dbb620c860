/* Runs every entry point of the CPU oracle (oracle/tv_fgp_oracle.c) on small
 * ragged volumes, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer (test infrastructure: the sanitizers flag any
 * out-of-bounds access, use of freed memory or undefined operation; the
 * results themselves are checked elsewhere).  Prints "ok" and exits 0 when
 * every call returned success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int tv_oracle_run_f32(const float *b, float *p0, float *p1, float *p2, float *r0, float *r1,
                      float *r2, float lam, int n_outer, int n_inner, int64_t nx, int64_t ny,
                      int64_t nz);
int tv_oracle_run_f64(const double *b, double *p0, double *p1, double *p2, double *r0,
                      double *r1, double *r2, double lam, int n_outer, int n_inner, int64_t nx,
                      int64_t ny, int64_t nz);
int tv_oracle_step_f32(const float *b, float *p0, float *p1, float *p2, const float *r0,
                       const float *r1, const float *r2, float *rn0, float *rn1, float *rn2,
                       float lam, float m, int64_t nx, int64_t ny, int64_t nz);
void tv_oracle_adjoint_f32(const float *r0, const float *r1, const float *r2, float *out,
                           int64_t nx, int64_t ny, int64_t nz);
void tv_oracle_gradient_f64(const double *z, double *g0, double *g1, double *g2, int64_t nx,
                            int64_t ny, int64_t nz);
void tv_oracle_primal_readout_f32(const float *b, const float *p0, const float *p1,
                                  const float *p2, float lam, float *z, int64_t nx, int64_t ny,
                                  int64_t nz);
int tv_oracle_duality_gap_f32(const float *b, const float *p0, const float *p1,
                              const float *p2, float lam, int64_t nx, int64_t ny, int64_t nz,
                              double *out);
int tv_oracle_duality_gap_f64(const double *b, const double *p0, const double *p1,
                              const double *p2, double lam, int64_t nx, int64_t ny, int64_t nz,
                              double *out);
int tv_oracle_run_h(const float *b, uint16_t *p0, uint16_t *p1, uint16_t *p2, uint16_t *r0,
                    uint16_t *r1, uint16_t *r2, float lam, int n_outer, int n_inner, int64_t nx,
                    int64_t ny, int64_t nz);
void tv_oracle_f32_to_f16_array(const float *in, uint16_t *out, int64_t n);
void tv_oracle_f16_to_f32_array(const uint16_t *in, float *out, int64_t n);
double tv_oracle_momentum(int k);

static uint64_t state = 12345;
static double uniform(void) { /* xorshift64*, values in [0, 1) */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (double)((state * 2685821657736338717ull) >> 11) / 9007199254740992.0;
}

static int run_shape(int64_t nx, int64_t ny, int64_t nz) {
  const int64_t n = nx * ny * nz;
  /* every array exactly as large as the call needs, so a stray access is
     outside an allocation */
  float *b = malloc(n * sizeof(float)), *z = malloc(n * sizeof(float));
  float *pf[3], *rf[3], *rn[3];
  double *bd = malloc(n * sizeof(double)), *pd[3], *rd[3], *gd[3], out[3];
  uint16_t *ph[3], *rh[3];
  int bad = 0;
  for (int a = 0; a < 3; ++a) {
    pf[a] = calloc(n, sizeof(float));
    rf[a] = calloc(n, sizeof(float));
    rn[a] = malloc(n * sizeof(float));
    pd[a] = calloc(n, sizeof(double));
    rd[a] = calloc(n, sizeof(double));
    gd[a] = malloc(n * sizeof(double));
    ph[a] = malloc(n * sizeof(uint16_t));
    rh[a] = malloc(n * sizeof(uint16_t));
  }
  for (int64_t i = 0; i < n; ++i) {
    b[i] = (float)(0.06 * uniform() - 0.01);
    bd[i] = b[i];
  }
  bad |= tv_oracle_run_f32(b, pf[0], pf[1], pf[2], rf[0], rf[1], rf[2], 0.003f, 2, 3, nx, ny, nz);
  bad |= tv_oracle_run_f64(bd, pd[0], pd[1], pd[2], rd[0], rd[1], rd[2], 0.003, 2, 3, nx, ny, nz);
  bad |= tv_oracle_step_f32(b, pf[0], pf[1], pf[2], rf[0], rf[1], rf[2], rn[0], rn[1], rn[2],
                            0.003f, (float)tv_oracle_momentum(4), nx, ny, nz);
  tv_oracle_adjoint_f32(rn[0], rn[1], rn[2], z, nx, ny, nz);
  tv_oracle_gradient_f64(bd, gd[0], gd[1], gd[2], nx, ny, nz);
  tv_oracle_primal_readout_f32(b, pf[0], pf[1], pf[2], 0.003f, z, nx, ny, nz);
  bad |= tv_oracle_duality_gap_f32(b, pf[0], pf[1], pf[2], 0.003f, nx, ny, nz, out);
  bad |= tv_oracle_duality_gap_f64(bd, pd[0], pd[1], pd[2], 0.003, nx, ny, nz, out);
  for (int a = 0; a < 3; ++a) {
    tv_oracle_f32_to_f16_array(pf[a], ph[a], n);
    tv_oracle_f32_to_f16_array(rf[a], rh[a], n);
  }
  bad |= tv_oracle_run_h(b, ph[0], ph[1], ph[2], rh[0], rh[1], rh[2], 0.003f, 1, 3, nx, ny, nz);
  for (int a = 0; a < 3; ++a) tv_oracle_f16_to_f32_array(ph[a], pf[a], n);
  free(b);
  free(z);
  free(bd);
  for (int a = 0; a < 3; ++a) {
    free(pf[a]);
    free(rf[a]);
    free(rn[a]);
    free(pd[a]);
    free(rd[a]);
    free(gd[a]);
    free(ph[a]);
    free(rh[a]);
  }
  return bad;
}

int main(void) {
  static const int64_t shapes[][3] = {{1, 1, 1}, {2, 1, 1}, {1, 3, 1}, {1, 1, 4}, {5, 7, 3},
                                      {17, 9, 6}, {33, 2, 11}, {64, 8, 5}, {3, 40, 2}};
  for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
    if (run_shape(shapes[s][0], shapes[s][1], shapes[s][2]) != 0) {
      printf("failed %lld %lld %lld\n", (long long)shapes[s][0], (long long)shapes[s][1],
             (long long)shapes[s][2]);
      return 1;
    }
  printf("ok\n");
  return 0;
}
