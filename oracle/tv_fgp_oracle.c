/*
 * CPU oracle of the FGP step on the 3D total-variation dual.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow reference the GPU
 * path is checked against.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load it; the product path never calls it, and it
 * shares no code, header or constant with the GPU library.
 *
 * What it computes follows the page "TV solver: the FGP step on the GPU",
 * section "What one step does".  Every step is written out loop by loop in
 * the order of that section: the primal z from the momentum copy r, the
 * forward differences of z, the dual step, the projection onto the unit
 * ball, the momentum update.  The body is compiled twice, for float (the
 * parity oracle, exact evaluation order) and for double (the accuracy
 * reference).  Build with -O2 -ffp-contract=off and no fast-math so that
 * each operation is one IEEE-754 round-to-nearest operation.
 *
 * OpenMP splits the outer z loop only, and only on volumes of at least
 * TV_ORACLE_PAR_MIN voxels (on smaller ones starting the threads costs more
 * than the loop).  No loop carries a reduction, so the result does not depend
 * on the number of threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define TV_ORACLE_PAR_MIN ((int64_t)1 << 15)

/*
 * Momentum coefficient of the k-th step of an outer iteration (k >= 1).
 * The page names the coefficient m of the update r = p' + m (p' - p) but not
 * its sequence; the reading taken is the FISTA sequence of Beck and Teboulle
 * that the fast gradient projection uses:
 *   t_1 = 1,  t_{k+1} = (1 + sqrt(1 + 4 t_k^2)) / 2,  m_k = (t_k - 1) / t_{k+1}.
 * Evaluated in double; callers round the result once to their precision.
 */
double tv_oracle_momentum(int k)
{
    double t = 1.0;
    double t_next = 1.0;
    if (k < 1)
        return 0.0;
    for (int s = 1; s <= k; ++s) {
        t_next = (1.0 + sqrt(1.0 + 4.0 * t * t)) / 2.0;
        if (s < k)
            t = t_next;
    }
    return (t - 1.0) / t_next;
}

void tv_oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int tv_oracle_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * IEEE-754 binary16 storage for the half-precision dual.  Conversions written
 * from the format's definition: binary16 has 1 sign bit, 5 exponent bits
 * (bias 15) and 10 fraction bits; its subnormals are k * 2^-24.
 */

/* binary16 -> binary32: exact. */
float tv_oracle_f16_to_f32(uint16_t h)
{
    const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    const uint32_t e = (h >> 10) & 0x1Fu;
    const uint32_t f = h & 0x3FFu;
    uint32_t bits;
    float out;
    if (e == 0) {
        /* zero or subnormal: f * 2^-24, exact in binary32 */
        out = (float)f * (1.0f / 16777216.0f);
        return (h & 0x8000u) ? -out : out;
    }
    if (e == 31)
        bits = sign | 0x7F800000u | (f << 13);
    else
        bits = sign | ((e - 15u + 127u) << 23) | (f << 13);
    memcpy(&out, &bits, sizeof out);
    return out;
}

/*
 * binary32 -> binary16, round to nearest, ties to even.  |v| is written as
 * m * 2^(E-150) with a 24-bit m; the binary16 quantum at that magnitude is
 * 2^(max(E-127, -14) - 10); the quotient is rounded half-to-even, and a carry
 * into the next binade or past the largest finite value (to infinity) falls
 * out of adding it to the exponent field.  NaN gives the quiet NaN 0x7E00
 * with the input's sign.
 */
uint16_t tv_oracle_f32_to_f16(float v)
{
    uint32_t x;
    memcpy(&x, &v, sizeof x);
    const uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    const int e = (int)((x >> 23) & 0xFFu);
    uint32_t m = x & 0x7FFFFFu;
    if (e == 255)
        return (uint16_t)(sign | (m ? 0x7E00u : 0x7C00u));
    if (e != 0)
        m |= 0x800000u;
    const int e_unb = (e == 0) ? -126 : e - 127;
    const int q_exp = (e_unb > -14 ? e_unb : -14) - 10;  /* quantum 2^q_exp */
    const int value_exp = (e == 0) ? -149 : e - 150;     /* |v| = m * 2^value_exp */
    const int sh = q_exp - value_exp;                      /* >= 13 */
    uint32_t k;
    if (sh >= 32) {
        k = 0;
    } else {
        k = m >> sh;
        const uint32_t rem = m & ((1u << sh) - 1u);
        const uint32_t half = 1u << (sh - 1);
        if (rem > half || (rem == half && (k & 1u)))
            k += 1;
    }
    uint32_t bits;
    if (e_unb < -14) {
        bits = k;                               /* subnormal; k == 1024 is 2^-14 */
    } else {
        const uint32_t eb = (uint32_t)(e_unb + 15);
        if (eb >= 31)
            return (uint16_t)(sign | 0x7C00u);
        bits = (eb << 10) + (k - 1024u);        /* k == 2048 carries into eb + 1 */
    }
    if (bits >= 0x7C00u)
        bits = 0x7C00u;
    return (uint16_t)(sign | bits);
}

void tv_oracle_f32_to_f16_array(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = tv_oracle_f32_to_f16(in[i]);
}

void tv_oracle_f16_to_f32_array(const uint16_t *in, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = tv_oracle_f16_to_f32(in[i]);
}

#define REAL float
#define SQRT sqrtf
#define FN(name) name##_f32
#include "tv_fgp_oracle_body.h"
#undef REAL
#undef SQRT
#undef FN

#define REAL double
#define SQRT sqrt
#define FN(name) name##_f64
#include "tv_fgp_oracle_body.h"
#undef REAL
#undef SQRT
#undef FN

/*
 * FGP with the dual p and its momentum copy r stored in binary16, b in
 * binary32, arithmetic in binary32: every step widens p and r exactly, runs
 * the binary32 step (same code as tv_oracle_run_f32), and rounds the new p
 * and r to binary16 (nearest, ties to even).  The conversions are element by
 * element, so splitting them over threads does not change the result.
 */
int tv_oracle_run_h(const float *b, uint16_t *p0, uint16_t *p1, uint16_t *p2,
                    uint16_t *r0, uint16_t *r1, uint16_t *r2, float lam,
                    int n_outer, int n_inner, int64_t nx, int64_t ny, int64_t nz)
{
    const int64_t n = nx * ny * nz;
    uint16_t *ph[3] = {p0, p1, p2};
    uint16_t *rh[3] = {r0, r1, r2};
    float *buf = (float *)malloc((size_t)n * 9 * sizeof(float));
    if (!buf)
        return -1;
    float *pf[3] = {buf, buf + n, buf + 2 * n};
    float *rf[3] = {buf + 3 * n, buf + 4 * n, buf + 5 * n};
    float *rn[3] = {buf + 6 * n, buf + 7 * n, buf + 8 * n};
    for (int o = 0; o < n_outer; ++o) {
        for (int k = 1; k <= n_inner; ++k) {
            const float m = (float)tv_oracle_momentum(k);
            for (int a = 0; a < 3; ++a) {
#pragma omp parallel for schedule(static) if (n >= TV_ORACLE_PAR_MIN)
                for (int64_t i = 0; i < n; ++i) {
                    pf[a][i] = tv_oracle_f16_to_f32(ph[a][i]);
                    rf[a][i] = tv_oracle_f16_to_f32(rh[a][i]);
                }
            }
            if (tv_oracle_step_f32(b, pf[0], pf[1], pf[2], rf[0], rf[1], rf[2],
                                   rn[0], rn[1], rn[2], lam, m, nx, ny, nz) != 0) {
                free(buf);
                return -1;
            }
            for (int a = 0; a < 3; ++a) {
#pragma omp parallel for schedule(static) if (n >= TV_ORACLE_PAR_MIN)
                for (int64_t i = 0; i < n; ++i) {
                    ph[a][i] = tv_oracle_f32_to_f16(pf[a][i]);
                    rh[a][i] = tv_oracle_f32_to_f16(rn[a][i]);
                }
            }
        }
    }
    free(buf);
    return 0;
}
