/*
 * Body of the CPU oracle, instantiated once per precision by tv_fgp_oracle.c
 * (REAL = float and REAL = double, FN(name) appends the precision suffix).
 *
 * TEST INFRASTRUCTURE ONLY. See the header of tv_fgp_oracle.c.
 *
 * Layout: every volume is a dense array of nx*ny*nz values, x fastest:
 * voxel (x, y, z) sits at index x + nx*(y + ny*z).  A vector field (the dual
 * p, its momentum copy r, the gradient g) is three such volumes, component 0
 * along x, 1 along y, 2 along z.
 *
 * Boundary reading (the page is silent on it):
 *   - below the lower face, r_a(j - e_a) is taken as 0;
 *   - at the upper face (i_a = n_a - 1) the forward difference g_a is 0.
 * The arithmetic is written out in the order it is evaluated; the file is
 * compiled with -ffp-contract=off so no multiply-add is fused.
 */

/*
 * Adjoint operator.  "TV solver: the FGP step on the GPU", section "What one
 * step does": L(r)(j) is the sum over the three axes a of
 * r_a(j) - r_a(j - e_a).  The per-axis differences are summed as
 * (d_x + d_y) + d_z.
 */
static void FN(tv_oracle_L)(const REAL *r0, const REAL *r1, const REAL *r2,
                            REAL *out, int64_t nx, int64_t ny, int64_t nz)
{
    const int64_t sy = nx, sz = nx * ny;
    int64_t z;
#pragma omp parallel for schedule(static) if (nx * ny * nz >= TV_ORACLE_PAR_MIN)
    for (z = 0; z < nz; ++z) {
        for (int64_t y = 0; y < ny; ++y) {
            for (int64_t x = 0; x < nx; ++x) {
                const int64_t j = x + sy * y + sz * z;
                const REAL below_x = (x > 0) ? r0[j - 1] : (REAL)0;
                const REAL below_y = (y > 0) ? r1[j - sy] : (REAL)0;
                const REAL below_z = (z > 0) ? r2[j - sz] : (REAL)0;
                const REAL dx = r0[j] - below_x;
                const REAL dy = r1[j] - below_y;
                const REAL dz = r2[j] - below_z;
                out[j] = (dx + dy) + dz;
            }
        }
    }
}

/*
 * Forward-difference operator.  "TV solver: the FGP step on the GPU", section
 * "What one step does": g_a = z(i) - z(i + e_a); 0 at the upper a-face.
 */
static void FN(tv_oracle_D)(const REAL *zv, REAL *g0, REAL *g1, REAL *g2,
                            int64_t nx, int64_t ny, int64_t nz)
{
    const int64_t sy = nx, sz = nx * ny;
    int64_t z;
#pragma omp parallel for schedule(static) if (nx * ny * nz >= TV_ORACLE_PAR_MIN)
    for (z = 0; z < nz; ++z) {
        for (int64_t y = 0; y < ny; ++y) {
            for (int64_t x = 0; x < nx; ++x) {
                const int64_t i = x + sy * y + sz * z;
                g0[i] = (x < nx - 1) ? zv[i] - zv[i + 1] : (REAL)0;
                g1[i] = (y < ny - 1) ? zv[i] - zv[i + sy] : (REAL)0;
                g2[i] = (z < nz - 1) ? zv[i] - zv[i + sz] : (REAL)0;
            }
        }
    }
}

/*
 * Nonnegative primal.  "TV solver: the FGP step on the GPU", section "What
 * one step does": z(j) = max(b(j) - lambda*L(r)(j), 0).
 * u = b - (lambda*L) is a multiply followed by a subtract.  max(u, 0) is
 * written (u > 0) ? u : +0, so a NaN or a negative zero gives +0.
 */
static void FN(tv_oracle_primal)(const REAL *b, const REAL *r0, const REAL *r1,
                                 const REAL *r2, REAL lam, REAL *zout,
                                 int64_t nx, int64_t ny, int64_t nz)
{
    const int64_t n = nx * ny * nz;
    int64_t j;
    FN(tv_oracle_L)(r0, r1, r2, zout, nx, ny, nz);
#pragma omp parallel for schedule(static) if (nx * ny * nz >= TV_ORACLE_PAR_MIN)
    for (j = 0; j < n; ++j) {
        const REAL u = b[j] - lam * zout[j];
        zout[j] = (u > (REAL)0) ? u : (REAL)0;
    }
}

/*
 * Dual step, projection and momentum.  "TV solver: the FGP step on the GPU",
 * section "What one step does":
 *   q = r(i) + g/(12 lambda)      with c = 1/(12 lambda) and q_a = r_a + c*g_a
 *   p' = q / max(1, |q|)          |q| the Euclidean norm of the 3-vector
 *   r(i) = p' + m (p' - p(i));  p(i) = p'
 * z is the primal computed from r; p is updated in place, the new momentum
 * copy goes to rn (r itself is left unchanged).
 */
static void FN(tv_oracle_dual_step)(const REAL *zv, REAL *p0, REAL *p1, REAL *p2,
                                    const REAL *r0, const REAL *r1,
                                    const REAL *r2, REAL *rn0, REAL *rn1,
                                    REAL *rn2, REAL c, REAL m,
                                    int64_t nx, int64_t ny, int64_t nz)
{
    const int64_t sy = nx, sz = nx * ny;
    int64_t z;
#pragma omp parallel for schedule(static) if (nx * ny * nz >= TV_ORACLE_PAR_MIN)
    for (z = 0; z < nz; ++z) {
        for (int64_t y = 0; y < ny; ++y) {
            for (int64_t x = 0; x < nx; ++x) {
                const int64_t i = x + sy * y + sz * z;
                const REAL gx = (x < nx - 1) ? zv[i] - zv[i + 1] : (REAL)0;
                const REAL gy = (y < ny - 1) ? zv[i] - zv[i + sy] : (REAL)0;
                const REAL gz = (z < nz - 1) ? zv[i] - zv[i + sz] : (REAL)0;
                const REAL qx = r0[i] + c * gx;
                const REAL qy = r1[i] + c * gy;
                const REAL qz = r2[i] + c * gz;
                const REAL s2 = (qx * qx + qy * qy) + qz * qz;
                const REAL nq = SQRT(s2);
                const REAL s = (nq > (REAL)1) ? nq : (REAL)1;
                const REAL px = qx / s;
                const REAL py = qy / s;
                const REAL pz = qz / s;
                rn0[i] = px + m * (px - p0[i]);
                rn1[i] = py + m * (py - p1[i]);
                rn2[i] = pz + m * (pz - p2[i]);
                p0[i] = px;
                p1[i] = py;
                p2[i] = pz;
            }
        }
    }
}

/* c = 1/(12 lambda), two rounded operations in REAL. */
static REAL FN(tv_oracle_step_size)(REAL lam)
{
    const REAL twelve_lam = (REAL)12 * lam;
    return (REAL)1 / twelve_lam;
}

/*
 * The whole iteration: n_outer outer iterations of n_inner FGP steps.  The
 * momentum sequence restarts (t = 1) at the start of every outer iteration;
 * p and r carry over from one outer iteration to the next.  On return p holds
 * the last projected dual and r the last momentum copy.
 * Returns 0, or -1 if scratch memory could not be allocated.
 */
int FN(tv_oracle_run)(const REAL *b, REAL *p0, REAL *p1, REAL *p2,
                      REAL *r0, REAL *r1, REAL *r2, REAL lam,
                      int n_outer, int n_inner,
                      int64_t nx, int64_t ny, int64_t nz)
{
    const int64_t n = nx * ny * nz;
    const REAL c = FN(tv_oracle_step_size)(lam);
    REAL *zv = (REAL *)malloc((size_t)n * sizeof(REAL));
    REAL *rn = (REAL *)malloc((size_t)n * 3 * sizeof(REAL));
    if (!zv || !rn) {
        free(zv);
        free(rn);
        return -1;
    }
    REAL *rn0 = rn, *rn1 = rn + n, *rn2 = rn + 2 * n;
    for (int o = 0; o < n_outer; ++o) {
        for (int k = 1; k <= n_inner; ++k) {
            const REAL m = (REAL)tv_oracle_momentum(k);
            FN(tv_oracle_primal)(b, r0, r1, r2, lam, zv, nx, ny, nz);
            FN(tv_oracle_dual_step)(zv, p0, p1, p2, r0, r1, r2, rn0, rn1, rn2,
                                    c, m, nx, ny, nz);
            memcpy(r0, rn0, (size_t)n * sizeof(REAL));
            memcpy(r1, rn1, (size_t)n * sizeof(REAL));
            memcpy(r2, rn2, (size_t)n * sizeof(REAL));
        }
    }
    free(zv);
    free(rn);
    return 0;
}

/* Exported single operators, for the self-tests. */
void FN(tv_oracle_adjoint)(const REAL *r0, const REAL *r1, const REAL *r2,
                           REAL *out, int64_t nx, int64_t ny, int64_t nz)
{
    FN(tv_oracle_L)(r0, r1, r2, out, nx, ny, nz);
}

void FN(tv_oracle_gradient)(const REAL *zv, REAL *g0, REAL *g1, REAL *g2,
                            int64_t nx, int64_t ny, int64_t nz)
{
    FN(tv_oracle_D)(zv, g0, g1, g2, nx, ny, nz);
}

/* z = max(b - lambda*L(p), 0): the primal read out from a dual field. */
void FN(tv_oracle_primal_readout)(const REAL *b, const REAL *p0, const REAL *p1,
                                  const REAL *p2, REAL lam, REAL *zout,
                                  int64_t nx, int64_t ny, int64_t nz)
{
    FN(tv_oracle_primal)(b, p0, p1, p2, lam, zout, nx, ny, nz);
}

/* One FGP step with an explicit momentum coefficient (r is read, rn written). */
int FN(tv_oracle_step)(const REAL *b, REAL *p0, REAL *p1, REAL *p2,
                       const REAL *r0, const REAL *r1, const REAL *r2,
                       REAL *rn0, REAL *rn1, REAL *rn2, REAL lam, REAL m,
                       int64_t nx, int64_t ny, int64_t nz)
{
    const int64_t n = nx * ny * nz;
    REAL *zv = (REAL *)malloc((size_t)n * sizeof(REAL));
    if (!zv)
        return -1;
    FN(tv_oracle_primal)(b, r0, r1, r2, lam, zv, nx, ny, nz);
    FN(tv_oracle_dual_step)(zv, p0, p1, p2, r0, r1, r2, rn0, rn1, rn2,
                            FN(tv_oracle_step_size)(lam), m, nx, ny, nz);
    free(zv);
    return 0;
}

/*
 * Duality gap of a dual field p, in the per-voxel form
 *   G(p) = lambda * sum_i ( |g(i)| - g(i).p(i) ),   g = D z,  z = max(b - lambda L(p), 0)
 * with |.| the Euclidean norm of the 3-vector.  For the problem the FGP step
 * solves (minimise 1/2||z - b||^2 + lambda sum_i |(Dz)(i)| over z >= 0) the
 * primal value is P(z) = 1/2||z - b||^2 + lambda sum_i |g(i)| and the dual
 * value d(p) = 1/2||b||^2 - 1/2||z||^2; because z = max(w, 0) with
 * w = b - lambda L(p) satisfies z (z - w) = 0 and <z, L p> = <D z, p> for an
 * admissible p, P(z) - d(p) = <z, z - b> + lambda sum |g| = the form above.
 * Each term is >= 0 when |p(i)| <= 1, so the sum has no cancellation.
 * z and g are computed in REAL exactly as the step does; the per-voxel
 * terms and the sums are in double, without contraction:
 *   norm = sqrt((gx*gx + gy*gy) + gz*gz),  dot = (gx*px + gy*py) + gz*pz.
 * out[0] = G, out[1] = sum_i |g(i)| (total variation of z),
 * out[2] = 1/2 sum_i (z - b)^2.   Returns 0, or -1 if scratch allocation fails.
 */
int FN(tv_oracle_duality_gap)(const REAL *b, const REAL *p0, const REAL *p1,
                              const REAL *p2, REAL lam, int64_t nx, int64_t ny,
                              int64_t nz, double *out)
{
    const int64_t n = nx * ny * nz;
    REAL *zv = (REAL *)malloc((size_t)n * sizeof(REAL));
    REAL *g = (REAL *)malloc((size_t)n * 3 * sizeof(REAL));
    if (!zv || !g) {
        free(zv);
        free(g);
        return -1;
    }
    FN(tv_oracle_primal)(b, p0, p1, p2, lam, zv, nx, ny, nz);
    FN(tv_oracle_D)(zv, g, g + n, g + 2 * n, nx, ny, nz);
    double sum_gap = 0.0, sum_tv = 0.0, sum_fid = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const double gx = (double)g[i], gy = (double)g[n + i], gz = (double)g[2 * n + i];
        const double norm = sqrt((gx * gx + gy * gy) + gz * gz);
        const double dot = (gx * (double)p0[i] + gy * (double)p1[i]) + gz * (double)p2[i];
        const double d = (double)zv[i] - (double)b[i];
        sum_gap += norm - dot;
        sum_tv += norm;
        sum_fid += 0.5 * (d * d);
    }
    out[0] = (double)lam * sum_gap;
    out[1] = sum_tv;
    out[2] = sum_fid;
    free(zv);
    free(g);
    return 0;
}
