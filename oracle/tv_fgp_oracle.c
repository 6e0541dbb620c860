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
 * OpenMP splits the outer z loop only.  No loop carries a reduction, so the
 * result does not depend on the number of threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

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
