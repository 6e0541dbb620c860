/*
 * tv_fgp.h — C ABI of the MI355X (gfx950) FGP step on the 3D total-variation
 * dual.
 *
 * The operation is the one described on the page "TV solver: the FGP step on
 * the GPU", section "What one step does".  For every voxel i, with b the input
 * volume, r the momentum copy of the dual and p the dual (three components
 * each):
 *     z(j)  = max(b(j) - lambda * L(r)(j), 0),
 *             L(r)(j) = sum over axes a of r_a(j) - r_a(j - e_a)
 *     g_a   = z(i) - z(i + e_a)
 *     q     = r(i) + g / (12 lambda)
 *     p'    = q / max(1, |q|)        (|q|: Euclidean norm of the 3-vector)
 *     r(i)  = p' + m (p' - p(i)),  p(i) = p'
 * Boundary rule (the page does not state one): r_a(j - e_a) is 0 below the
 * lower a-face, and g_a is 0 at the upper a-face.
 *
 * Conventions shared by every entry point:
 *   - All data pointers are DEVICE pointers (memory on the current HIP
 *     device), owned by the caller.  The library never allocates or frees.
 *   - A volume is nx*ny*nz contiguous floats, x fastest: voxel (x, y, z) is at
 *     index x + nx*(y + ny*z).  A vector field is three such volumes passed as
 *     an array of three pointers, component 0 along x, 1 along y, 2 along z.
 *   - Arithmetic is IEEE fp32 with round-to-nearest, no fused multiply-add,
 *     correctly rounded square root and division; every variant evaluates the
 *     same expressions in the same order, so all variants give the same bits.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream).
 *     Calls return as soon as the work is enqueued and do not synchronise
 *     the host (the one exception, tv_fgp_solve, says so).  Results are
 *     valid once the stream has completed.
 *   - Errors are negative status codes (below); nothing is enqueued when a
 *     call fails validation.  No call aborts, throws or prints.  NaN or Inf
 *     in the data is not checked; it propagates.
 *   - Concurrent calls that write the same buffers race; the caller orders
 *     them (same stream, or events).
 */
#ifndef TV_FGP_H
#define TV_FGP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define TV_OK             0
#define TV_ERR_NULL      -1  /* a required pointer is NULL                           */
#define TV_ERR_DIMS      -2  /* a dimension < 1, or nx*ny*nz*4 bytes overflows        */
#define TV_ERR_ALIAS     -3  /* a written buffer overlaps another buffer of the call  */
#define TV_ERR_PARAM     -4  /* lambda <= 0 or not finite, 1/(12 lambda) not finite,
                                m not finite, negative step counts, NaN tolerance    */
#define TV_ERR_WORKSPACE -5  /* a required workspace is missing or too small          */
#define TV_ERR_VARIANT   -6  /* unknown variant                                      */
#define TV_ERR_LAUNCH    -7  /* the HIP runtime reported an error                     */
#define TV_ERR_ALIGN     -8  /* a pointer is not aligned to its element size          */

/* Kernel variants.  All give bit-identical results. */
#define TV_FGP_FUSED      0  /* default: one fused pass; 64x8 x-y tiles march along
                                z, z is computed once per point and exchanged
                                through LDS, r is read through the caches            */
#define TV_FGP_LDS_MARCH  1  /* ablation: 64x4 x-y tiles march along z with two
                                planes of r and of z staged in LDS and three
                                barriers per plane                                   */
#define TV_FGP_TWO_KERNEL 2  /* ablation: a primal kernel writes z to the workspace,
                                a dual kernel reads it (18 volumes per step)         */
#define TV_FGP_POINT      3  /* ablation: one voxel per thread, z recomputed at the
                                voxel and its three upper neighbours                 */
#define TV_FGP_REG_MARCH  4  /* ablation: each thread walks a column along z,
                                carries its own z and r in registers and recomputes
                                z at the +x and +y neighbours                        */
#define TV_FGP_PAIR       5  /* the fused march with two x-adjacent voxels per lane
                                (128x8 tiles, pair loads and stores) where nx is even
                                and every volume is aligned to two elements; the
                                fused kernel otherwise                               */
#define TV_FGP_TB2        6  /* two steps per pass over HBM: the first step runs on
                                the tile grown by one voxel and stays on chip, the
                                second is written (temporal blocking along z; 52 B
                                per voxel per two steps).  Used by tv_fgp_run and
                                tv_fgp_solve, which need a workspace of three
                                volumes for the second p; a single step
                                (tv_fgp_step_ex) runs the fused kernel            */
#define TV_FGP_CUBE       7  /* ablation: the page's shared-memory cube tiling; a
                                workgroup stages b and r of a 16x8x4 cube plus a
                                one-voxel shell in LDS, computes z once for the
                                cube and its upper faces, then updates the cube   */
#define TV_FGP_CUBE_32x8x2 8 /* the same with 32x8x2 cubes (tile-shape sweep)    */
#define TV_FGP_CUBE_64x8x1 9 /* ... 64x8x1 (one plane per cube)                   */
#define TV_FGP_CUBE_8x8x8 10 /* ... 8x8x8                                         */
#define TV_FGP_CUBE_32x4x4 11 /* ... 32x4x4                                       */
#define TV_FGP_TB3        12 /* three steps per pass over HBM: step one runs on the
                                tile grown by two voxels, step two on the tile
                                grown by one, both stay on chip, step three is
                                written (52 B per voxel per three steps).  Used
                                by tv_fgp_run and tv_fgp_solve with a workspace
                                of three volumes, like TV_FGP_TB2; a single step
                                (tv_fgp_step_ex) runs the fused kernel            */

/*
 * One FGP step ("TV solver: the FGP step on the GPU", section "What one step
 * does") with the default fused variant.
 *   b       [in]      volume b (nx*ny*nz floats).
 *   p       [in/out]  the dual, three volumes; overwritten with p'.
 *   r_in    [in]      momentum copy read by the step, three volumes.
 *   r_out   [out]     new momentum copy p' + m (p' - p), three volumes.
 *   lambda  [in]      regularisation weight, finite and > 0; the dual step
 *                     size is c = 1/(12 lambda), rounded in fp32 as
 *                     1.0f / (12.0f * lambda).
 *   m       [in]      momentum coefficient of this step, finite.
 *   nx, ny, nz        dimensions, each >= 1.
 *   stream            hipStream_t to enqueue on.
 * p, r_out must not overlap each other or b, r_in (r_in is still read by
 * neighbouring voxels while r_out is written, hence the two buffers).
 * Returns TV_OK or a negative status.
 */
int tv_fgp_step(const float *b, float *const p[3], const float *const r_in[3],
                float *const r_out[3], float lambda, float m,
                int64_t nx, int64_t ny, int64_t nz, void *stream);

/*
 * tv_fgp_step with an explicit variant (TV_FGP_*).  z_ws is a device buffer
 * of at least tv_fgp_workspace_bytes(variant, ...) bytes; it is required by
 * TV_FGP_TWO_KERNEL (which leaves the primal z of r in it) and ignored
 * (may be NULL) otherwise (TV_FGP_TB2 runs a single step with the fused
 * kernel and needs none here).  Same page and section as tv_fgp_step.
 */
int tv_fgp_step_ex(const float *b, float *const p[3],
                   const float *const r_in[3], float *const r_out[3],
                   float lambda, float m, int64_t nx, int64_t ny, int64_t nz,
                   int variant, float *z_ws, void *stream);

/*
 * One step with the LDS z-marching kernel at a chosen tile shape: the
 * ablation behind the sweep of marching tile shapes on the page "TV solver:
 * the FGP step on the GPU" (section "What made the difference").  A workgroup
 * of tile_x * tile_y threads owns a tile_x x tile_y (x, y) tile and walks
 * `planes` consecutive z planes, staging two planes of r and of z in LDS.
 * Same step, arguments and results as tv_fgp_step (bit for bit).
 *   tile_x, tile_y  32 x 4, 32 x 8, 32 x 16, 64 x 4 or 64 x 8; any other
 *                   shape is TV_ERR_PARAM
 *   planes          planes per tile, 1..1024, else TV_ERR_PARAM
 * The variant TV_FGP_LDS_MARCH is this kernel at 64 x 4 x 8.
 */
int tv_fgp_step_march(const float *b, float *const p[3], const float *const r_in[3],
                      float *const r_out[3], float lambda, float m, int64_t nx, int64_t ny,
                      int64_t nz, int tile_x, int tile_y, int planes, void *stream);

/*
 * The inner loop of the solver: n_outer outer iterations of n_inner FGP
 * steps ("TV solver: the FGP step on the GPU", opening paragraph: an outer
 * iteration runs tv_inner FGP steps).  The momentum sequence is the FISTA
 * one, restarted at every outer iteration:
 *     t_1 = 1,  t_{k+1} = (1 + sqrt(1 + 4 t_k^2)) / 2,
 *     m_k = (t_k - 1) / t_{k+1}   (computed in double, rounded once to fp32)
 * for the k-th step of each outer iteration (m_1 = 0).  p and r carry over
 * between outer iterations.
 *   r_a, r_b  [in/out]  the two momentum buffers; the first step reads r_a.
 *                       After every step the roles swap (with TV_FGP_TB2,
 *                       after every launch, which may run two steps).
 *   r_final   [out]     host pointer, may be NULL; receives 0 if the last
 *                       momentum copy is in r_a, 1 if in r_b.
 * With n_outer * n_inner == 0 nothing is enqueued and *r_final = 0.
 * Other arguments as tv_fgp_step_ex.  p, r_a, r_b and z_ws must not overlap
 * each other or b.
 * TV_FGP_TB2, TV_FGP_TB3: z_ws holds three volumes (tv_fgp_workspace_bytes),
 * used as a second p buffer.  The n_outer * n_inner steps run as one sequence
 * in passes of two (TB2) or of three ending in twos (TB3: 10 = 3+3+2+2,
 * 200 = 66 x 3 + 2), one launch per pass, p alternating between the caller's
 * p and z_ws; a pass may span two outer iterations, each step taking the
 * momentum of its own position; a single step left over runs the fused kernel
 * in place; if p ends in z_ws it is copied back into p on the stream.
 * Results equal those of the other variants bit for bit; only the buffer
 * named by r_final may differ.
 */
int tv_fgp_run(const float *b, float *const p[3], float *const r_a[3],
               float *const r_b[3], float lambda, int n_outer, int n_inner,
               int64_t nx, int64_t ny, int64_t nz, int variant, float *z_ws,
               void *stream, int *r_final);

/*
 * tv_fgp_run without the copy of p back from the workspace: with TV_FGP_TB2
 * and TV_FGP_TB3, p alternates between the caller's p and z_ws from pass to
 * pass, as r alternates between r_a and r_b, and the call reports where the
 * last p is, as it reports r.  Same steps, same bits.
 *   p_final   [out]  host pointer, required: 0 if the last p is in p, 1 if
 *                    it is in z_ws (its three components at z_ws,
 *                    z_ws + nx*ny*nz and z_ws + 2*nx*ny*nz); always 0 for the
 *                    one-step variants, which update p in place.
 * A run of an odd number of multi-step passes (20 steps with TB3: six passes
 * of three and one of two) saves the copy of three volumes that tv_fgp_run
 * makes.  Other arguments, errors and overlap rules as tv_fgp_run.
 */
int tv_fgp_run_pp(const float *b, float *const p[3], float *const r_a[3],
                  float *const r_b[3], float lambda, int n_outer, int n_inner, int64_t nx,
                  int64_t ny, int64_t nz, int variant, float *z_ws, void *stream,
                  int *r_final, int *p_final);

/*
 * Two consecutive FGP steps ("TV solver: the FGP step on the GPU", section
 * "What one step does", applied twice) in one pass over the volumes: the
 * first with momentum m1, the second with m2.  Reads b, p_in and r_in once,
 * writes p_out and r_out once (52 bytes per voxel for two steps).  The result
 * is bit for bit that of tv_fgp_step(m1) followed by tv_fgp_step(m2), with p
 * ending in p_out and the second step's momentum copy in r_out.
 *   p_in  [in]   the dual before the first step (not modified)
 *   p_out [out]  the dual after the second step
 * p_in must be a separate buffer from p_out: the pass reads p_in around each
 * tile while neighbouring tiles write p_out.  No written buffer (p_out,
 * r_out) may overlap any other buffer.  Status codes as tv_fgp_step; m1 and
 * m2 must be finite.
 */
int tv_fgp_step2(const float *b, const float *const p_in[3], float *const p_out[3],
                 const float *const r_in[3], float *const r_out[3], float lambda,
                 float m1, float m2, int64_t nx, int64_t ny, int64_t nz, void *stream);

/*
 * Three consecutive FGP steps ("TV solver: the FGP step on the GPU", section
 * "What one step does", applied three times) in one pass over the volumes,
 * with momenta m1, m2, m3.  Reads b, p_in and r_in once, writes p_out and
 * r_out once (52 bytes per voxel for three steps).  The result is bit for bit
 * that of tv_fgp_step(m1), tv_fgp_step(m2), tv_fgp_step(m3), with p ending in
 * p_out and the third step's momentum copy in r_out.  Arguments, overlap
 * rules and status codes as tv_fgp_step2; m3 must be finite.
 */
int tv_fgp_step3(const float *b, const float *const p_in[3], float *const p_out[3],
                 const float *const r_in[3], float *const r_out[3], float lambda,
                 float m1, float m2, float m3, int64_t nx, int64_t ny, int64_t nz,
                 void *stream);

/*
 * Primal read-out z = max(b - lambda * L(p), 0) from a dual field p, with the
 * same expression and boundary rule as the step ("TV solver: the FGP step on
 * the GPU", section "What one step does", first formula).
 *   z [out] nx*ny*nz floats; must not overlap b or p.
 */
int tv_primal(const float *b, const float *const p[3], float *z, float lambda,
              int64_t nx, int64_t ny, int64_t nz, void *stream);

/*
 * One FGP step with the dual p and its momentum copy r stored as IEEE
 * binary16 (the page "TV solver: the FGP step on the GPU" names a
 * half-precision dual as a way to move fewer bytes, in its closing
 * paragraph; the step itself is the one of section "What one step does").
 * p, r_in, r_out are arrays of nx*ny*nz binary16 values (uint16_t bit
 * patterns, 2-byte aligned); b is float.  Each value of p and r is widened to
 * float exactly, the step is computed in float exactly as tv_fgp_step does,
 * and the new p and r_out are rounded to binary16 (nearest, ties to even).
 * 28 bytes per voxel instead of 52.  The result differs from the float
 * dual; it is not an approximation of tv_fgp_step but its own iteration.
 * Kernel: the two-voxels-per-lane march of TV_FGP_PAIR when nx is even and
 * every volume is 4-byte aligned, the fused one-voxel march otherwise (same
 * bits either way).  Overlap rules and status codes as tv_fgp_step.
 */
int tv_fgp_step_h(const float *b, uint16_t *const p[3],
                  const uint16_t *const r_in[3], uint16_t *const r_out[3],
                  float lambda, float m, int64_t nx, int64_t ny, int64_t nz,
                  void *stream);

/* tv_fgp_run with the binary16 dual of tv_fgp_step_h (same kernel choice). */
int tv_fgp_run_h(const float *b, uint16_t *const p[3], uint16_t *const r_a[3],
                 uint16_t *const r_b[3], float lambda, int n_outer, int n_inner,
                 int64_t nx, int64_t ny, int64_t nz, void *stream, int *r_final);

/*
 * tv_fgp_step2 with the binary16 dual of tv_fgp_step_h: two steps in one
 * pass, each step's p and r rounded to binary16 as tv_fgp_step_h rounds them
 * (the first step's rounded p' and r' feed the second), so the result equals
 * two tv_fgp_step_h calls bit for bit.  p_in and p_out must be separate
 * buffers (the pass reads p_in around each tile while others write p_out).
 * Binary16 volumes 2-byte aligned; status codes as tv_fgp_step2.
 */
int tv_fgp_step2_h(const float *b, const uint16_t *const p_in[3], uint16_t *const p_out[3],
                   const uint16_t *const r_in[3], uint16_t *const r_out[3], float lambda,
                   float m1, float m2, int64_t nx, int64_t ny, int64_t nz, void *stream);

/*
 * tv_fgp_run_h with two steps per pass (tv_fgp_step2_h): the steps of each
 * outer iteration run in pairs, p alternating between p and p_ws, an odd
 * last step runs tv_fgp_step_h's kernel in place, and if p ends in p_ws it is
 * copied back into p on the stream.  p_ws: 3*nx*ny*nz binary16 values (three
 * consecutive volumes), overlapping nothing else.  Results equal
 * tv_fgp_run_h's bit for bit; r_final names the buffer with the last r.
 */
int tv_fgp_run2_h(const float *b, uint16_t *const p[3], uint16_t *p_ws,
                  uint16_t *const r_a[3], uint16_t *const r_b[3], float lambda, int n_outer,
                  int n_inner, int64_t nx, int64_t ny, int64_t nz, void *stream,
                  int *r_final);

/* tv_primal from a binary16 dual: z = max(b - lambda * L(p), 0) in float. */
int tv_primal_h(const float *b, const uint16_t *const p[3], float *z, float lambda,
                int64_t nx, int64_t ny, int64_t nz, void *stream);

/*
 * Bytes of device workspace tv_fgp_duality_gap needs at these dimensions
 * (at most 24 KiB); 0 for invalid dimensions.
 */
size_t tv_fgp_gap_workspace_bytes(int64_t nx, int64_t ny, int64_t nz);

/*
 * Duality gap of a dual field p for the problem the FGP iteration solves
 * (minimise 1/2||z - b||^2 + lambda * sum_i |(Dz)(i)| over z >= 0; the page
 * "TV solver: the FGP step on the GPU", section "What one step does", gives
 * the step).  With z = max(b - lambda L(p), 0) and g = D z computed in fp32
 * exactly as the step computes them, writes to the DEVICE buffer `out`:
 *   out[0] = G = lambda * sum_i (|g(i)| - g(i).p(i))
 *   out[1] = sum_i |g(i)|          (total variation of z)
 *   out[2] = 1/2 sum_i (z(i) - b(i))^2
 * G equals P(z) - d(p), the gap between the primal value
 * P(z) = out[2] + lambda*out[1] and the dual value 1/2||b||^2 - 1/2||z||^2,
 * because z (z - w) = 0 for z = max(w, 0) and <z, L p> = <D z, p> when the
 * upper-face slots of p are zero; each term is >= 0 when |p(i)| <= 1, and
 * G -> 0 as the iteration converges.  Per-voxel terms and sums are fp64; the
 * sum order is fixed, so repeated calls give identical bits.
 *   out        [out] device, 3 doubles, 8-byte aligned.
 *   workspace  [scratch] device, tv_fgp_gap_workspace_bytes(...) bytes,
 *              8-byte aligned; contents on return are unspecified.
 * out and workspace must not overlap each other or b, p.  Enqueued on
 * `stream`, no host synchronisation.
 */
int tv_fgp_duality_gap(const float *b, const float *const p[3], float lambda,
                       int64_t nx, int64_t ny, int64_t nz, double *out,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * tv_fgp_duality_gap for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and the same output bits, with the partial
 * sums kept in a static device array of the library instead of a caller's
 * workspace.  The array holds 3 * 1024 doubles (24 KiB) on each GPU the
 * library runs on, from the first such call on that GPU until the process
 * ends; the reduction never needs more (its first pass runs at most 1024
 * workgroups at any size), and a size that would is TV_ERR_WORKSPACE.  The
 * call allocates and frees nothing.  Its device is the current device, which
 * must be the device of `stream`.  Every call on one GPU shares the array:
 * calls that overlap on one GPU (on different streams, or from different
 * threads) race and give wrong results; calls in stream order are safe.  The
 * first call on a device looks the array up (TV_ERR_LAUNCH if that fails).
 *   out  [out] device, 3 doubles, 8-byte aligned, as tv_fgp_duality_gap.
 * Other arguments, errors and overlap rules as tv_fgp_duality_gap.
 */
int tv_fgp_duality_gap_noalloc(const float *b, const float *const p[3], float lambda,
                               int64_t nx, int64_t ny, int64_t nz, double *out,
                               void *stream);

/*
 * The inner loop with a convergence check: outer iterations of n_inner steps
 * (as tv_fgp_run, momentum restarted per outer iteration) until the duality
 * gap of p satisfies G <= tol * P(z) (tv_fgp_duality_gap), or max_outer outer
 * iterations have run.  The gap is computed before the first iteration and
 * after each one.  THIS CALL SYNCHRONISES `stream`: the gap is copied to the
 * host after each check.
 *   gap_ws, gap_ws_bytes  workspace of tv_fgp_duality_gap
 *   gap_dev     [out] device, 3 doubles (the last gap triple)
 *   r_final     [out] host, may be NULL: 0 if the last r is in r_a, 1 if r_b
 *   outer_done  [out] host, may be NULL: outer iterations run
 *   gap_host    [out] host, 3 doubles: the last gap triple
 * tol < 0 never stops early; tol NaN is TV_ERR_PARAM.  Other arguments and
 * overlap rules as tv_fgp_run and tv_fgp_duality_gap.
 */
int tv_fgp_solve(const float *b, float *const p[3], float *const r_a[3],
                 float *const r_b[3], float lambda, int max_outer, int n_inner,
                 double tol, int64_t nx, int64_t ny, int64_t nz, int variant,
                 float *z_ws, void *gap_ws, size_t gap_ws_bytes, double *gap_dev,
                 void *stream, int *r_final, int *outer_done,
                 double gap_host[3]);

/*
 * Bytes of workspace a run of `variant` needs at these dimensions:
 * nx*ny*nz*4 for TV_FGP_TWO_KERNEL (z), 3*nx*ny*nz*4 for TV_FGP_TB2 and
 * TV_FGP_TB3 (a second p, three consecutive volumes), 0 for the others.  Returns 0 for
 * invalid dimensions or an unknown variant.
 */
size_t tv_fgp_workspace_bytes(int variant, int64_t nx, int64_t ny, int64_t nz);

/*
 * m_k used by tv_fgp_run for the k-th step of an outer iteration (k >= 1),
 * as the fp32 value passed to the kernels; 0 for k < 1.  Host-only.
 */
float tv_fgp_momentum(int k);

/*
 * Measurement helper, not a step: moves the traffic of one fused step as a
 * plain linear stream, so that a step kernel's time can be set against what
 * the part achieves for the same bytes.  The page "TV solver: the FGP step on
 * the GPU" (section "Profiler counters" and its closing paragraph) prices a
 * fused step at 13 volumes, 7 read (b, p, r) and 6 written (p, r).  This call
 * writes dst[k][i] = src[k][i] + src[6][i] for k = 0..5 and i < n, reading
 * every src volume once and writing every dst volume once, with
 * non-temporal 16-byte loads and stores.
 *   src  [in]  7 device volumes of n floats, 16-byte aligned
 *   dst  [out] 6 device volumes of n floats, 16-byte aligned
 *   n    elements per volume, >= 1
 * No dst may overlap any other volume of the call.  Errors: TV_ERR_NULL,
 * TV_ERR_DIMS (n < 1 or n*4 overflows), TV_ERR_ALIGN, TV_ERR_ALIAS,
 * TV_ERR_LAUNCH.  Enqueued on `stream`, no host synchronisation.
 */
int tv_fgp_stream_probe(const float *const src[7], float *const dst[6], int64_t n,
                        void *stream);

/*
 * Measurement helper, not a step: the part's streaming rates for the read and
 * write halves of a step's traffic, beside the 13-volume mix above.  Shapes
 * (n_src, n_dst) and what they write, for i < n:
 *   (7, 6)  dst[k][i] = src[k][i] + src[6][i], k = 0..5 (tv_fgp_stream_probe)
 *   (7, 0)  reads the seven volumes and writes nothing (their sum is dropped)
 *   (0, 6)  dst[k][i] = k, k = 0..5
 *   (1, 1)  dst[0][i] = src[0][i]
 * Every volume is read or written once, with non-temporal 16-byte loads and
 * stores.  src holds n_src device pointers (may be NULL when n_src = 0), dst
 * holds n_dst (may be NULL when n_dst = 0); each volume is n floats, 16-byte
 * aligned; no dst may overlap any other volume of the call.  Errors:
 * TV_ERR_PARAM (another shape), TV_ERR_NULL, TV_ERR_DIMS (n < 1 or n*4
 * overflows), TV_ERR_ALIGN, TV_ERR_ALIAS, TV_ERR_LAUNCH.  Enqueued on
 * `stream`, no host synchronisation.
 */
int tv_fgp_stream_probe_ex(const float *const *src, int n_src, float *const *dst, int n_dst,
                           int64_t n, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *tv_fgp_status_string(int status);

/* Static name of a variant: "fused", "lds_march", "two_kernel", "point",
   "reg_march", "pair", "tb2", "cube", "cube_32x8x2", "cube_64x8x1",
   "cube_8x8x8", "cube_32x4x4", "tb3" for TV_FGP_FUSED .. TV_FGP_TB3; NULL
   for any other value.  Host-only. */
const char *tv_fgp_variant_name(int variant);

#ifdef __cplusplus
}
#endif

#endif /* TV_FGP_H */
