"""Brute-force fp64 FGP with the forward-difference operator as a matrix.

TEST INFRASTRUCTURE ONLY.  An independent check of the stencil oracle on tiny
volumes (a few hundred voxels).  Nothing here is shared with the C oracle or
with the GPU library.

The forward-difference operator D of "TV solver: the FGP step on the GPU",
section "What one step does" (g_a(i) = z(i) - z(i + e_a), zero at the upper
a-face), is built as a dense (3N x N) matrix by enumerating the voxel pairs it
couples.  The adjoint is then taken as the matrix transpose, L := D^T, instead
of the page's stencil formula, so that a wrong sign, index or boundary in the
stencil oracle's L shows up as a difference.  The iteration is the page's:
primal z = max(b - lam*L r, 0), q = r + D z / (12 lam), p' = q / max(1, |q|)
per voxel, r = p' + m (p' - p).
"""
import numpy as np


def difference_matrix(nx, ny, nz):
    """Dense D: row a*N + i holds +1 at column i and -1 at column i + e_a."""
    n = nx * ny * nz
    d = np.zeros((3 * n, n))

    def flat(x, y, z):
        return x + nx * (y + ny * z)

    for z in range(nz):
        for y in range(ny):
            for x in range(nx):
                i = flat(x, y, z)
                ups = ((x + 1, y, z, x + 1 < nx),
                       (x, y + 1, z, y + 1 < ny),
                       (x, y, z + 1, z + 1 < nz))
                for a, (ux, uy, uz, inside) in enumerate(ups):
                    if inside:
                        d[a * n + i, i] = 1.0
                        d[a * n + i, flat(ux, uy, uz)] = -1.0
    return d


def fista_momentum(k):
    """m_k = (t_k - 1)/t_{k+1}, t_1 = 1, t_{k+1} = (1 + sqrt(1 + 4 t_k^2))/2."""
    t = 1.0
    for _ in range(k - 1):
        t = (1.0 + np.sqrt(1.0 + 4.0 * t * t)) / 2.0
    t_next = (1.0 + np.sqrt(1.0 + 4.0 * t * t)) / 2.0
    return (t - 1.0) / t_next


def run(b, p0, r0, lam, n_outer, n_inner):
    """fp64 FGP on flattened vectors.  b: (nz, ny, nx); p0, r0: (3, nz, ny, nx)."""
    nz, ny, nx = b.shape
    n = b.size
    d = difference_matrix(nx, ny, nz)
    bv = b.astype(np.float64).ravel()
    p = p0.astype(np.float64).reshape(3, n).copy()
    r = r0.astype(np.float64).reshape(3, n).copy()
    for _ in range(n_outer):
        for k in range(1, n_inner + 1):
            m = fista_momentum(k)
            z = np.maximum(bv - lam * (d.T @ r.ravel()), 0.0)
            q = r + (d @ z).reshape(3, n) / (12.0 * lam)
            norm = np.sqrt((q * q).sum(axis=0))
            pn = q / np.maximum(1.0, norm)
            r = pn + m * (pn - p)
            p = pn
    z = np.maximum(bv - lam * (d.T @ p.ravel()), 0.0)
    shape = (3, nz, ny, nx)
    return p.reshape(shape), r.reshape(shape), z.reshape(nz, ny, nx)
