"""ctypes binding of libtvfgp.so (the C ABI declared in include/tv_fgp.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  torch tensors supply device memory and the
stream; their data pointers are passed through unchanged.  There is no CPU
fallback: importing this module fails if the library has not been built.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtvfgp.so")

TV_OK = 0
TV_ERR_NULL = -1
TV_ERR_DIMS = -2
TV_ERR_ALIAS = -3
TV_ERR_PARAM = -4
TV_ERR_WORKSPACE = -5
TV_ERR_VARIANT = -6
TV_ERR_LAUNCH = -7
TV_ERR_ALIGN = -8

FUSED = 0
LDS_MARCH = 1
TWO_KERNEL = 2
POINT = 3
REG_MARCH = 4
PAIR = 5
TB2 = 6
CUBE = 7
TB3 = 12
VARIANTS = {"fused": FUSED, "lds_march": LDS_MARCH, "two_kernel": TWO_KERNEL,
            "point": POINT, "reg_march": REG_MARCH, "pair": PAIR,
            "tb2": TB2, "cube": CUBE, "cube_32x8x2": 8, "cube_64x8x1": 9, "cube_8x8x8": 10,
            "cube_32x4x4": 11, "tb3": TB3}

# Names declared in include/tv_fgp.h, in declaration order.
EXPORTS = ("tv_fgp_step", "tv_fgp_step_ex", "tv_fgp_step_march", "tv_fgp_run", "tv_fgp_run_pp", "tv_fgp_step2", "tv_fgp_step3",
           "tv_primal",
           "tv_fgp_step_h", "tv_fgp_run_h", "tv_fgp_step2_h", "tv_fgp_run2_h", "tv_primal_h", "tv_fgp_gap_workspace_bytes", "tv_fgp_duality_gap",
           "tv_fgp_duality_gap_noalloc", "tv_fgp_solve",
           "tv_fgp_workspace_bytes", "tv_fgp_momentum", "tv_fgp_stream_probe",
           "tv_fgp_stream_probe_ex", "tv_fgp_status_string", "tv_fgp_variant_name")


class TvFgpError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (where, status_string(status), status))


def _load():
    # torch ships its own HIP runtime.  Import it first so that the library's
    # dependency on libamdhip64.so.7 resolves (by SONAME) to the runtime torch
    # already loaded; loading the library first would bring a second HIP and
    # HSA runtime into the process, and torch's streams and allocations would
    # then be handed to a runtime that does not know them.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libtvfgp.so is not built (expected at %s); run "
            "`python -c 'import __graft_entry__ as g; g.build()'` or "
            "`python stencil_dual_update_amd/build_lib.py`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    _check_single_runtime()
    P = ctypes.c_void_p
    P3 = ctypes.POINTER(ctypes.c_void_p)  # float *const x[3]; NULL allowed
    I64 = ctypes.c_int64
    F = ctypes.c_float
    lib.tv_fgp_step.restype = ctypes.c_int
    lib.tv_fgp_step.argtypes = [P, P3, P3, P3, F, F, I64, I64, I64, P]
    lib.tv_fgp_step_ex.restype = ctypes.c_int
    lib.tv_fgp_step_ex.argtypes = [P, P3, P3, P3, F, F, I64, I64, I64,
                                   ctypes.c_int, P, P]
    lib.tv_fgp_step_march.restype = ctypes.c_int
    lib.tv_fgp_step_march.argtypes = [P, P3, P3, P3, F, F, I64, I64, I64, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, P]
    lib.tv_fgp_run.restype = ctypes.c_int
    lib.tv_fgp_run.argtypes = [P, P3, P3, P3, F, ctypes.c_int, ctypes.c_int,
                               I64, I64, I64, ctypes.c_int, P, P,
                               ctypes.POINTER(ctypes.c_int)]
    lib.tv_fgp_run_pp.restype = ctypes.c_int
    lib.tv_fgp_run_pp.argtypes = [P, P3, P3, P3, F, ctypes.c_int, ctypes.c_int,
                                  I64, I64, I64, ctypes.c_int, P, P,
                                  ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    lib.tv_fgp_step2.restype = ctypes.c_int
    lib.tv_fgp_step2.argtypes = [P, P3, P3, P3, P3, F, F, F, I64, I64, I64, P]
    lib.tv_fgp_step3.restype = ctypes.c_int
    lib.tv_fgp_step3.argtypes = [P, P3, P3, P3, P3, F, F, F, F, I64, I64, I64, P]
    lib.tv_primal.restype = ctypes.c_int
    lib.tv_primal.argtypes = [P, P3, P, F, I64, I64, I64, P]
    lib.tv_fgp_step_h.restype = ctypes.c_int
    lib.tv_fgp_step_h.argtypes = [P, P3, P3, P3, F, F, I64, I64, I64, P]
    lib.tv_fgp_run_h.restype = ctypes.c_int
    lib.tv_fgp_run_h.argtypes = [P, P3, P3, P3, F, ctypes.c_int, ctypes.c_int, I64, I64, I64,
                                 P, ctypes.POINTER(ctypes.c_int)]
    lib.tv_fgp_step2_h.restype = ctypes.c_int
    lib.tv_fgp_step2_h.argtypes = [P, P3, P3, P3, P3, F, F, F, I64, I64, I64, P]
    lib.tv_fgp_run2_h.restype = ctypes.c_int
    lib.tv_fgp_run2_h.argtypes = [P, P3, P, P3, P3, F, ctypes.c_int, ctypes.c_int, I64, I64, I64,
                                  P, ctypes.POINTER(ctypes.c_int)]
    lib.tv_primal_h.restype = ctypes.c_int
    lib.tv_primal_h.argtypes = [P, P3, P, F, I64, I64, I64, P]
    lib.tv_fgp_gap_workspace_bytes.restype = ctypes.c_size_t
    lib.tv_fgp_gap_workspace_bytes.argtypes = [I64, I64, I64]
    lib.tv_fgp_duality_gap.restype = ctypes.c_int
    lib.tv_fgp_duality_gap.argtypes = [P, P3, F, I64, I64, I64, P, P, ctypes.c_size_t, P]
    lib.tv_fgp_duality_gap_noalloc.restype = ctypes.c_int
    lib.tv_fgp_duality_gap_noalloc.argtypes = [P, P3, F, I64, I64, I64, P, P]
    lib.tv_fgp_solve.restype = ctypes.c_int
    lib.tv_fgp_solve.argtypes = [P, P3, P3, P3, F, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                 I64, I64, I64, ctypes.c_int, P, P, ctypes.c_size_t, P, P,
                                 ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                 ctypes.POINTER(ctypes.c_double)]
    lib.tv_fgp_workspace_bytes.restype = ctypes.c_size_t
    lib.tv_fgp_workspace_bytes.argtypes = [ctypes.c_int, I64, I64, I64]
    lib.tv_fgp_momentum.restype = ctypes.c_float
    lib.tv_fgp_momentum.argtypes = [ctypes.c_int]
    lib.tv_fgp_stream_probe.restype = ctypes.c_int
    lib.tv_fgp_stream_probe.argtypes = [P3, P3, I64, P]
    lib.tv_fgp_stream_probe_ex.restype = ctypes.c_int
    lib.tv_fgp_stream_probe_ex.argtypes = [P, ctypes.c_int, P, ctypes.c_int, I64, P]
    lib.tv_fgp_status_string.restype = ctypes.c_char_p
    lib.tv_fgp_status_string.argtypes = [ctypes.c_int]
    lib.tv_fgp_variant_name.restype = ctypes.c_char_p
    lib.tv_fgp_variant_name.argtypes = [ctypes.c_int]
    return lib


def _check_single_runtime():
    """Fail loudly if two different HIP runtimes are mapped into the process."""
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return
    real = {os.path.realpath(p) for p in paths if p.startswith("/")}
    if len(real) > 1:
        raise ImportError("two HIP runtimes are loaded (%s); import torch before "
                          "loading libtvfgp.so" % ", ".join(sorted(real)))


lib = _load()


def status_string(status):
    return lib.tv_fgp_status_string(int(status)).decode()


def variant_name(variant):
    s = lib.tv_fgp_variant_name(int(variant))
    return None if s is None else s.decode()


def momentum(k):
    """m_k as the fp32 value the library passes to its kernels."""
    return float(lib.tv_fgp_momentum(int(k)))


def workspace_bytes(variant, nx, ny, nz):
    return int(lib.tv_fgp_workspace_bytes(int(variant), nx, ny, nz))


def gap_workspace_bytes(nx, ny, nz):
    return int(lib.tv_fgp_gap_workspace_bytes(nx, ny, nz))


# --------------------------------------------------------------------------
# marshalling helpers

def _addr(t):
    """Device address of a tensor (or a raw integer address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _check_volume(t, shape, what):
    if t is None or isinstance(t, int):
        return
    import torch
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % what)
    if t.dtype != torch.float32:
        raise ValueError("%s must be float32" % what)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % what)
    if tuple(t.shape) != shape:
        raise ValueError("%s has shape %s, expected %s" % (what, tuple(t.shape), shape))


def _check_ws(t, shape, variant, what="z_ws"):
    """The run workspace: one volume, or three (a (3, nz, ny, nx) tensor) for TB2 and TB3."""
    if variant in (TB2, TB3) and t is not None and not isinstance(t, int):
        _check_volume(t, (3,) + shape, what)
    else:
        _check_volume(t, shape, what)


def _check_half(t, shape, what):
    if t is None or isinstance(t, int):
        return
    import torch
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous device tensor" % what)
    if t.dtype not in (torch.float16, torch.int16):
        raise ValueError("%s must hold binary16 values (float16 or int16 bit patterns)" % what)
    if tuple(t.shape) != shape:
        raise ValueError("%s has shape %s, expected %s" % (what, tuple(t.shape), shape))


def _hfield(f, shape, what):
    if f is None:
        return (ctypes.c_void_p * 3)(None, None, None)
    comps = [f[0], f[1], f[2]] if not isinstance(f, (list, tuple)) else list(f)
    if len(comps) != 3:
        raise ValueError("%s needs three components" % what)
    for a, c in enumerate(comps):
        _check_half(c, shape, "%s[%d]" % (what, a))
    return (ctypes.c_void_p * 3)(*[_addr(c) for c in comps])


def _field(f, shape, what):
    """Three component addresses of a vector field.

    ``f`` is a (3, nz, ny, nx) tensor, a sequence of three (nz, ny, nx)
    tensors, or a sequence of three raw addresses.
    """
    if f is None:
        return (ctypes.c_void_p * 3)(None, None, None)
    comps = [f[0], f[1], f[2]] if not isinstance(f, (list, tuple)) else list(f)
    if len(comps) != 3:
        raise ValueError("%s needs three components" % what)
    for a, c in enumerate(comps):
        _check_volume(c, shape, "%s[%d]" % (what, a))
    return (ctypes.c_void_p * 3)(*[_addr(c) for c in comps])


def _dims_of(b, dims):
    if dims is not None:
        nx, ny, nz = dims
        return int(nx), int(ny), int(nz)
    nz, ny, nx = b.shape
    return int(nx), int(ny), int(nz)


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _raise(status, where):
    if status != TV_OK:
        raise TvFgpError(status, where)


# --------------------------------------------------------------------------
# entry points (same names as the C ABI)

def tv_fgp_step(b, p, r_in, r_out, lam, m, variant=FUSED, z_ws=None,
                stream=None, dims=None):
    """One FGP step; p is updated in place, the new momentum copy goes to r_out."""
    nx, ny, nz = _dims_of(b, dims)
    shape = (nz, ny, nx)
    _check_volume(b, shape, "b")
    _check_volume(z_ws, shape, "z_ws")
    st = lib.tv_fgp_step_ex(_addr(b), _field(p, shape, "p"),
                            _field(r_in, shape, "r_in"),
                            _field(r_out, shape, "r_out"), float(lam), float(m),
                            nx, ny, nz, int(variant), _addr(z_ws), _stream(stream))
    _raise(st, "tv_fgp_step")


MARCH_SHAPES = ((32, 4), (32, 8), (32, 16), (64, 4), (64, 8))


def tv_fgp_step_march(b, p, r_in, r_out, lam, m, tile_x, tile_y, planes, stream=None,
                      dims=None):
    """One step with the LDS z-march kernel on tile_x x tile_y tiles of `planes` planes."""
    nx, ny, nz = _dims_of(b, dims)
    shape = (nz, ny, nx)
    _check_volume(b, shape, "b")
    st = lib.tv_fgp_step_march(_addr(b), _field(p, shape, "p"), _field(r_in, shape, "r_in"),
                               _field(r_out, shape, "r_out"), float(lam), float(m), nx, ny, nz,
                               int(tile_x), int(tile_y), int(planes), _stream(stream))
    _raise(st, "tv_fgp_step_march")


def tv_fgp_run(b, p, r_a, r_b, lam, n_outer, n_inner, variant=FUSED, z_ws=None,
               stream=None, dims=None):
    """n_outer x n_inner FGP steps; returns 0 if the last r is in r_a, 1 if in r_b."""
    nx, ny, nz = _dims_of(b, dims)
    shape = (nz, ny, nx)
    _check_volume(b, shape, "b")
    _check_ws(z_ws, shape, variant)
    where = ctypes.c_int(-1)
    st = lib.tv_fgp_run(_addr(b), _field(p, shape, "p"), _field(r_a, shape, "r_a"),
                        _field(r_b, shape, "r_b"), float(lam), int(n_outer),
                        int(n_inner), nx, ny, nz, int(variant), _addr(z_ws),
                        _stream(stream), ctypes.byref(where))
    _raise(st, "tv_fgp_run")
    return where.value


def tv_fgp_run_pp(b, p, r_a, r_b, lam, n_outer, n_inner, variant=FUSED, z_ws=None,
                  stream=None, dims=None):
    """tv_fgp_run without copying p back: returns (r_final, p_final), p_final 1
    if the last p is in z_ws (its three volumes), 0 if in p."""
    nx, ny, nz = _dims_of(b, dims)
    shape = (nz, ny, nx)
    _check_volume(b, shape, "b")
    _check_ws(z_ws, shape, variant)
    where = ctypes.c_int(-1)
    pwhere = ctypes.c_int(-1)
    st = lib.tv_fgp_run_pp(_addr(b), _field(p, shape, "p"), _field(r_a, shape, "r_a"),
                           _field(r_b, shape, "r_b"), float(lam), int(n_outer),
                           int(n_inner), nx, ny, nz, int(variant), _addr(z_ws),
                           _stream(stream), ctypes.byref(where), ctypes.byref(pwhere))
    _raise(st, "tv_fgp_run_pp")
    return where.value, pwhere.value


def tv_fgp_step2(b, p_in, p_out, r_in, r_out, lam, m1, m2, stream=None, dims=None):
    """Two FGP steps (momentum m1, then m2) in one pass: p_in -> p_out, r_in -> r_out."""
    nx, ny, nz = _dims_of(b, dims)
    shape = (nz, ny, nx)
    _check_volume(b, shape, "b")
    st = lib.tv_fgp_step2(_addr(b), _field(p_in, shape, "p_in"), _field(p_out, shape, "p_out"),
                          _field(r_in, shape, "r_in"), _field(r_out, shape, "r_out"),
                          float(lam), float(m1), float(m2), nx, ny, nz, _stream(stream))
    _raise(st, "tv_fgp_step2")


def tv_fgp_step3(b, p_in, p_out, r_in, r_out, lam, m1, m2, m3, stream=None, dims=None):
    """Three FGP steps (momentum m1, m2, m3) in one pass: p_in -> p_out, r_in -> r_out."""
    nx, ny, nz = _dims_of(b, dims)
    shape = (nz, ny, nx)
    _check_volume(b, shape, "b")
    st = lib.tv_fgp_step3(_addr(b), _field(p_in, shape, "p_in"), _field(p_out, shape, "p_out"),
                          _field(r_in, shape, "r_in"), _field(r_out, shape, "r_out"),
                          float(lam), float(m1), float(m2), float(m3), nx, ny, nz,
                          _stream(stream))
    _raise(st, "tv_fgp_step3")


def tv_primal(b, p, z, lam, stream=None, dims=None):
    """z = max(b - lam*L(p), 0) into the caller's buffer z."""
    nx, ny, nz = _dims_of(b, dims)
    shape = (nz, ny, nx)
    _check_volume(b, shape, "b")
    _check_volume(z, shape, "z")
    st = lib.tv_primal(_addr(b), _field(p, shape, "p"), _addr(z), float(lam),
                       nx, ny, nz, _stream(stream))
    _raise(st, "tv_primal")


def _check_dev(t, what, dtype_name, numel):
    if t is None or isinstance(t, int):
        return
    import torch
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous device tensor" % what)
    if str(t.dtype) != "torch." + dtype_name:
        raise ValueError("%s must be %s" % (what, dtype_name))
    if t.numel() < numel:
        raise ValueError("%s needs at least %d elements" % (what, numel))


def tv_fgp_duality_gap(b, p, lam, out, workspace, stream=None, dims=None):
    """Gap triple (G, TV(z), 1/2||z-b||^2) of p into the float64 device tensor `out`."""
    nx, ny, nz = _dims_of(b, dims)
    shape = (nz, ny, nx)
    _check_volume(b, shape, "b")
    _check_dev(out, "out", "float64", 3)
    ws_bytes = gap_workspace_bytes(nx, ny, nz)
    _check_dev(workspace, "workspace", "float64", ws_bytes // 8)
    st = lib.tv_fgp_duality_gap(_addr(b), _field(p, shape, "p"), float(lam), nx, ny, nz,
                                _addr(out), _addr(workspace),
                                ws_bytes if not isinstance(workspace, int) else ws_bytes,
                                _stream(stream))
    _raise(st, "tv_fgp_duality_gap")


def tv_fgp_duality_gap_noalloc(b, p, lam, out, stream=None, dims=None):
    """tv_fgp_duality_gap without a workspace: the partial sums live in the
    library's static device array (calls that overlap on one GPU race)."""
    nx, ny, nz = _dims_of(b, dims)
    shape = (nz, ny, nx)
    _check_volume(b, shape, "b")
    _check_dev(out, "out", "float64", 3)
    st = lib.tv_fgp_duality_gap_noalloc(_addr(b), _field(p, shape, "p"), float(lam), nx, ny,
                                        nz, _addr(out), _stream(stream))
    _raise(st, "tv_fgp_duality_gap_noalloc")


def tv_fgp_solve(b, p, r_a, r_b, lam, max_outer, n_inner, tol, gap_ws, gap_dev,
                 variant=FUSED, z_ws=None, stream=None, dims=None):
    """Outer iterations until G <= tol * P(z) or max_outer; synchronises the stream.

    Returns (outer_done, r_final, (G, TV(z), 1/2||z-b||^2)).
    """
    nx, ny, nz = _dims_of(b, dims)
    shape = (nz, ny, nx)
    _check_volume(b, shape, "b")
    _check_ws(z_ws, shape, variant)
    ws_bytes = gap_workspace_bytes(nx, ny, nz)
    _check_dev(gap_ws, "gap_ws", "float64", ws_bytes // 8)
    _check_dev(gap_dev, "gap_dev", "float64", 3)
    where = ctypes.c_int(-1)
    done = ctypes.c_int(-1)
    host = (ctypes.c_double * 3)()
    st = lib.tv_fgp_solve(_addr(b), _field(p, shape, "p"), _field(r_a, shape, "r_a"),
                          _field(r_b, shape, "r_b"), float(lam), int(max_outer), int(n_inner),
                          float(tol), nx, ny, nz, int(variant), _addr(z_ws), _addr(gap_ws),
                          ws_bytes, _addr(gap_dev), _stream(stream), ctypes.byref(where),
                          ctypes.byref(done), host)
    _raise(st, "tv_fgp_solve")
    return done.value, where.value, (host[0], host[1], host[2])


def tv_fgp_step_h(b, p, r_in, r_out, lam, m, stream=None, dims=None):
    """One FGP step with p, r stored as binary16 (float16 tensors)."""
    nx, ny, nz = _dims_of(b, dims)
    shape = (nz, ny, nx)
    _check_volume(b, shape, "b")
    st = lib.tv_fgp_step_h(_addr(b), _hfield(p, shape, "p"), _hfield(r_in, shape, "r_in"),
                           _hfield(r_out, shape, "r_out"), float(lam), float(m), nx, ny, nz,
                           _stream(stream))
    _raise(st, "tv_fgp_step_h")


def tv_fgp_run_h(b, p, r_a, r_b, lam, n_outer, n_inner, stream=None, dims=None):
    """tv_fgp_run with the binary16 dual; returns 0 if the last r is in r_a, 1 if in r_b."""
    nx, ny, nz = _dims_of(b, dims)
    shape = (nz, ny, nx)
    _check_volume(b, shape, "b")
    where = ctypes.c_int(-1)
    st = lib.tv_fgp_run_h(_addr(b), _hfield(p, shape, "p"), _hfield(r_a, shape, "r_a"),
                          _hfield(r_b, shape, "r_b"), float(lam), int(n_outer), int(n_inner),
                          nx, ny, nz, _stream(stream), ctypes.byref(where))
    _raise(st, "tv_fgp_run_h")
    return where.value


def tv_fgp_step2_h(b, p_in, p_out, r_in, r_out, lam, m1, m2, stream=None, dims=None):
    """tv_fgp_step2 with the binary16 dual (float16 or int16 tensors)."""
    nx, ny, nz = _dims_of(b, dims)
    shape = (nz, ny, nx)
    _check_volume(b, shape, "b")
    st = lib.tv_fgp_step2_h(_addr(b), _hfield(p_in, shape, "p_in"),
                            _hfield(p_out, shape, "p_out"), _hfield(r_in, shape, "r_in"),
                            _hfield(r_out, shape, "r_out"), float(lam), float(m1), float(m2),
                            nx, ny, nz, _stream(stream))
    _raise(st, "tv_fgp_step2_h")


def tv_fgp_run2_h(b, p, p_ws, r_a, r_b, lam, n_outer, n_inner, stream=None, dims=None):
    """tv_fgp_run_h with two steps per pass; p_ws holds three binary16 volumes
    ((3, nz, ny, nx) tensor).  Returns 0 if the last r is in r_a, 1 if in r_b."""
    nx, ny, nz = _dims_of(b, dims)
    shape = (nz, ny, nx)
    _check_volume(b, shape, "b")
    _check_half(p_ws, (3,) + shape, "p_ws")
    where = ctypes.c_int(-1)
    st = lib.tv_fgp_run2_h(_addr(b), _hfield(p, shape, "p"), _addr(p_ws),
                           _hfield(r_a, shape, "r_a"), _hfield(r_b, shape, "r_b"), float(lam),
                           int(n_outer), int(n_inner), nx, ny, nz, _stream(stream),
                           ctypes.byref(where))
    _raise(st, "tv_fgp_run2_h")
    return where.value


def tv_primal_h(b, p, z, lam, stream=None, dims=None):
    nx, ny, nz = _dims_of(b, dims)
    shape = (nz, ny, nx)
    _check_volume(b, shape, "b")
    _check_volume(z, shape, "z")
    st = lib.tv_primal_h(_addr(b), _hfield(p, shape, "p"), _addr(z), float(lam), nx, ny, nz,
                         _stream(stream))
    _raise(st, "tv_primal_h")


def tv_fgp_stream_probe(src, dst, stream=None):
    """dst[k] = src[k] + src[6] for k < 6: the 7-read / 6-write traffic of one
    step as a linear stream (a bandwidth ceiling, not a step).  src: 7 float32
    device tensors, dst: 6, all contiguous with the same number of elements."""
    if len(src) != 7 or len(dst) != 6:
        raise ValueError("tv_fgp_stream_probe takes 7 sources and 6 destinations")
    n = src[0].numel()
    for t in list(src) + list(dst):
        _check_dev(t, "probe volume", "float32", n)
        if t.numel() != n:
            raise ValueError("probe volumes must have the same number of elements")
    arr_s = (ctypes.c_void_p * 7)(*[t.data_ptr() for t in src])
    arr_d = (ctypes.c_void_p * 6)(*[t.data_ptr() for t in dst])
    st = lib.tv_fgp_stream_probe(arr_s, arr_d, n, _stream(stream))
    _raise(st, "tv_fgp_stream_probe")


# Shapes of tv_fgp_stream_probe_ex: (sources, destinations)
STREAM_SHAPES = ((7, 6), (7, 0), (0, 6), (1, 1))


def tv_fgp_stream_probe_ex(src, dst, stream=None):
    """The part's streaming rates for a step's read and write halves: with
    (len(src), len(dst)) = (7, 6) dst[k] = src[k] + src[6]; (7, 0) the sources
    are read and nothing is written; (0, 6) dst[k] = k; (1, 1) dst[0] = src[0].
    All float32 device tensors, contiguous, with the same number of elements."""
    src, dst = list(src), list(dst)
    if (len(src), len(dst)) not in STREAM_SHAPES:
        raise ValueError("tv_fgp_stream_probe_ex takes (sources, destinations) in %s"
                         % (STREAM_SHAPES,))
    n = (src or dst)[0].numel()
    for t in src + dst:
        _check_dev(t, "probe volume", "float32", n)
        if t.numel() != n:
            raise ValueError("probe volumes must have the same number of elements")
    arr_s = (ctypes.c_void_p * max(1, len(src)))(*[t.data_ptr() for t in src])
    arr_d = (ctypes.c_void_p * max(1, len(dst)))(*[t.data_ptr() for t in dst])
    st = lib.tv_fgp_stream_probe_ex(arr_s if src else None, len(src), arr_d if dst else None,
                                    len(dst), n, _stream(stream))
    _raise(st, "tv_fgp_stream_probe_ex")
