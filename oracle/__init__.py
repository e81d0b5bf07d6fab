"""fp64 CPU oracle for the fused attention-KL primitive -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  It is a thin ctypes wrapper over oracle/streamkl_oracle.c, a
plain materialising fp64 implementation of forward KL between the teacher and
student attention rows (teacher first, natural log), as defined on the pages
"StreamKL: Fast and Memory-Efficient KL Divergence for Boosting Attention
Distillation" (abstract) and "Lecture 05 - Where It All Lands" (section 3.1).
It shares no code with the HIP path and never imports it.

Inputs are numpy arrays shaped [B, H, N, d] holding the exact values the GPU
sees (bf16/fp32 inputs are widened to fp64 here, which is exact).  Outputs are
fp64.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libstreamkl_oracle.so")
_lib = None

_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_I = ctypes.c_int
_D = ctypes.c_double


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    common = [_f64p, _f64p, _f64p, _f64p, _I, _I, _I, _I, _I, _I, _D, _D, _I]
    lib.oracle_fwd.argtypes = common + [_f64p, _f64p, _f64p, ctypes.POINTER(ctypes.c_double)]
    lib.oracle_fwd.restype = None
    lib.oracle_fwd_rows.argtypes = common + [_I, _i64p, _f64p, _f64p, _f64p]
    lib.oracle_fwd_rows.restype = None
    lib.oracle_bwd.argtypes = common + [ctypes.c_void_p, _D, _f64p, _f64p]
    lib.oracle_bwd.restype = None
    lib.oracle_dq_rows.argtypes = common + [ctypes.c_void_p, _D, _I, _i64p, _f64p]
    lib.oracle_dq_rows.restype = None
    lib.oracle_dk_keys.argtypes = common + [ctypes.c_void_p, _D, _I, _I, _I, _i64p, _f64p]
    lib.oracle_dk_keys.restype = None
    lib.oracle_bwd_teacher.argtypes = common + [ctypes.c_void_p, _D, _f64p, _f64p]
    lib.oracle_bwd_teacher.restype = None
    lib.oracle_dqt_rows.argtypes = common + [ctypes.c_void_p, _D, _I, _i64p, _f64p]
    lib.oracle_dqt_rows.restype = None
    lib.oracle_dkt_keys.argtypes = common + [ctypes.c_void_p, _D, _I, _I, _I, _i64p, _f64p]
    lib.oracle_dkt_keys.restype = None
    lib.oracle_vocab_fwd.argtypes = [_f64p, _f64p, _I, _I, _D, _f64p, _f64p, _f64p, ctypes.POINTER(ctypes.c_double)]
    lib.oracle_vocab_fwd.restype = None
    lib.oracle_vocab_bwd.argtypes = [_f64p, _f64p, _I, _I, _D, ctypes.c_void_p, _D, _f64p, ctypes.c_void_p]
    lib.oracle_vocab_bwd.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = _I
    _lib = lib
    return lib


def _prep(q_t, k_t, q_s, k_s):
    arrs = [np.ascontiguousarray(a, dtype=np.float64) for a in (q_t, k_t, q_s, k_s)]
    for a in arrs:
        if a.ndim != 4:
            raise ValueError("oracle inputs must be [B, H, N, d]")
    q_t, k_t, q_s, k_s = arrs
    B, H, n_q, d_t = q_t.shape
    n_k = k_t.shape[2]
    d_s = q_s.shape[3]
    if k_t.shape != (B, H, n_k, d_t) or q_s.shape != (B, H, n_q, d_s) or k_s.shape != (B, H, n_k, d_s):
        raise ValueError("inconsistent oracle input shapes")
    return arrs, (B, H, n_q, n_k, d_t, d_s)


def _g_arg(g, B, H, n_q):
    if g is None or np.isscalar(g):
        return None, float(1.0 if g is None else g)
    g = np.ascontiguousarray(g, dtype=np.float64).reshape(-1)
    if g.size != B * H * n_q:
        raise ValueError("g must have B*H*n_q entries")
    return g, 0.0


def fwd(q_t, k_t, q_s, k_s, tau_t, tau_s, causal=False):
    """Per-row KL, LSE_t, LSE_s ([B, H, n_q] fp64) and their compensated sum."""
    lib = _load()
    arrs, (B, H, n_q, n_k, d_t, d_s) = _prep(q_t, k_t, q_s, k_s)
    kl = np.empty((B, H, n_q)); lt = np.empty_like(kl); ls = np.empty_like(kl)
    tot = ctypes.c_double(0.0)
    lib.oracle_fwd(*arrs, B, H, n_q, n_k, d_t, d_s, float(tau_t), float(tau_s), int(causal),
                   kl, lt, ls, ctypes.byref(tot))
    return kl, lt, ls, tot.value


def fwd_rows(q_t, k_t, q_s, k_s, tau_t, tau_s, causal, rows):
    """KL, LSE_t, LSE_s for flat row indices r = (b*H + h)*n_q + i."""
    lib = _load()
    arrs, (B, H, n_q, n_k, d_t, d_s) = _prep(q_t, k_t, q_s, k_s)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    n = rows.size
    kl = np.empty(n); lt = np.empty(n); ls = np.empty(n)
    lib.oracle_fwd_rows(*arrs, B, H, n_q, n_k, d_t, d_s, float(tau_t), float(tau_s), int(causal),
                        n, rows, kl, lt, ls)
    return kl, lt, ls


def bwd(q_t, k_t, q_s, k_s, tau_t, tau_s, causal=False, g=None):
    """dQ_s, dK_s (fp64) of L = sum_r g_r KL_r; g None means every g_r = 1."""
    lib = _load()
    arrs, (B, H, n_q, n_k, d_t, d_s) = _prep(q_t, k_t, q_s, k_s)
    garr, gs = _g_arg(g, B, H, n_q)
    dq = np.empty((B, H, n_q, d_s)); dk = np.empty((B, H, n_k, d_s))
    gp = garr.ctypes.data if garr is not None else None
    lib.oracle_bwd(*arrs, B, H, n_q, n_k, d_t, d_s, float(tau_t), float(tau_s), int(causal),
                   gp, gs, dq, dk)
    return dq, dk


def dq_rows(q_t, k_t, q_s, k_s, tau_t, tau_s, causal, rows, g=None):
    """dQ_s rows [len(rows), d_s] for flat row indices."""
    lib = _load()
    arrs, (B, H, n_q, n_k, d_t, d_s) = _prep(q_t, k_t, q_s, k_s)
    garr, gs = _g_arg(g, B, H, n_q)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, d_s))
    gp = garr.ctypes.data if garr is not None else None
    lib.oracle_dq_rows(*arrs, B, H, n_q, n_k, d_t, d_s, float(tau_t), float(tau_s), int(causal),
                       gp, gs, rows.size, rows, out)
    return out


def dk_keys(q_t, k_t, q_s, k_s, tau_t, tau_s, causal, b, h, keys, g=None):
    """dK_s rows [len(keys), d_s] for keys of head (b, h)."""
    lib = _load()
    arrs, (B, H, n_q, n_k, d_t, d_s) = _prep(q_t, k_t, q_s, k_s)
    garr, gs = _g_arg(g, B, H, n_q)
    keys = np.ascontiguousarray(keys, dtype=np.int64)
    out = np.empty((keys.size, d_s))
    gp = garr.ctypes.data if garr is not None else None
    lib.oracle_dk_keys(*arrs, B, H, n_q, n_k, d_t, d_s, float(tau_t), float(tau_s), int(causal),
                       gp, gs, int(b), int(h), keys.size, keys, out)
    return out


def num_threads():
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def bwd_teacher(q_t, k_t, q_s, k_s, tau_t, tau_s, causal=False, g=None):
    """dQ_t, dK_t (fp64) of L = sum_r g_r KL_r: gradients with respect to the
    first (teacher) distribution's queries and keys.  With the two
    distributions swapped these are the student gradients of the reverse KL."""
    lib = _load()
    arrs, (B, H, n_q, n_k, d_t, d_s) = _prep(q_t, k_t, q_s, k_s)
    garr, gs = _g_arg(g, B, H, n_q)
    dq = np.empty((B, H, n_q, d_t)); dk = np.empty((B, H, n_k, d_t))
    gp = garr.ctypes.data if garr is not None else None
    lib.oracle_bwd_teacher(*arrs, B, H, n_q, n_k, d_t, d_s, float(tau_t), float(tau_s), int(causal),
                           gp, gs, dq, dk)
    return dq, dk


def dqt_rows(q_t, k_t, q_s, k_s, tau_t, tau_s, causal, rows, g=None):
    """dQ_t rows [len(rows), d_t] for flat row indices."""
    lib = _load()
    arrs, (B, H, n_q, n_k, d_t, d_s) = _prep(q_t, k_t, q_s, k_s)
    garr, gs = _g_arg(g, B, H, n_q)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, d_t))
    gp = garr.ctypes.data if garr is not None else None
    lib.oracle_dqt_rows(*arrs, B, H, n_q, n_k, d_t, d_s, float(tau_t), float(tau_s), int(causal),
                        gp, gs, rows.size, rows, out)
    return out


def dkt_keys(q_t, k_t, q_s, k_s, tau_t, tau_s, causal, b, h, keys, g=None):
    """dK_t rows [len(keys), d_t] for keys of head (b, h)."""
    lib = _load()
    arrs, (B, H, n_q, n_k, d_t, d_s) = _prep(q_t, k_t, q_s, k_s)
    garr, gs = _g_arg(g, B, H, n_q)
    keys = np.ascontiguousarray(keys, dtype=np.int64)
    out = np.empty((keys.size, d_t))
    gp = garr.ctypes.data if garr is not None else None
    lib.oracle_dkt_keys(*arrs, B, H, n_q, n_k, d_t, d_s, float(tau_t), float(tau_s), int(causal),
                        gp, gs, int(b), int(h), keys.size, keys, out)
    return out


def _vocab_prep(z_t, z_s):
    z_t = np.ascontiguousarray(z_t, dtype=np.float64)
    z_s = np.ascontiguousarray(z_s, dtype=np.float64)
    if z_t.shape != z_s.shape or z_t.ndim < 1:
        raise ValueError("z_t and z_s must share a shape [..., V]")
    V = z_t.shape[-1]
    return z_t.reshape(-1, V), z_s.reshape(-1, V), z_t.shape


def vocab_fwd(z_t, z_s, temperature=1.0):
    """Per-row KL(softmax(z_t / T) || softmax(z_s / T)), LSE_t, LSE_s of the
    scaled logits (shape [...] of the leading dims) and their compensated sum."""
    lib = _load()
    zt, zs, shape = _vocab_prep(z_t, z_s)
    rows, V = zt.shape
    kl = np.empty(rows); lt = np.empty(rows); ls = np.empty(rows)
    tot = ctypes.c_double(0.0)
    lib.oracle_vocab_fwd(zt, zs, rows, V, 1.0 / float(temperature), kl, lt, ls, ctypes.byref(tot))
    lead = shape[:-1]
    return kl.reshape(lead), lt.reshape(lead), ls.reshape(lead), tot.value


def vocab_bwd(z_t, z_s, temperature=1.0, g=None, teacher=False):
    """dz_s (and dz_t if teacher) of L = sum_r g_r KL_r; g None means g_r = 1."""
    lib = _load()
    zt, zs, shape = _vocab_prep(z_t, z_s)
    rows, V = zt.shape
    if g is None or np.isscalar(g):
        garr, gs = None, float(1.0 if g is None else g)
    else:
        garr = np.ascontiguousarray(g, dtype=np.float64).reshape(-1)
        if garr.size != rows:
            raise ValueError("g must have one value per row")
        gs = 0.0
    dzs = np.empty((rows, V))
    dzt = np.empty((rows, V)) if teacher else None
    lib.oracle_vocab_bwd(zt, zs, rows, V, 1.0 / float(temperature), garr.ctypes.data if garr is not None else None,
                         gs, dzs, dzt.ctypes.data if dzt is not None else None)
    return (dzs.reshape(shape), dzt.reshape(shape)) if teacher else dzs.reshape(shape)
