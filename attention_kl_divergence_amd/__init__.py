"""Fused attention-KL primitive for MI355X: thin Python binding over libstreamkl.so.

The library (csrc/streamkl.hip, C ABI in include/streamkl.h) computes, per
query row, the forward KL divergence between the teacher and the student
attention distributions, teacher first, in nats, without materialising either
N_Q x N_K matrix, and the gradients of sum_r g_r KL_r with respect to the
student queries and keys ("StreamKL: Fast and Memory-Efficient KL Divergence
for Boosting Attention Distillation", abstract; direction and units: "Lecture
05 - Where It All Lands", section 3.1).

This module only marshals arguments: it checks tensor placement, dtype and
shape, allocates the outputs with torch (device memory), and passes raw device
pointers and torch's current HIP stream to the C entry points of the same
names.  Every step of the computation runs in the HIP kernels; there is no
fallback.  If the library is missing the calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libstreamkl.so")

STREAMKL_OK, STREAMKL_ERR_INVALID, STREAMKL_ERR_UNSUPPORTED, STREAMKL_ERR_WORKSPACE, STREAMKL_ERR_HIP = range(5)
STREAMKL_F32, STREAMKL_BF16 = 0, 1

_lib = None


class StreamKLLayout(ctypes.Structure):
    """streamkl_layout: head counts of q_t, k_t, q_s, k_s (0 = H), per-batch
    valid lengths (device int32 [B] pointers, or None) and packed-sequence
    offsets (device int32 [B + 1] pointers, or None)."""
    _fields_ = [("heads_q_t", ctypes.c_int), ("heads_k_t", ctypes.c_int), ("heads_q_s", ctypes.c_int),
                ("heads_k_s", ctypes.c_int), ("seqlen_q", ctypes.c_void_p), ("seqlen_k", ctypes.c_void_p),
                ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p)]


class StreamKLError(RuntimeError):
    def __init__(self, where: str, code: int, text: str):
        super().__init__(f"{where} failed: status {code} ({text})")
        self.code = code


def load_library():
    """Load libstreamkl.so and declare its C signatures (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -m attention_kl_divergence_amd.build "
                           f"or __graft_entry__.build()); there is no non-HIP fallback")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f, i64p = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.POINTER(ctypes.c_int64)
    lib.streamkl_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i64p, f, f, i, vp, vp, vp, vp, vp]
    lib.streamkl_fwd.restype = i
    lib.streamkl_bwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i64p, f, f, i, vp, vp, vp, f, vp, vp, vp]
    lib.streamkl_bwd.restype = i
    lib.streamkl_bwd_teacher.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i64p, f, f, i, vp, vp, vp, vp, f,
                                         vp, vp, vp]
    lib.streamkl_bwd_teacher.restype = i
    sz = ctypes.c_size_t
    lib.streamkl_fwd_partial.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i64p, f, f, i, i, i, vp, vp]
    lib.streamkl_fwd_partial.restype = i
    lib.streamkl_fwd_merge.argtypes = [vp, i, ctypes.c_int64, f, f, vp, vp, vp, vp, vp]
    lib.streamkl_fwd_merge.restype = i
    lib.streamkl_fwd_split_count.argtypes = [i, i, i, i, i]
    lib.streamkl_fwd_split_count.restype = i
    lib.streamkl_fwd_split_workspace_size.argtypes = [i, i, i, i]
    lib.streamkl_fwd_split_workspace_size.restype = sz
    lib.streamkl_fwd_split.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i64p, f, f, i, i, vp, sz, vp, vp, vp,
                                       vp, vp]
    lib.streamkl_fwd_split.restype = i
    lib.streamkl_fwd_split_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i64p, f, f, i, i, vp, vp, vp,
                                               vp, vp]
    lib.streamkl_fwd_split_noalloc.restype = i
    lay = ctypes.POINTER(StreamKLLayout)
    lib.streamkl_fwd_ex.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i64p, lay, f, f, i, vp, vp, vp, vp, vp]
    lib.streamkl_fwd_ex.restype = i
    lib.streamkl_bwd_ex.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i64p, lay, f, f, i, vp, vp, vp, f, vp, vp,
                                    vp, ctypes.c_size_t, vp]
    lib.streamkl_bwd_ex.restype = i
    lib.streamkl_bwd_teacher_ex.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i64p, lay, f, f, i, vp, vp, vp, vp,
                                            f, vp, vp, vp, ctypes.c_size_t, vp]
    lib.streamkl_bwd_teacher_ex.restype = i
    lib.streamkl_bwd_ex_workspace_size.argtypes = [i, i, i, i, i, i, lay, i]
    lib.streamkl_bwd_ex_workspace_size.restype = ctypes.c_size_t
    i64 = ctypes.c_int64
    lib.streamkl_vocab_fwd.argtypes = [vp, vp, i, i64, i, i64, i64, f, vp, vp, vp, vp, vp]
    lib.streamkl_vocab_fwd.restype = i
    lib.streamkl_vocab_bwd.argtypes = [vp, vp, i, i64, i, i64, i64, f, vp, vp, vp, vp, f, vp, vp, vp]
    lib.streamkl_vocab_bwd.restype = i
    lib.streamkl_vocab_fwd_bwd.argtypes = [vp, vp, i, i64, i, i64, i64, f, vp, f, vp, vp, vp, vp, vp, vp, vp]
    lib.streamkl_vocab_fwd_bwd.restype = i
    lib.streamkl_bwd_workspace_size.argtypes = [i, i, i, i, i, i, i, i]
    lib.streamkl_bwd_workspace_size.restype = ctypes.c_size_t
    lib.streamkl_status_string.argtypes = [i]
    lib.streamkl_status_string.restype = ctypes.c_char_p
    lib.streamkl_supported.argtypes = [i, i, i]
    lib.streamkl_supported.restype = i
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load_library().streamkl_status_string(int(code)).decode()


def supported(dtype_code: int, d_t: int, d_s: int) -> bool:
    return bool(load_library().streamkl_supported(int(dtype_code), int(d_t), int(d_s)))


def _check(where, code):
    if code != STREAMKL_OK:
        raise StreamKLError(where, code, status_string(code))


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return STREAMKL_BF16
    if t.dtype == torch.float32:
        return STREAMKL_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _inputs(q_t, k_t, q_s, k_s):
    """Check the four [B, heads, N, d] tensors; returns ((B, H, n_q, n_k, d_t,
    d_s), strides, heads) with H the number of KL heads (the larger query head
    count) and heads the four tensors' own head counts."""
    import torch
    ts = (q_t, k_t, q_s, k_s)
    for t in ts:
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise ValueError("q_t, k_t, q_s, k_s must be 4-D tensors [B, heads, N, d]")
        if t.device.type != "cuda":
            raise ValueError("inputs must be device (HIP) tensors")
        if t.stride(-1) != 1:
            raise ValueError("the last dimension must be contiguous")
    if len({t.dtype for t in ts}) != 1 or len({t.device for t in ts}) != 1:
        raise ValueError("inputs must share dtype and device")
    B, hq_t, n_q, d_t = q_t.shape
    hk_t, n_k = k_t.shape[1], k_t.shape[2]
    hq_s, d_s = q_s.shape[1], q_s.shape[3]
    hk_s = k_s.shape[1]
    if tuple(k_t.shape) != (B, hk_t, n_k, d_t) or tuple(q_s.shape) != (B, hq_s, n_q, d_s) or \
            tuple(k_s.shape) != (B, hk_s, n_k, d_s):
        raise ValueError("inconsistent shapes: q_t [B,Hqt,Nq,dt], k_t [B,Hkt,Nk,dt], q_s [B,Hqs,Nq,ds], "
                         "k_s [B,Hks,Nk,ds]")
    H = max(hq_t, hq_s)
    if H % hq_t or H % hq_s or hq_t % hk_t or hq_s % hk_s:
        raise ValueError("head counts must nest: each query head count divides the larger one and each key "
                         "head count divides its model's query head count")
    strides = (ctypes.c_int64 * 12)(*[s for t in ts for s in (t.stride(0), t.stride(1), t.stride(2))])
    return (B, H, n_q, n_k, d_t, d_s), strides, (hq_t, hk_t, hq_s, hk_s)


def _layout(B, H, heads, seqlen_q, seqlen_k, dev):
    """A StreamKLLayout when head counts differ or lengths are given, else None.
    Also returns the int32 length tensors it points to (kept alive by the caller)."""
    import torch
    if all(h == H for h in heads) and seqlen_q is None and seqlen_k is None:
        return None, ()
    keep = []
    ptrs = []
    for name, t in (("seqlen_q", seqlen_q), ("seqlen_k", seqlen_k)):
        if t is None:
            ptrs.append(None)
            continue
        if not isinstance(t, torch.Tensor):
            t = torch.tensor(t, dtype=torch.int32, device=dev)
        if t.dtype != torch.int32 or t.device != dev or tuple(t.shape) != (B,):
            raise ValueError(f"{name} must be an int32 [B] tensor on the inputs' device")
        t = t.contiguous()
        keep.append(t)
        ptrs.append(t.data_ptr())
    lay = StreamKLLayout(heads[0], heads[1], heads[2], heads[3], ptrs[0], ptrs[1], None, None)
    return lay, tuple(keep)


def _stream_ptr(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _taus(tau_t, tau_s, d_t, d_s):
    return (float(1.0 / math.sqrt(d_t)) if tau_t is None else float(tau_t),
            float(1.0 / math.sqrt(d_s)) if tau_s is None else float(tau_s))


def streamkl_fwd(q_t, k_t, q_s, k_s, tau_t=None, tau_s=None, causal=False, with_sum=True, split=None,
                 seqlen_q=None, seqlen_k=None):
    """Forward: returns (kl_rows, lse_t, lse_s, kl_sum), fp32 device tensors.

    kl_rows/lse_t/lse_s are [B, H, N_Q]; kl_sum is a 1-element tensor (None if
    with_sum is False).  tau defaults to 1/sqrt(d) per side.  split: number of
    key ranges run as separate workgroups and merged (split-K); None takes the
    library's suggestion for the shape (1 when the GPU is already full).

    Grouped heads: the four tensors may have their own head counts (see
    include/streamkl.h): H is the larger query head count, a model with fewer
    query heads is broadcast over consecutive KL heads and keys are shared by
    consecutive query heads.  seqlen_q / seqlen_k: int32 [B] valid lengths of
    each batch inside the padded N_Q / N_K (rows past them are empty: KL 0).
    """
    import torch
    lib = load_library()
    (B, H, n_q, n_k, d_t, d_s), strides, heads = _inputs(q_t, k_t, q_s, k_s)
    tau_t, tau_s = _taus(tau_t, tau_s, d_t, d_s)
    dev = q_t.device
    kl = torch.empty((B, H, n_q), dtype=torch.float32, device=dev)
    lt = torch.empty_like(kl)
    ls = torch.empty_like(kl)
    tot = torch.empty((1,), dtype=torch.float32, device=dev) if with_sum else None
    lay, _keep = _layout(B, H, heads, seqlen_q, seqlen_k, dev)
    if lay is not None:
        code = lib.streamkl_fwd_ex(q_t.data_ptr(), k_t.data_ptr(), q_s.data_ptr(), k_s.data_ptr(), _dtype_code(q_t),
                                   B, H, n_q, n_k, d_t, d_s, strides, ctypes.byref(lay), tau_t, tau_s,
                                   int(bool(causal)), kl.data_ptr(), lt.data_ptr(), ls.data_ptr(),
                                   tot.data_ptr() if tot is not None else None, _stream_ptr(dev))
        _check("streamkl_fwd_ex", code)
        return kl, lt, ls, tot
    n_split = int(lib.streamkl_fwd_split_count(B, H, n_q, n_k, int(bool(causal)))) if split is None else int(split)
    if n_split > 1:
        nbytes = int(lib.streamkl_fwd_split_workspace_size(B, H, n_q, n_split))
        ws = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
        code = lib.streamkl_fwd_split(q_t.data_ptr(), k_t.data_ptr(), q_s.data_ptr(), k_s.data_ptr(),
                                      _dtype_code(q_t), B, H, n_q, n_k, d_t, d_s, strides, tau_t, tau_s,
                                      int(bool(causal)), n_split, ws.data_ptr(), nbytes,
                                      kl.data_ptr(), lt.data_ptr(), ls.data_ptr(),
                                      tot.data_ptr() if tot is not None else None, _stream_ptr(dev))
        _check("streamkl_fwd_split", code)
        return kl, lt, ls, tot
    code = lib.streamkl_fwd(q_t.data_ptr(), k_t.data_ptr(), q_s.data_ptr(), k_s.data_ptr(), _dtype_code(q_t),
                            B, H, n_q, n_k, d_t, d_s, strides, tau_t, tau_s, int(bool(causal)),
                            kl.data_ptr(), lt.data_ptr(), ls.data_ptr(),
                            tot.data_ptr() if tot is not None else None, _stream_ptr(dev))
    _check("streamkl_fwd", code)
    return kl, lt, ls, tot


NOALLOC_SCRATCH_BYTES = 16 << 20  # STREAMKL_NOALLOC_SCRATCH_BYTES


def streamkl_fwd_noalloc(q_t, k_t, q_s, k_s, tau_t=None, tau_s=None, causal=False, split=None, kl=None, lse_t=None,
                         lse_s=None, kl_sum=None):
    """The split forward through streamkl_fwd_split_noalloc, whose split states
    live in the library's per-GPU scratch array: no device memory is allocated
    for them.  Pass preallocated fp32 outputs (kl, lse_t, lse_s [B, H, N_Q],
    kl_sum [1] or None) to allocate nothing at all; missing ones are
    allocated here.  Calls that overlap on one GPU race (see the header)."""
    import torch
    lib = load_library()
    (B, H, n_q, n_k, d_t, d_s), strides, heads = _inputs(q_t, k_t, q_s, k_s)
    if any(h != H for h in heads):
        raise ValueError("streamkl_fwd_noalloc takes equal head counts")
    tau_t, tau_s = _taus(tau_t, tau_s, d_t, d_s)
    dev = q_t.device
    n_split = int(lib.streamkl_fwd_split_count(B, H, n_q, n_k, int(bool(causal)))) if split is None else int(split)
    outs = []
    for t in (kl, lse_t, lse_s):
        if t is None:
            t = torch.empty((B, H, n_q), dtype=torch.float32, device=dev)
        elif t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (B, H, n_q) or t.device != dev:
            raise ValueError("kl, lse_t and lse_s must be contiguous fp32 [B, H, N_Q] tensors on the inputs' device")
        outs.append(t)
    code = lib.streamkl_fwd_split_noalloc(q_t.data_ptr(), k_t.data_ptr(), q_s.data_ptr(), k_s.data_ptr(),
                                          _dtype_code(q_t), B, H, n_q, n_k, d_t, d_s, strides, tau_t, tau_s,
                                          int(bool(causal)), n_split, outs[0].data_ptr(), outs[1].data_ptr(),
                                          outs[2].data_ptr(), kl_sum.data_ptr() if kl_sum is not None else None,
                                          _stream_ptr(dev))
    _check("streamkl_fwd_split_noalloc", code)
    return outs[0], outs[1], outs[2], kl_sum


STATE_FLOATS = 6


def streamkl_fwd_partial(q_t, k_t, q_s, k_s, k_begin, k_end, tau_t=None, tau_s=None, causal=False):
    """Partial forward over global keys [k_begin, k_end): returns the per-row
    online states, fp32 [B, H, N_Q, 6] (see include/streamkl.h).  Partial
    states of disjoint key ranges combine with streamkl_fwd_merge."""
    import torch
    lib = load_library()
    (B, H, n_q, n_k, d_t, d_s), strides, heads = _inputs(q_t, k_t, q_s, k_s)
    if any(h != H for h in heads):
        raise ValueError("streamkl_fwd_partial takes equal head counts")
    tau_t, tau_s = _taus(tau_t, tau_s, d_t, d_s)
    dev = q_t.device
    st = torch.empty((B, H, n_q, STATE_FLOATS), dtype=torch.float32, device=dev)
    code = lib.streamkl_fwd_partial(q_t.data_ptr(), k_t.data_ptr(), q_s.data_ptr(), k_s.data_ptr(),
                                    _dtype_code(q_t), B, H, n_q, n_k, d_t, d_s, strides, tau_t, tau_s,
                                    int(bool(causal)), int(k_begin), int(k_end), st.data_ptr(), _stream_ptr(dev))
    _check("streamkl_fwd_partial", code)
    return st


def streamkl_fwd_merge(states, tau_t, tau_s, with_sum=True):
    """Merge partial states [S, B, H, N_Q, 6] (or a list of [B, H, N_Q, 6])
    into (kl_rows, lse_t, lse_s, kl_sum) as streamkl_fwd returns them."""
    import torch
    lib = load_library()
    if isinstance(states, (list, tuple)):
        states = torch.stack(list(states))
    if states.dtype != torch.float32 or states.dim() != 5 or states.shape[-1] != STATE_FLOATS:
        raise ValueError("states must be fp32 [S, B, H, N_Q, 6]")
    states = states.contiguous()
    S, B, H, n_q, _ = states.shape
    dev = states.device
    kl = torch.empty((B, H, n_q), dtype=torch.float32, device=dev)
    lt, ls = torch.empty_like(kl), torch.empty_like(kl)
    tot = torch.empty((1,), dtype=torch.float32, device=dev) if with_sum else None
    code = lib.streamkl_fwd_merge(states.data_ptr(), S, B * H * n_q, float(tau_t), float(tau_s), kl.data_ptr(),
                                  lt.data_ptr(), ls.data_ptr(), tot.data_ptr() if tot is not None else None,
                                  _stream_ptr(dev))
    _check("streamkl_fwd_merge", code)
    return kl, lt, ls, tot


def streamkl_bwd(q_t, k_t, q_s, k_s, lse_t, lse_s, grad_rows=None, grad_scalar=1.0,
                 tau_t=None, tau_s=None, causal=False, seqlen_q=None, seqlen_k=None):
    """Backward: returns (dq_s, dk_s) in the input dtype for L = sum_r g_r KL_r,
    shaped like q_s and k_s (a head shared by several KL heads gets the sum).

    grad_rows: fp32 [B, H, N_Q] device tensor of dL/dKL_r, or None to use
    grad_scalar for every row.  seqlen_q / seqlen_k as in streamkl_fwd.
    """
    import torch
    lib = load_library()
    (B, H, n_q, n_k, d_t, d_s), strides, heads = _inputs(q_t, k_t, q_s, k_s)
    tau_t, tau_s = _taus(tau_t, tau_s, d_t, d_s)
    dev = q_t.device
    for name, t in (("lse_t", lse_t), ("lse_s", lse_s)) + ((("grad_rows", grad_rows),) if grad_rows is not None else ()):
        if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (B, H, n_q) or t.device != dev:
            raise ValueError(f"{name} must be a contiguous fp32 [B, H, N_Q] tensor on the inputs' device")
    dq = torch.empty((B, heads[2], n_q, d_s), dtype=q_s.dtype, device=dev)
    dk = torch.empty((B, heads[3], n_k, d_s), dtype=q_s.dtype, device=dev)
    lay, _keep = _layout(B, H, heads, seqlen_q, seqlen_k, dev)
    if lay is not None:
        wsb = int(lib.streamkl_bwd_ex_workspace_size(B, H, n_q, n_k, d_t, d_s, ctypes.byref(lay), 0))
        ws = torch.empty((wsb,), dtype=torch.uint8, device=dev) if wsb else None
        code = lib.streamkl_bwd_ex(q_t.data_ptr(), k_t.data_ptr(), q_s.data_ptr(), k_s.data_ptr(), _dtype_code(q_t),
                                   B, H, n_q, n_k, d_t, d_s, strides, ctypes.byref(lay), tau_t, tau_s,
                                   int(bool(causal)), lse_t.data_ptr(), lse_s.data_ptr(),
                                   grad_rows.data_ptr() if grad_rows is not None else None, float(grad_scalar),
                                   dq.data_ptr(), dk.data_ptr(), ws.data_ptr() if ws is not None else None, wsb,
                                   _stream_ptr(dev))
        _check("streamkl_bwd_ex", code)
        return dq, dk
    code = lib.streamkl_bwd(q_t.data_ptr(), k_t.data_ptr(), q_s.data_ptr(), k_s.data_ptr(), _dtype_code(q_t),
                            B, H, n_q, n_k, d_t, d_s, strides, tau_t, tau_s, int(bool(causal)),
                            lse_t.data_ptr(), lse_s.data_ptr(),
                            grad_rows.data_ptr() if grad_rows is not None else None, float(grad_scalar),
                            dq.data_ptr(), dk.data_ptr(), _stream_ptr(dev))
    _check("streamkl_bwd", code)
    return dq, dk


def streamkl_bwd_teacher(q_t, k_t, q_s, k_s, lse_t, lse_s, kl_rows, grad_rows=None, grad_scalar=1.0,
                         tau_t=None, tau_s=None, causal=False, seqlen_q=None, seqlen_k=None):
    """Backward with respect to the first (teacher) distribution: returns
    (dq_t, dk_t) in the input dtype for L = sum_r g_r KL_r, shaped like q_t and
    k_t.  kl_rows, lse_t and lse_s are the forward's outputs.  With the two
    distributions swapped it gives the student gradients of the reverse
    divergence KL(P_s || P_t)."""
    import torch
    lib = load_library()
    (B, H, n_q, n_k, d_t, d_s), strides, heads = _inputs(q_t, k_t, q_s, k_s)
    tau_t, tau_s = _taus(tau_t, tau_s, d_t, d_s)
    dev = q_t.device
    rowargs = (("lse_t", lse_t), ("lse_s", lse_s), ("kl_rows", kl_rows)) + \
        ((("grad_rows", grad_rows),) if grad_rows is not None else ())
    for name, t in rowargs:
        if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (B, H, n_q) or t.device != dev:
            raise ValueError(f"{name} must be a contiguous fp32 [B, H, N_Q] tensor on the inputs' device")
    dq = torch.empty((B, heads[0], n_q, d_t), dtype=q_t.dtype, device=dev)
    dk = torch.empty((B, heads[1], n_k, d_t), dtype=q_t.dtype, device=dev)
    lay, _keep = _layout(B, H, heads, seqlen_q, seqlen_k, dev)
    if lay is not None:
        wsb = int(lib.streamkl_bwd_ex_workspace_size(B, H, n_q, n_k, d_t, d_s, ctypes.byref(lay), 1))
        ws = torch.empty((wsb,), dtype=torch.uint8, device=dev) if wsb else None
        code = lib.streamkl_bwd_teacher_ex(q_t.data_ptr(), k_t.data_ptr(), q_s.data_ptr(), k_s.data_ptr(),
                                           _dtype_code(q_t), B, H, n_q, n_k, d_t, d_s, strides, ctypes.byref(lay),
                                           tau_t, tau_s, int(bool(causal)), lse_t.data_ptr(), lse_s.data_ptr(),
                                           kl_rows.data_ptr(),
                                           grad_rows.data_ptr() if grad_rows is not None else None,
                                           float(grad_scalar), dq.data_ptr(), dk.data_ptr(),
                                           ws.data_ptr() if ws is not None else None, wsb, _stream_ptr(dev))
        _check("streamkl_bwd_teacher_ex", code)
        return dq, dk
    code = lib.streamkl_bwd_teacher(q_t.data_ptr(), k_t.data_ptr(), q_s.data_ptr(), k_s.data_ptr(),
                                    _dtype_code(q_t), B, H, n_q, n_k, d_t, d_s, strides, tau_t, tau_s,
                                    int(bool(causal)), lse_t.data_ptr(), lse_s.data_ptr(), kl_rows.data_ptr(),
                                    grad_rows.data_ptr() if grad_rows is not None else None, float(grad_scalar),
                                    dq.data_ptr(), dk.data_ptr(), _stream_ptr(dev))
    _check("streamkl_bwd_teacher", code)
    return dq, dk


def _vocab_rows(z_t, z_s):
    """Flatten [..., V] logits to rows; returns (zt2, zs2, lead_shape, rows, V, ld_t, ld_s)."""
    import torch
    for t in (z_t, z_s):
        if not isinstance(t, torch.Tensor) or t.dim() < 1:
            raise ValueError("z_t and z_s must be tensors [..., V]")
        if t.device.type != "cuda":
            raise ValueError("logits must be device (HIP) tensors")
    if z_t.dtype != z_s.dtype or z_t.device != z_s.device:
        raise ValueError("z_t and z_s must share dtype and device")
    if tuple(z_t.shape) != tuple(z_s.shape):
        raise ValueError("z_t and z_s must have the same shape [..., V]")
    V = z_t.shape[-1]
    lead = tuple(z_t.shape[:-1])
    zt2 = z_t.reshape(-1, V)  # a view when the rows share one stride, else a copy
    zs2 = z_s.reshape(-1, V)
    if zt2.stride(-1) != 1:
        zt2 = zt2.contiguous()
    if zs2.stride(-1) != 1:
        zs2 = zs2.contiguous()
    rows = zt2.shape[0]
    ld_t = zt2.stride(0) if rows > 1 else V
    ld_s = zs2.stride(0) if rows > 1 else V
    return zt2, zs2, lead, rows, V, ld_t, ld_s


def _row_vec(name, t, rows, dev, lead):
    import torch
    if t.dtype != torch.float32 or t.device != dev or t.numel() != rows or tuple(t.shape) != lead:
        raise ValueError(f"{name} must be an fp32 tensor of shape {lead} on the logits' device")
    return t.contiguous()


def streamkl_vocab_fwd(z_t, z_s, temperature=1.0, with_sum=True):
    """Per-row KL(softmax(z_t / T) || softmax(z_s / T)) over the last dim.

    Returns (kl_rows, lse_t, lse_s, kl_sum): fp32 tensors of the leading shape
    and a 1-element sum (None if with_sum is False)."""
    import torch
    lib = load_library()
    zt, zs, lead, rows, V, ld_t, ld_s = _vocab_rows(z_t, z_s)
    dev = zt.device
    kl = torch.empty(lead, dtype=torch.float32, device=dev)
    lt, ls = torch.empty_like(kl), torch.empty_like(kl)
    tot = torch.empty((1,), dtype=torch.float32, device=dev) if with_sum else None
    code = lib.streamkl_vocab_fwd(zt.data_ptr(), zs.data_ptr(), _dtype_code(zt), rows, V, ld_t, ld_s,
                                  float(temperature), kl.data_ptr(), lt.data_ptr(), ls.data_ptr(),
                                  tot.data_ptr() if tot is not None else None, _stream_ptr(dev))
    _check("streamkl_vocab_fwd", code)
    return kl, lt, ls, tot


def streamkl_vocab_bwd(z_t, z_s, lse_t, lse_s, kl_rows=None, temperature=1.0, grad_rows=None, grad_scalar=1.0,
                       teacher=False):
    """Gradients of L = sum_r g_r KL_r: dz_s, or (dz_s, dz_t) if teacher
    (then kl_rows, the forward's, is needed).  Same shape and dtype as z_s."""
    import torch
    lib = load_library()
    zt, zs, lead, rows, V, ld_t, ld_s = _vocab_rows(z_t, z_s)
    dev = zt.device
    lse_t = _row_vec("lse_t", lse_t, rows, dev, lead)
    lse_s = _row_vec("lse_s", lse_s, rows, dev, lead)
    if teacher:
        if kl_rows is None:
            raise ValueError("teacher gradients need the forward's kl_rows")
        kl_rows = _row_vec("kl_rows", kl_rows, rows, dev, lead)
    if grad_rows is not None:
        grad_rows = _row_vec("grad_rows", grad_rows, rows, dev, lead)
    dzs = torch.empty((rows, V), dtype=zs.dtype, device=dev)
    dzt = torch.empty((rows, V), dtype=zs.dtype, device=dev) if teacher else None
    code = lib.streamkl_vocab_bwd(zt.data_ptr(), zs.data_ptr(), _dtype_code(zt), rows, V, ld_t, ld_s,
                                  float(temperature), lse_t.data_ptr(), lse_s.data_ptr(),
                                  kl_rows.data_ptr() if teacher else None,
                                  grad_rows.data_ptr() if grad_rows is not None else None, float(grad_scalar),
                                  dzs.data_ptr(), dzt.data_ptr() if dzt is not None else None, _stream_ptr(dev))
    _check("streamkl_vocab_bwd", code)
    shape = lead + (V,)
    return (dzs.view(shape), dzt.view(shape)) if teacher else dzs.view(shape)


def streamkl_vocab_fwd_bwd(z_t, z_s, temperature=1.0, grad_rows=None, grad_scalar=1.0, teacher=False,
                           with_sum=True):
    """Loss and gradients in one launch for upstream weights known up front:
    returns (kl_rows, lse_t, lse_s, kl_sum, dz_s, dz_t); dz_t is None unless
    teacher."""
    import torch
    lib = load_library()
    zt, zs, lead, rows, V, ld_t, ld_s = _vocab_rows(z_t, z_s)
    dev = zt.device
    if grad_rows is not None:
        grad_rows = _row_vec("grad_rows", grad_rows, rows, dev, lead)
    kl = torch.empty(lead, dtype=torch.float32, device=dev)
    lt, ls = torch.empty_like(kl), torch.empty_like(kl)
    tot = torch.empty((1,), dtype=torch.float32, device=dev) if with_sum else None
    dzs = torch.empty((rows, V), dtype=zs.dtype, device=dev)
    dzt = torch.empty((rows, V), dtype=zs.dtype, device=dev) if teacher else None
    code = lib.streamkl_vocab_fwd_bwd(zt.data_ptr(), zs.data_ptr(), _dtype_code(zt), rows, V, ld_t, ld_s,
                                      float(temperature), grad_rows.data_ptr() if grad_rows is not None else None,
                                      float(grad_scalar), kl.data_ptr(), lt.data_ptr(), ls.data_ptr(),
                                      tot.data_ptr() if tot is not None else None, dzs.data_ptr(),
                                      dzt.data_ptr() if dzt is not None else None, _stream_ptr(dev))
    _check("streamkl_vocab_fwd_bwd", code)
    shape = lead + (V,)
    return kl, lt, ls, tot, dzs.view(shape), (dzt.view(shape) if dzt is not None else None)


def _inputs_varlen(q_t, k_t, q_s, k_s, cu_q, cu_k, max_q, max_k):
    """Check packed [rows, heads, d] tensors and their int32 [B + 1] offsets;
    returns ((B, H, n_q, n_k, d_t, d_s), strides, heads)."""
    import torch
    ts = (q_t, k_t, q_s, k_s)
    for t in ts:
        if not isinstance(t, torch.Tensor) or t.dim() != 3:
            raise ValueError("packed q_t, k_t, q_s, k_s must be 3-D tensors [rows, heads, d]")
        if t.device.type != "cuda" or t.stride(-1) != 1:
            raise ValueError("inputs must be device (HIP) tensors with a contiguous last dimension")
    if len({t.dtype for t in ts}) != 1 or len({t.device for t in ts}) != 1:
        raise ValueError("inputs must share dtype and device")
    for name, c in (("cu_seqlens_q", cu_q), ("cu_seqlens_k", cu_k)):
        if not isinstance(c, torch.Tensor) or c.dtype != torch.int32 or c.dim() != 1 or c.device != q_t.device:
            raise ValueError(f"{name} must be an int32 [B + 1] tensor on the inputs' device")
    if cu_q.numel() != cu_k.numel() or cu_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B + 1 offsets")
    hq_t, d_t = q_t.shape[1], q_t.shape[2]
    hk_t, hq_s, d_s, hk_s = k_t.shape[1], q_s.shape[1], q_s.shape[2], k_s.shape[1]
    if k_t.shape[2] != d_t or k_s.shape[2] != d_s or q_s.shape[0] != q_t.shape[0] or k_s.shape[0] != k_t.shape[0]:
        raise ValueError("inconsistent packed shapes: q_t [Tq,Hqt,dt], k_t [Tk,Hkt,dt], q_s [Tq,Hqs,ds], "
                         "k_s [Tk,Hks,ds]")
    H = max(hq_t, hq_s)
    if H % hq_t or H % hq_s or hq_t % hk_t or hq_s % hk_s:
        raise ValueError("head counts must nest as for grouped heads")
    strides = (ctypes.c_int64 * 12)(*[s for t in ts for s in (0, t.stride(1), t.stride(0))])
    return (cu_q.numel() - 1, H, int(max_q), int(max_k), d_t, d_s), strides, (hq_t, hk_t, hq_s, hk_s)


def check_cu_seqlens(cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, total_q=None, total_k=None):
    """Host-side check of packed-sequence offsets (copies them to the host,
    which synchronises the device): offsets start at 0 or above, never
    decrease, stay within the packed rows, and no sequence is longer than its
    max_seqlen.  The kernels themselves clamp a longer sequence to max_seqlen
    (its extra rows are ignored), so a caller that cannot vouch for its
    offsets should call this first."""
    for name, cu, mx, total in (("cu_seqlens_q", cu_seqlens_q, max_seqlen_q, total_q),
                                ("cu_seqlens_k", cu_seqlens_k, max_seqlen_k, total_k)):
        c = [int(v) for v in cu.detach().cpu().tolist()]
        if c[0] < 0:
            raise ValueError(f"{name}: negative first offset {c[0]}")
        lens = [b - a for a, b in zip(c[:-1], c[1:])]
        if any(n < 0 for n in lens):
            raise ValueError(f"{name}: offsets decrease")
        if any(n > int(mx) for n in lens):
            raise ValueError(f"{name}: a sequence of length {max(lens)} exceeds max_seqlen {int(mx)}")
        if total is not None and c[-1] > total:
            raise ValueError(f"{name}: last offset {c[-1]} past the {total} packed rows")


def streamkl_fwd_varlen(q_t, k_t, q_s, k_s, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                        tau_t=None, tau_s=None, causal=False, with_sum=True, check_lengths=False):
    """Forward over packed sequences: q_* [total_q, heads, d], k_* [total_k,
    heads, d], batch b owning rows cu_seqlens[b] .. cu_seqlens[b + 1] - 1.
    Returns (kl_rows, lse_t, lse_s, kl_sum) with the per-row outputs padded
    to [B, H, max_seqlen_q] (rows past a sequence's length are 0).  A sequence
    longer than its max_seqlen is cut to max_seqlen rows; check_lengths=True
    runs check_cu_seqlens first (a device synchronisation)."""
    import torch
    lib = load_library()
    (B, H, n_q, n_k, d_t, d_s), strides, heads = _inputs_varlen(q_t, k_t, q_s, k_s, cu_seqlens_q, cu_seqlens_k,
                                                                 max_seqlen_q, max_seqlen_k)
    if check_lengths:
        check_cu_seqlens(cu_seqlens_q, cu_seqlens_k, n_q, n_k, q_t.shape[0], k_t.shape[0])
    tau_t, tau_s = _taus(tau_t, tau_s, d_t, d_s)
    dev = q_t.device
    kl = torch.empty((B, H, n_q), dtype=torch.float32, device=dev)
    lt, ls = torch.empty_like(kl), torch.empty_like(kl)
    tot = torch.empty((1,), dtype=torch.float32, device=dev) if with_sum else None
    lay = StreamKLLayout(*heads, None, None, cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr())
    code = lib.streamkl_fwd_ex(q_t.data_ptr(), k_t.data_ptr(), q_s.data_ptr(), k_s.data_ptr(), _dtype_code(q_t), B, H,
                               n_q, n_k, d_t, d_s, strides, ctypes.byref(lay), tau_t, tau_s, int(bool(causal)),
                               kl.data_ptr(), lt.data_ptr(), ls.data_ptr(), tot.data_ptr() if tot is not None else None,
                               _stream_ptr(dev))
    _check("streamkl_fwd_ex", code)
    return kl, lt, ls, tot


def streamkl_bwd_varlen(q_t, k_t, q_s, k_s, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, lse_t, lse_s,
                        grad_rows=None, grad_scalar=1.0, tau_t=None, tau_s=None, causal=False, teacher=False,
                        kl_rows=None, check_lengths=False):
    """Backward over packed sequences: (dq, dk) packed like the inputs of the
    differentiated model (the student, or the teacher if teacher=True, which
    needs the forward's kl_rows).  Per-row arrays are [B, H, max_seqlen_q].
    The kernels write the rows some sequence owns; the outputs start zeroed,
    so packed rows that no sequence owns get zero gradients."""
    import torch
    lib = load_library()
    (B, H, n_q, n_k, d_t, d_s), strides, heads = _inputs_varlen(q_t, k_t, q_s, k_s, cu_seqlens_q, cu_seqlens_k,
                                                                 max_seqlen_q, max_seqlen_k)
    if check_lengths:
        check_cu_seqlens(cu_seqlens_q, cu_seqlens_k, n_q, n_k, q_t.shape[0], k_t.shape[0])
    tau_t, tau_s = _taus(tau_t, tau_s, d_t, d_s)
    dev = q_t.device
    rowargs = (("lse_t", lse_t), ("lse_s", lse_s)) + ((("kl_rows", kl_rows),) if teacher else ()) + \
        ((("grad_rows", grad_rows),) if grad_rows is not None else ())
    for name, t in rowargs:
        if t is None or t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (B, H, n_q):
            raise ValueError(f"{name} must be a contiguous fp32 [B, H, max_seqlen_q] tensor")
    if teacher:
        dq = torch.zeros((q_t.shape[0], heads[0], d_t), dtype=q_t.dtype, device=dev)
        dk = torch.zeros((k_t.shape[0], heads[1], d_t), dtype=q_t.dtype, device=dev)
    else:
        dq = torch.zeros((q_s.shape[0], heads[2], d_s), dtype=q_s.dtype, device=dev)
        dk = torch.zeros((k_s.shape[0], heads[3], d_s), dtype=q_s.dtype, device=dev)
    lay = StreamKLLayout(*heads, None, None, cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr())
    args = [q_t.data_ptr(), k_t.data_ptr(), q_s.data_ptr(), k_s.data_ptr(), _dtype_code(q_t), B, H, n_q, n_k, d_t,
            d_s, strides, ctypes.byref(lay), tau_t, tau_s, int(bool(causal)), lse_t.data_ptr(), lse_s.data_ptr()]
    g = grad_rows.data_ptr() if grad_rows is not None else None
    if teacher:
        code = lib.streamkl_bwd_teacher_ex(*args, kl_rows.data_ptr(), g, float(grad_scalar), dq.data_ptr(),
                                           dk.data_ptr(), None, 0, _stream_ptr(dev))
        _check("streamkl_bwd_teacher_ex", code)
    else:
        code = lib.streamkl_bwd_ex(*args, g, float(grad_scalar), dq.data_ptr(), dk.data_ptr(), None, 0,
                                   _stream_ptr(dev))
        _check("streamkl_bwd_ex", code)
    return dq, dk


def _autograd_function():
    import torch

    class StreamKLFunction(torch.autograd.Function):
        """Per-row attention KL with gradients for the student queries and keys,
        and for the teacher queries and keys when those require them.

        forward(q_t, k_t, q_s, k_s, tau_t, tau_s, causal) -> kl_rows [B, H, N_Q]
        """

        @staticmethod
        def forward(ctx, q_t, k_t, q_s, k_s, tau_t=None, tau_s=None, causal=False, seqlen_q=None, seqlen_k=None):
            kl, lt, ls, _ = streamkl_fwd(q_t, k_t, q_s, k_s, tau_t, tau_s, causal, with_sum=False,
                                         seqlen_q=seqlen_q, seqlen_k=seqlen_k)
            ctx.save_for_backward(q_t, k_t, q_s, k_s, lt, ls, kl)
            ctx.cfg = (tau_t, tau_s, causal, seqlen_q, seqlen_k)
            return kl

        @staticmethod
        def backward(ctx, g):
            q_t, k_t, q_s, k_s, lt, ls, kl = ctx.saved_tensors
            tau_t, tau_s, causal, sq, sk = ctx.cfg
            g = g.to(torch.float32).contiguous()
            dq_s = dk_s = dq_t = dk_t = None
            if ctx.needs_input_grad[2] or ctx.needs_input_grad[3]:
                dq_s, dk_s = streamkl_bwd(q_t, k_t, q_s, k_s, lt, ls, grad_rows=g,
                                          tau_t=tau_t, tau_s=tau_s, causal=causal, seqlen_q=sq, seqlen_k=sk)
            if ctx.needs_input_grad[0] or ctx.needs_input_grad[1]:
                dq_t, dk_t = streamkl_bwd_teacher(q_t, k_t, q_s, k_s, lt, ls, kl, grad_rows=g,
                                                  tau_t=tau_t, tau_s=tau_s, causal=causal, seqlen_q=sq, seqlen_k=sk)
            return dq_t, dk_t, dq_s, dk_s, None, None, None, None, None

    return StreamKLFunction


def _vocab_autograd_function():
    import torch

    class VocabKLFunction(torch.autograd.Function):
        """Per-row vocabulary KL with gradients for z_s, and for z_t when it
        requires them.  forward(z_t, z_s, temperature) -> kl_rows [...]"""

        @staticmethod
        def forward(ctx, z_t, z_s, temperature=1.0):
            kl, lt, ls, _ = streamkl_vocab_fwd(z_t, z_s, temperature, with_sum=False)
            ctx.save_for_backward(z_t, z_s, lt, ls, kl)
            ctx.temperature = temperature
            return kl

        @staticmethod
        def backward(ctx, g):
            z_t, z_s, lt, ls, kl = ctx.saved_tensors
            g = g.to(torch.float32).contiguous()
            want_t = ctx.needs_input_grad[0]
            if not (want_t or ctx.needs_input_grad[1]):
                return None, None, None
            out = streamkl_vocab_bwd(z_t, z_s, lt, ls, kl, ctx.temperature, grad_rows=g, teacher=want_t)
            dzs, dzt = out if want_t else (out, None)
            return dzt, (dzs if ctx.needs_input_grad[1] else None), None

    return VocabKLFunction


def _varlen_autograd_function():
    import torch

    class StreamKLVarlenFunction(torch.autograd.Function):
        """Per-row attention KL over packed sequences, with gradients for the
        student tensors and, when they require them, the teacher tensors.
        forward(q_t, k_t, q_s, k_s, cu_q, cu_k, max_q, max_k, tau_t, tau_s,
        causal) -> kl_rows [B, H, max_q]"""

        @staticmethod
        def forward(ctx, q_t, k_t, q_s, k_s, cu_q, cu_k, max_q, max_k, tau_t=None, tau_s=None, causal=False):
            kl, lt, ls, _ = streamkl_fwd_varlen(q_t, k_t, q_s, k_s, cu_q, cu_k, max_q, max_k, tau_t, tau_s, causal,
                                                with_sum=False)
            ctx.save_for_backward(q_t, k_t, q_s, k_s, cu_q, cu_k, lt, ls, kl)
            ctx.cfg = (max_q, max_k, tau_t, tau_s, causal)
            return kl

        @staticmethod
        def backward(ctx, g):
            q_t, k_t, q_s, k_s, cu_q, cu_k, lt, ls, kl = ctx.saved_tensors
            max_q, max_k, tau_t, tau_s, causal = ctx.cfg
            g = g.to(torch.float32).contiguous()
            dq_s = dk_s = dq_t = dk_t = None
            common = (q_t, k_t, q_s, k_s, cu_q, cu_k, max_q, max_k, lt, ls)
            if ctx.needs_input_grad[2] or ctx.needs_input_grad[3]:
                dq_s, dk_s = streamkl_bwd_varlen(*common, grad_rows=g, tau_t=tau_t, tau_s=tau_s, causal=causal)
            if ctx.needs_input_grad[0] or ctx.needs_input_grad[1]:
                dq_t, dk_t = streamkl_bwd_varlen(*common, grad_rows=g, tau_t=tau_t, tau_s=tau_s, causal=causal,
                                                 teacher=True, kl_rows=kl)
            return dq_t, dk_t, dq_s, dk_s, None, None, None, None, None, None, None

    return StreamKLVarlenFunction


_fn_cache = None
_varlen_fn_cache = None
_vocab_fn_cache = None


def attention_kl_varlen(q_t, k_t, q_s, k_s, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, tau_t=None,
                        tau_s=None, causal=False, check_lengths=False):
    """Differentiable per-row attention KL over packed sequences ([rows, heads,
    d] tensors, int32 offsets [B + 1]); returns [B, H, max_seqlen_q], rows past
    a sequence's length 0.  Packed rows that no sequence owns get zero
    gradients.  check_lengths=True checks the offsets on the host first (see
    check_cu_seqlens)."""
    global _varlen_fn_cache
    if _varlen_fn_cache is None:
        _varlen_fn_cache = _varlen_autograd_function()
    if check_lengths:
        check_cu_seqlens(cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, q_t.shape[0], k_t.shape[0])
    return _varlen_fn_cache.apply(q_t, k_t, q_s, k_s, cu_seqlens_q, cu_seqlens_k, int(max_seqlen_q),
                                  int(max_seqlen_k), tau_t, tau_s, causal)


def vocab_kl(z_t, z_s, temperature=1.0):
    """Differentiable per-row KL(softmax(z_t / T) || softmax(z_s / T)) over the
    last dimension (shape z_t.shape[:-1]); gradients flow to z_s and, when it
    requires them, to z_t.  The T^2 factor of the distillation loss is the
    caller's (multiply the result)."""
    global _vocab_fn_cache
    if _vocab_fn_cache is None:
        _vocab_fn_cache = _vocab_autograd_function()
    return _vocab_fn_cache.apply(z_t, z_s, temperature)


def attention_kl(q_t, k_t, q_s, k_s, tau_t=None, tau_s=None, causal=False, seqlen_q=None, seqlen_k=None):
    """Differentiable per-row attention KL(P_t || P_s) [B, H, N_Q]; gradients
    flow to whichever of q_s, k_s, q_t, k_t require them.  The reverse
    divergence KL(P_s || P_t) is attention_kl(q_s, k_s, q_t, k_t, tau_s, tau_t).
    Grouped heads and per-batch lengths as in streamkl_fwd."""
    global _fn_cache
    if _fn_cache is None:
        _fn_cache = _autograd_function()
    return _fn_cache.apply(q_t, k_t, q_s, k_s, tau_t, tau_s, causal, seqlen_q, seqlen_k)


__all__ = [
    "streamkl_fwd", "streamkl_fwd_noalloc", "streamkl_fwd_partial", "streamkl_fwd_merge", "streamkl_bwd", "streamkl_bwd_teacher",
    "attention_kl", "streamkl_fwd_varlen", "streamkl_bwd_varlen", "attention_kl_varlen", "check_cu_seqlens",
    "streamkl_vocab_fwd",
    "streamkl_vocab_bwd", "streamkl_vocab_fwd_bwd", "vocab_kl", "load_library", "supported", "status_string",
    "StreamKLError", "STREAMKL_F32", "STREAMKL_BF16"
]
