"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
entry point include/streamkl.h declares, and rejects bad arguments with the
documented status before making any HIP call (so fake device addresses are safe)."""
import ctypes
import os
import re

import pytest

import attention_kl_divergence_amd as skl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "streamkl.h")

A = 0x7f0000000000  # fake, 256-byte aligned "device" addresses; never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(streamkl_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = skl.load_library()
    names = declared_functions()
    assert {"streamkl_fwd", "streamkl_bwd", "streamkl_bwd_workspace_size", "streamkl_status_string",
            "streamkl_supported"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_support_matrix():
    assert skl.status_string(0) == "ok"
    assert "invalid" in skl.status_string(1)
    assert "unsupported" in skl.status_string(2)
    for code in (skl.STREAMKL_BF16, skl.STREAMKL_F32):
        for dt in (64, 128):
            for ds in (64, 128):
                assert skl.supported(code, dt, ds)
        assert not skl.supported(code, 96, 128)
        assert not skl.supported(code, 128, 32)
    assert not skl.supported(9, 128, 128)
    assert skl.load_library().streamkl_bwd_workspace_size(2, 16, 16384, 16384, 128, 128, 1, 0) == 0


def fwd(**kw):
    a = dict(q_t=A, k_t=A + 0x100000, q_s=A + 0x200000, k_s=A + 0x300000, dtype=skl.STREAMKL_BF16,
             B=2, H=3, n_q=100, n_k=77, d_t=128, d_s=64, strides=None, tau_t=0.088, tau_s=0.125, causal=0,
             kl=A + 0x400000, lt=A + 0x500000, ls=A + 0x600000, tot=None, stream=None)
    a.update(kw)
    st = None
    if a["strides"] is not None:
        st = (ctypes.c_int64 * 12)(*a["strides"])
    return skl.load_library().streamkl_fwd(a["q_t"], a["k_t"], a["q_s"], a["k_s"], a["dtype"], a["B"], a["H"],
                                           a["n_q"], a["n_k"], a["d_t"], a["d_s"], st, a["tau_t"], a["tau_s"],
                                           a["causal"], a["kl"], a["lt"], a["ls"], a["tot"], a["stream"])


def bwd(**kw):
    a = dict(q_t=A, k_t=A + 0x100000, q_s=A + 0x200000, k_s=A + 0x300000, dtype=skl.STREAMKL_BF16,
             B=2, H=3, n_q=100, n_k=77, d_t=128, d_s=64, strides=None, tau_t=0.088, tau_s=0.125, causal=0,
             lt=A + 0x500000, ls=A + 0x600000, g=None, gs=1.0, dq=A + 0x700000, dk=A + 0x800000, stream=None)
    a.update(kw)
    return skl.load_library().streamkl_bwd(a["q_t"], a["k_t"], a["q_s"], a["k_s"], a["dtype"], a["B"], a["H"],
                                           a["n_q"], a["n_k"], a["d_t"], a["d_s"], None, a["tau_t"], a["tau_s"],
                                           a["causal"], a["lt"], a["ls"], a["g"], a["gs"], a["dq"], a["dk"],
                                           a["stream"])


INV, UNS = skl.STREAMKL_ERR_INVALID, skl.STREAMKL_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,code", [
    (dict(q_t=None), INV), (dict(k_s=None), INV), (dict(kl=None), INV), (dict(lt=None), INV),
    (dict(B=0), INV), (dict(H=-1), INV), (dict(n_q=0), INV), (dict(n_k=0), INV),
    (dict(tau_t=-0.1), INV), (dict(tau_s=float("nan")), INV), (dict(tau_t=float("inf")), INV),
    (dict(causal=1), INV),            # n_q = 100 > n_k = 77
    (dict(causal=2, n_k=200), INV),
    (dict(dtype=5), INV),
    (dict(d_t=96), UNS), (dict(d_s=32), UNS), (dict(d_t=0), INV),
    (dict(q_s=A + 8), INV),           # not 16-byte aligned
    (dict(strides=[3 * 100 * 128, 100 * 128, 120] + [0, 0, 128] * 3), INV),  # 120 bf16 = 240 B ok, k_t b/h 0 ok ...
    (dict(strides=[3 * 100 * 128, 100 * 128, 100] + [0, 0, 128] * 3), INV),  # row stride < d_t
    (dict(strides=[3 * 100 * 128, 100 * 128, 132] + [0, 0, 128] * 3), INV),  # 264 B rows, not 16-B aligned
    (dict(strides=[0, 0, 128] * 3 + [0, 0, 1 << 25]), INV),  # k_s rows 64 MiB apart: tile offsets past 32 bits
    (dict(strides=[0, 0, 1 << 25] + [0, 0, 128] * 3, dtype=skl.STREAMKL_F32, d_t=64), INV),  # 128 MiB fp32 rows
    (dict(B=1024, H=1024, n_q=4096, n_k=4096), INV),  # 2^20 heads x 64 blocks x 256 threads >= 2^32 work-items
    (dict(n_q=(1 << 30), n_k=(1 << 30), B=1, H=1), INV),  # row indices beyond 32-bit kernel arithmetic
])
def test_fwd_rejects_bad_arguments_before_any_hip_call(kw, code):
    assert fwd(**kw) == code


def test_bwd_rejects_bad_arguments_before_any_hip_call():
    assert bwd(lt=None) == INV
    assert bwd(dq=None) == INV
    assert bwd(dk=A + 4) == INV
    assert bwd(gs=float("nan")) == INV
    assert bwd(causal=1) == INV
    assert bwd(d_s=80) == UNS
    assert bwd(tau_s=-1.0) == INV
    assert bwd(B=1024, H=1024, n_q=4096, n_k=4096) == INV


def test_python_binding_fails_loudly_without_device_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        skl.streamkl_fwd(x, x, x, x)


def test_bwd_teacher_rejects_bad_arguments_before_any_hip_call():
    lib = skl.load_library()

    def call(**kw):
        a = dict(q_t=A, k_t=A + 0x100000, q_s=A + 0x200000, k_s=A + 0x300000, dtype=skl.STREAMKL_BF16,
                 B=2, H=3, n_q=100, n_k=77, d_t=128, d_s=64, tau_t=0.088, tau_s=0.125, causal=0,
                 lt=A + 0x500000, ls=A + 0x600000, kl=A + 0x680000, g=None, gs=1.0,
                 dq=A + 0x700000, dk=A + 0x800000)
        a.update(kw)
        return lib.streamkl_bwd_teacher(a["q_t"], a["k_t"], a["q_s"], a["k_s"], a["dtype"], a["B"], a["H"],
                                        a["n_q"], a["n_k"], a["d_t"], a["d_s"], None, a["tau_t"], a["tau_s"],
                                        a["causal"], a["lt"], a["ls"], a["kl"], a["g"], a["gs"], a["dq"], a["dk"],
                                        None)
    assert call(kl=None) == INV
    assert call(lt=None) == INV
    assert call(dq=None) == INV
    assert call(dk=A + 8) == INV
    assert call(gs=float("inf")) == INV
    assert call(causal=1) == INV
    assert call(d_t=32) == UNS
    assert call(tau_t=-0.5) == INV


def test_split_forward_pieces_reject_bad_arguments_before_any_hip_call():
    lib = skl.load_library()
    base = dict(q_t=A, k_t=A + 0x100000, q_s=A + 0x200000, k_s=A + 0x300000, dtype=skl.STREAMKL_BF16,
                B=2, H=3, n_q=100, n_k=300, d_t=128, d_s=64, tau_t=0.088, tau_s=0.125, causal=0)

    def partial(k0, k1, st=A + 0x400000, **kw):
        a = dict(base); a.update(kw)
        return lib.streamkl_fwd_partial(a["q_t"], a["k_t"], a["q_s"], a["k_s"], a["dtype"], a["B"], a["H"],
                                        a["n_q"], a["n_k"], a["d_t"], a["d_s"], None, a["tau_t"], a["tau_s"],
                                        a["causal"], k0, k1, st, None)
    assert partial(16, 64) == INV       # k_begin not a multiple of 32
    assert partial(0, 70) == INV        # k_end neither a multiple of 32 nor n_k
    assert partial(64, 64) == INV       # empty range
    assert partial(0, 301) == INV       # beyond n_k
    assert partial(0, 64, st=None) == INV
    assert partial(0, 64, st=A + 4) == INV
    assert partial(0, 64, d_t=48) == UNS

    def split(n, ws=A + 0x500000, nbytes=1 << 30, **kw):
        a = dict(base); a.update(kw)
        return lib.streamkl_fwd_split(a["q_t"], a["k_t"], a["q_s"], a["k_s"], a["dtype"], a["B"], a["H"],
                                      a["n_q"], a["n_k"], a["d_t"], a["d_s"], None, a["tau_t"], a["tau_s"],
                                      a["causal"], n, ws, nbytes, A + 0x600000, A + 0x700000, A + 0x800000, None,
                                      None)
    need = lib.streamkl_fwd_split_workspace_size(2, 3, 100, 4)
    assert need == 4 * 2 * 3 * 100 * 6 * 4
    assert split(4, nbytes=need - 1) == skl.STREAMKL_ERR_WORKSPACE
    assert split(4, ws=None) == INV
    assert split(0) == INV and split(65) == INV
    assert split(4, tau_s=-1.0) == INV
    assert lib.streamkl_fwd_merge(None, 2, 100, 0.1, 0.1, A, A, A, None, None) == INV
    assert lib.streamkl_fwd_merge(A, 0, 100, 0.1, 0.1, A, A, A, None, None) == INV
    assert lib.streamkl_fwd_merge(A, 2, 0, 0.1, 0.1, A, A, A, None, None) == INV
    # the suggested split count: 1 when the unsplit forward fills the GPU (or
    # exactly fills whole rounds of 768 workgroups), more for small launches,
    # never below 16 key tiles per split; causal launches only below one round
    assert lib.streamkl_fwd_split_count(2, 16, 16384, 16384, 0) == 1
    assert lib.streamkl_fwd_split_count(4, 12, 2048, 2048, 0) == 1  # 768 blocks: one full round
    assert lib.streamkl_fwd_split_count(2, 16, 4096, 4096, 0) == 2
    assert lib.streamkl_fwd_split_count(8, 16, 512, 16384, 0) == 4
    assert lib.streamkl_fwd_split_count(1, 8, 32768, 32768, 1) == 1
    assert lib.streamkl_fwd_split_count(1, 2, 4096, 4096, 1) == 8  # 64 blocks, causal
    assert lib.streamkl_fwd_split_count(1, 1, 128, 128, 0) == 1


def test_vocab_entry_points_reject_bad_arguments_before_any_hip_call():
    lib = skl.load_library()
    BF = skl.STREAMKL_BF16
    zt, zs, out = A, A + 0x10000000, A + 0x20000000

    def fwd(z_t=zt, z_s=zs, dtype=BF, rows=4, V=1000, ld_t=1000, ld_s=1000, T=2.0, kl=out, lt=out + 64,
            ls=out + 128):
        return lib.streamkl_vocab_fwd(z_t, z_s, dtype, rows, V, ld_t, ld_s, T, kl, lt, ls, None, None)
    assert fwd(z_t=None) == INV and fwd(z_s=None) == INV
    assert fwd(dtype=7) == INV
    assert fwd(rows=0) == INV and fwd(V=0) == INV and fwd(V=(1 << 30) + 1, ld_t=1 << 31, ld_s=1 << 31) == INV
    assert fwd(ld_t=999) == INV and fwd(ld_s=10) == INV
    assert fwd(T=0.0) == INV and fwd(T=-1.0) == INV and fwd(T=float("nan")) == INV and fwd(T=2e6) == INV
    assert fwd(T=float("inf")) == INV
    assert fwd(z_t=zt + 1) == INV                      # not aligned to the bf16 element
    assert fwd(dtype=skl.STREAMKL_F32, z_s=zs + 2) == INV  # not aligned to the fp32 element
    assert fwd(kl=None) == INV and fwd(lt=None) == INV and fwd(ls=None) == INV
    assert fwd(rows=1 << 60, V=8192, ld_t=8192, ld_s=8192) == INV   # row offsets beyond the address space

    def bwd(lt=out, ls=out + 64, kl=None, g=None, dzs=out + 0x1000, dzt=None, **kw):
        a = dict(z_t=zt, z_s=zs, dtype=BF, rows=4, V=1000, ld_t=1000, ld_s=1000, T=2.0); a.update(kw)
        return lib.streamkl_vocab_bwd(a["z_t"], a["z_s"], a["dtype"], a["rows"], a["V"], a["ld_t"], a["ld_s"],
                                      a["T"], lt, ls, kl, g, 1.0, dzs, dzt, None)
    assert bwd(lt=None) == INV and bwd(ls=None) == INV
    assert bwd(dzs=None) == INV and bwd(dzs=out + 0x1001) == INV
    assert bwd(dzt=out + 0x2000) == INV                # teacher gradients need kl_rows
    assert bwd(dzt=out + 0x2001, kl=out + 128) == INV  # misaligned dz_t
    assert bwd(T=0.0) == INV and bwd(rows=0) == INV

    def fused(kl=out, dzs=out + 0x1000, **kw):
        a = dict(z_t=zt, z_s=zs, dtype=BF, rows=4, V=1000, ld_t=1000, ld_s=1000, T=2.0); a.update(kw)
        return lib.streamkl_vocab_fwd_bwd(a["z_t"], a["z_s"], a["dtype"], a["rows"], a["V"], a["ld_t"], a["ld_s"],
                                          a["T"], None, 1.0, kl, out + 64, out + 128, None, dzs, None, None)
    assert fused(kl=None) == INV and fused(dzs=None) == INV and fused(V=0) == INV and fused(ld_s=5) == INV


def test_vocab_binding_fails_loudly_without_device_tensors():
    import torch
    z = torch.zeros(2, 16)
    with pytest.raises(ValueError):
        skl.streamkl_vocab_fwd(z, z)
    with pytest.raises(ValueError):
        skl.vocab_kl(z, z)


def test_layout_entry_points_reject_bad_layouts_before_any_hip_call():
    lib = skl.load_library()

    def fwd(hq_t=0, hk_t=0, hq_s=0, hk_s=0, sq=None, sk=None, H=8):
        lay = skl.StreamKLLayout(hq_t, hk_t, hq_s, hk_s, sq, sk)
        return lib.streamkl_fwd_ex(A, A + 0x100000, A + 0x200000, A + 0x300000, skl.STREAMKL_BF16, 2, H, 100, 300,
                                   128, 64, None, ctypes.byref(lay), 0.088, 0.125, 0, A + 0x400000, A + 0x500000,
                                   A + 0x600000, None, None)
    assert fwd(hq_t=-1) == INV
    assert fwd(hq_s=3) == INV           # 3 does not divide H = 8
    assert fwd(hq_t=4, hk_t=8) == INV   # more key heads than query heads
    assert fwd(hq_s=4, hk_s=3) == INV   # 3 does not divide 4
    assert fwd(sq=A + 2) == INV         # misaligned length array
    assert fwd(sk=A + 6) == INV
    assert fwd(hq_t=4, hk_t=2, hq_s=8, hk_s=1, H=0) == INV

    def bwd(first, **kw):
        lay = skl.StreamKLLayout(kw.get("hq_t", 0), kw.get("hk_t", 0), kw.get("hq_s", 0), kw.get("hk_s", 0), None,
                                 None)
        if first:
            return lib.streamkl_bwd_teacher_ex(A, A + 0x100000, A + 0x200000, A + 0x300000, skl.STREAMKL_BF16, 2, 8,
                                               100, 300, 128, 64, None, ctypes.byref(lay), 0.088, 0.125, 0, A, A,
                                               kw.get("kl", A), None, 1.0, A + 0x700000, A + 0x800000, None, 0, None)
        return lib.streamkl_bwd_ex(A, A + 0x100000, A + 0x200000, A + 0x300000, skl.STREAMKL_BF16, 2, 8, 100, 300,
                                   128, 64, None, ctypes.byref(lay), 0.088, 0.125, 0, A, A, None, 1.0,
                                   kw.get("dq", A + 0x700000), A + 0x800000, kw.get("ws", None), 1 << 30, None)
    assert bwd(False, hk_s=5) == INV
    assert bwd(False, hk_s=2, dq=None) == INV
    assert bwd(True, hk_t=2, kl=None) == INV
    assert bwd(True, hq_t=16) == INV    # 16 does not divide H = 8
    assert bwd(False, hk_s=2, ws=A + 8) == INV   # misaligned workspace
    # workspace sizes: none for single heads or plentiful blocks, partial sums for a long group over few blocks
    one = skl.StreamKLLayout(0, 0, 0, 1, None, None)
    four = skl.StreamKLLayout(0, 0, 0, 4, None, None)
    assert lib.streamkl_bwd_ex_workspace_size(2, 16, 16384, 16384, 128, 128, None, 0) == 0
    # groups of 4 over 2 x 4 x 128 key blocks: already 1024 work items, no split
    assert lib.streamkl_bwd_ex_workspace_size(2, 16, 16384, 16384, 128, 128, ctypes.byref(four), 0) == 0
    # one key head: 2 x 128 key blocks, groups of 16 split 4 ways: 4 partial dK_s tensors in fp32
    n16 = lib.streamkl_bwd_ex_workspace_size(2, 16, 16384, 16384, 128, 128, ctypes.byref(one), 0)
    assert n16 == 4 * 2 * 1 * 16384 * 128 * 4
    # 2 x 32 key blocks at 4K: split 16 ways
    n4 = lib.streamkl_bwd_ex_workspace_size(2, 16, 4096, 4096, 128, 128, ctypes.byref(one), 0)
    assert n4 == 16 * 2 * 1 * 4096 * 128 * 4
    # the teacher's heads decide the teacher gradients' split: none here
    assert lib.streamkl_bwd_ex_workspace_size(2, 16, 4096, 4096, 128, 128, ctypes.byref(one), 1) == 0


def test_packed_sequence_layout_is_validated_before_any_hip_call():
    lib = skl.load_library()

    def fwd(sq=None, sk=None, cq=None, ck=None):
        lay = skl.StreamKLLayout(0, 0, 0, 0, sq, sk, cq, ck)
        return lib.streamkl_fwd_ex(A, A + 0x100000, A + 0x200000, A + 0x300000, skl.STREAMKL_BF16, 2, 4, 100, 300,
                                   128, 64, None, ctypes.byref(lay), 0.088, 0.125, 0, A + 0x400000, A + 0x500000,
                                   A + 0x600000, None, None)
    assert fwd(cq=A + 2) == INV                 # misaligned offsets
    assert fwd(ck=A + 6) == INV
    assert fwd(sq=A, cq=A + 64) == INV          # a kind cannot be both padded with lengths and packed
    assert fwd(sk=A, ck=A + 64) == INV


def test_noalloc_split_forward_rejects_on_the_host():
    """streamkl_fwd_split_noalloc: states past its fixed scratch array give
    STREAMKL_ERR_WORKSPACE, and bad arguments INVALID, before any HIP call."""
    lib = skl.load_library()
    big = (64, 16, 4096, 8)  # 768 MiB of split states
    assert lib.streamkl_fwd_split_workspace_size(big[0], big[1], big[2], big[3]) > skl.NOALLOC_SCRATCH_BYTES

    def call(B, H, n_q, n_split, q_t=A, kl=A + 0x400000, tau=0.088):
        return lib.streamkl_fwd_split_noalloc(q_t, A + 0x100000, A + 0x200000, A + 0x300000, skl.STREAMKL_BF16, B, H,
                                              n_q, 8192, 128, 128, None, tau, tau, 0, n_split, kl, A + 0x500000,
                                              A + 0x600000, None, None)
    assert call(*big) == skl.STREAMKL_ERR_WORKSPACE
    assert call(2, 2, 64, 2, q_t=None) == INV
    assert call(2, 2, 64, 2, kl=None) == INV
    assert call(2, 2, 64, 0) == INV
    assert call(2, 2, 64, 65) == INV
    assert call(2, 2, 64, 2, tau=-1.0) == INV
