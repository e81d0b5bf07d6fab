"""GPU parity of grouped heads and per-batch lengths (streamkl_fwd_ex,
streamkl_bwd_ex, streamkl_bwd_teacher_ex) against the fp64 oracle.

The reference is the oracle applied to the definition of the layout: KL head h
reads head h // (H / heads) of each tensor (np.repeat over the head axis), each
batch is cut to its valid lengths (under a causal mask with more valid
queries than keys, the first rows have no key and are empty), and the gradient
of a shared head is the sum over the KL heads that read it."""
import numpy as np
import pytest

import attention_kl_divergence_amd as skl
import oracle
from tests.gpu_util import check_grad, check_kl, check_lse, check_sum

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _round_bf16(a):
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _draw(seed, B, heads, n_q, n_k, d_t, d_s, dtype, sigma=0.3):
    """Teacher and student tensors with their own head counts (student = a
    noisy copy of the teacher where the head counts allow)."""
    rng = np.random.default_rng(seed)
    hq_t, hk_t, hq_s, hk_s = heads
    x = {"q_t": rng.standard_normal((B, hq_t, n_q, d_t), dtype=np.float32),
         "k_t": rng.standard_normal((B, hk_t, n_k, d_t), dtype=np.float32),
         "q_s": rng.standard_normal((B, hq_s, n_q, d_s), dtype=np.float32),
         "k_s": rng.standard_normal((B, hk_s, n_k, d_s), dtype=np.float32)}
    if d_t == d_s and hq_t == hq_s:
        x["q_s"] = (x["q_t"] + np.float32(sigma) * x["q_s"]).astype(np.float32)
    if d_t == d_s and hk_t == hk_s:
        x["k_s"] = (x["k_t"] + np.float32(sigma) * x["k_s"]).astype(np.float32)
    if dtype == "bf16":
        x = {k: _round_bf16(v) for k, v in x.items()}
    return x


def _reference(x, H, tau_t, tau_s, causal, lq=None, lk=None, g=None):
    xo = {k: np.repeat(v.astype(np.float64), H // v.shape[1], axis=1) for k, v in x.items()}
    B, _, n_q, d_t = xo["q_t"].shape
    n_k, d_s = xo["k_t"].shape[2], xo["q_s"].shape[3]
    kl = np.zeros((B, H, n_q)); lt = np.zeros_like(kl); ls = np.zeros_like(kl)
    dqs = np.zeros((B, H, n_q, d_s)); dks = np.zeros((B, H, n_k, d_s))
    dqt = np.zeros((B, H, n_q, d_t)); dkt = np.zeros((B, H, n_k, d_t))
    for b in range(B):
        nq = n_q if lq is None else int(lq[b])
        nk = n_k if lk is None else int(lk[b])
        q0 = nq - nk if (causal and nq > nk) else 0  # rows before q0 have no allowed key
        if nq - q0 <= 0 or nk <= 0:
            continue
        a = [xo["q_t"][b:b + 1, :, q0:nq], xo["k_t"][b:b + 1, :, :nk], xo["q_s"][b:b + 1, :, q0:nq],
             xo["k_s"][b:b + 1, :, :nk]]
        a = [np.ascontiguousarray(t) for t in a]
        rkl, rlt, rls, _ = oracle.fwd(*a, tau_t, tau_s, causal)
        kl[b, :, q0:nq], lt[b, :, q0:nq], ls[b, :, q0:nq] = rkl[0], rlt[0], rls[0]
        gb = None if g is None else np.ascontiguousarray(g[b:b + 1, :, q0:nq], dtype=np.float64)
        rdq, rdk = oracle.bwd(*a, tau_t, tau_s, causal, g=gb)
        dqs[b, :, q0:nq], dks[b, :, :nk] = rdq[0], rdk[0]
        tdq, tdk = oracle.bwd_teacher(*a, tau_t, tau_s, causal, g=gb)
        dqt[b, :, q0:nq], dkt[b, :, :nk] = tdq[0], tdk[0]

    def fold(gr, h):
        return gr.reshape(gr.shape[0], h, H // h, *gr.shape[2:]).sum(axis=2)
    return dict(kl=kl, lse_t=lt, lse_s=ls, dq_s=fold(dqs, x["q_s"].shape[1]), dk_s=fold(dks, x["k_s"].shape[1]),
                dq_t=fold(dqt, x["q_t"].shape[1]), dk_t=fold(dkt, x["k_t"].shape[1]))


def _gpu(x, dtype, causal, lq=None, lk=None, g=None, g_scalar=1.0, tau=(None, None)):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    d = {k: torch.from_numpy(np.ascontiguousarray(v)).to(tdt).cuda() for k, v in x.items()}
    sq = None if lq is None else torch.tensor(lq, dtype=torch.int32, device="cuda")
    sk = None if lk is None else torch.tensor(lk, dtype=torch.int32, device="cuda")
    args = (d["q_t"], d["k_t"], d["q_s"], d["k_s"])
    kl, lt, ls, tot = skl.streamkl_fwd(*args, tau[0], tau[1], causal, seqlen_q=sq, seqlen_k=sk)
    gt = None if g is None else torch.from_numpy(np.ascontiguousarray(g, dtype=np.float32)).cuda()
    dqs, dks = skl.streamkl_bwd(*args, lt, ls, grad_rows=gt, grad_scalar=g_scalar, tau_t=tau[0], tau_s=tau[1],
                                causal=causal, seqlen_q=sq, seqlen_k=sk)
    dqt, dkt = skl.streamkl_bwd_teacher(*args, lt, ls, kl, grad_rows=gt, grad_scalar=g_scalar, tau_t=tau[0],
                                        tau_s=tau[1], causal=causal, seqlen_q=sq, seqlen_k=sk)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    return dict(kl=f(kl), lse_t=f(lt), lse_s=f(ls), sum=float(tot.item()), dq_s=f(dqs), dk_s=f(dks), dq_t=f(dqt),
                dk_t=f(dkt))


# (name, B, heads (q_t, k_t, q_s, k_s), n_q, n_k, d_t, d_s, dtype, causal, lengths (q, k) or None)
CASES = [
    ("student_gqa4_bf16", 2, (8, 8, 8, 2), 200, 300, 128, 64, "bf16", False, None),
    ("both_gqa_f32_causal", 2, (4, 2, 4, 1), 130, 130, 64, 64, "f32", True, None),
    ("student_fewer_q_heads_bf16", 1, (8, 8, 4, 2), 160, 200, 128, 128, "bf16", False, None),
    ("teacher_fewer_q_heads_bf16_causal", 2, (2, 1, 4, 4), 100, 140, 64, 128, "bf16", True, None),
    ("lengths_bf16", 3, (4, 4, 4, 4), 256, 320, 128, 128, "bf16", False, ([200, 17, 0], [300, 40, 5])),
    ("lengths_causal_f32", 3, (2, 2, 2, 2), 160, 192, 64, 64, "f32", True, ([150, 64, 100], [192, 64, 37])),
    ("lengths_gqa_bf16_causal", 2, (8, 4, 4, 1), 200, 256, 128, 64, "bf16", True, ([199, 60], [256, 61])),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_grouped_and_lengths_match_oracle(case):
    name, B, heads, n_q, n_k, d_t, d_s, dtype, causal, lens = case
    print(f"[grouped] {case}", flush=True)
    H = max(heads[0], heads[2])
    x = _draw(100 + [c[0] for c in CASES].index(name), B, heads, n_q, n_k, d_t, d_s, dtype)
    lq, lk = (None, None) if lens is None else lens
    # per-row upstream weights of both signs: shared query heads fold KL heads of different signs
    g = np.random.default_rng(7).standard_normal((B, H, n_q)).astype(np.float32)
    tau_t, tau_s = float(np.float32(1 / np.sqrt(d_t))), float(np.float32(1 / np.sqrt(d_s)))
    out = _gpu(x, dtype, causal, lq, lk, g=g)
    ref = _reference(x, H, tau_t, tau_s, causal, lq, lk, g=g)
    check_kl(out["kl"], ref["kl"], dtype, f"{name} kl")
    check_lse(out["lse_t"], ref["lse_t"], dtype, f"{name} lse_t")
    check_lse(out["lse_s"], ref["lse_s"], dtype, f"{name} lse_s")
    check_sum(out["sum"], ref["kl"], dtype)
    for k in ("dq_s", "dk_s", "dq_t", "dk_t"):
        assert out[k].shape == ref[k].shape, (k, out[k].shape, ref[k].shape)
        check_grad(out[k], ref[k], dtype, f"{name} {k}")
    if lens is not None:
        # rows and keys past the valid lengths: KL 0 and zero gradients, exactly
        for b in range(B):
            assert not np.any(out["kl"][b, :, lq[b]:]) and not np.any(out["lse_t"][b, :, lq[b]:])
            assert not np.any(out["dq_s"][b, :, lq[b]:]) and not np.any(out["dk_s"][b, :, lk[b]:])
            assert not np.any(out["dq_t"][b, :, lq[b]:]) and not np.any(out["dk_t"][b, :, lk[b]:])


def test_grouped_scalar_upstream_gradient():
    B, heads, n_q, n_k = 2, (8, 8, 4, 2), 96, 160
    x = _draw(11, B, heads, n_q, n_k, 128, 128, "bf16")
    out = _gpu(x, "bf16", False, g=None, g_scalar=-1.5)
    ref = _reference(x, 8, float(np.float32(1 / np.sqrt(128))), float(np.float32(1 / np.sqrt(128))), False,
                     g=np.full((B, 8, n_q), -1.5))
    for k in ("dq_s", "dk_s", "dq_t", "dk_t"):
        check_grad(out[k], ref[k], "bf16", f"scalar {k}")


def test_equal_heads_through_the_layout_match_the_plain_entry_points():
    """A layout that changes nothing (equal heads, full lengths) gives the same
    bits as the plain entry points."""
    B, heads, n_q, n_k = 2, (4, 4, 4, 4), 130, 200
    x = _draw(12, B, heads, n_q, n_k, 128, 128, "bf16")
    d = {k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in x.items()}
    args = (d["q_t"], d["k_t"], d["q_s"], d["k_s"])
    full_q = torch.full((B,), n_q, dtype=torch.int32, device="cuda")
    full_k = torch.full((B,), n_k, dtype=torch.int32, device="cuda")
    a = skl.streamkl_fwd(*args, causal=True, split=1)
    b = skl.streamkl_fwd(*args, causal=True, seqlen_q=full_q, seqlen_k=full_k)
    ga = skl.streamkl_bwd(*args, a[1], a[2], causal=True)
    gb = skl.streamkl_bwd(*args, b[1], b[2], causal=True, seqlen_q=full_q, seqlen_k=full_k)
    torch.cuda.synchronize()
    for u, v in zip(tuple(a[:3]) + tuple(ga), tuple(b[:3]) + tuple(gb)):
        assert torch.equal(u, v)


def test_grouped_autograd():
    B, heads, n_q, n_k = 1, (4, 4, 4, 2), 64, 96
    x = _draw(13, B, heads, n_q, n_k, 64, 64, "f32")
    d = {k: torch.from_numpy(v).cuda().requires_grad_(k.endswith("_s")) for k, v in x.items()}
    sk = torch.tensor([80], dtype=torch.int32, device="cuda")
    kl = skl.attention_kl(d["q_t"], d["k_t"], d["q_s"], d["k_s"], seqlen_k=sk)
    kl.sum().backward()
    torch.cuda.synchronize()
    t = float(np.float32(1 / 8.0))
    ref = _reference(x, 4, t, t, False, lk=[80], g=np.ones((B, 4, n_q)))
    check_kl(kl.detach().cpu().numpy(), ref["kl"], "f32", "autograd kl")
    check_grad(d["q_s"].grad.cpu().numpy(), ref["dq_s"], "f32", "autograd dq_s")
    check_grad(d["k_s"].grad.cpu().numpy(), ref["dk_s"], "f32", "autograd dk_s")
    assert d["k_s"].grad.shape == (B, 2, n_k, 64)


@pytest.mark.parametrize("causal", [False, True])
def test_split_groups_equal_unsplit_and_oracle(causal):
    """One key head shared by all 16 query heads of the student (and of the
    teacher): the key-major blocks are few, so each head group is split over
    several blocks writing fp32 partial sums to the workspace.  The split and
    unsplit launches agree to rounding, and both match the oracle, for
    student and teacher gradients with per-row weights of both signs."""
    import ctypes
    B, H, n = 1, 16, 256
    heads = (H, 1, H, 1)
    x = _draw(21 + causal, B, heads, n, n, 128, 128, "bf16")
    g = np.random.default_rng(8).standard_normal((B, H, n)).astype(np.float32)
    t = float(np.float32(1 / np.sqrt(128)))
    ref = _reference(x, H, t, t, causal, g=g)
    d = {k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in x.items()}
    kl, lt, ls, _ = skl.streamkl_fwd(d["q_t"], d["k_t"], d["q_s"], d["k_s"], causal=causal)
    gt = torch.from_numpy(g).cuda()
    lib = skl.load_library()
    lay = skl.StreamKLLayout(*heads, None, None)
    strides = (ctypes.c_int64 * 12)(*[s for k in ("q_t", "k_t", "q_s", "k_s") for s in d[k].stride()[:3]])
    outs = {}
    for first in (0, 1):
        wsb = int(lib.streamkl_bwd_ex_workspace_size(B, H, n, n, 128, 128, ctypes.byref(lay), first))
        assert wsb > 0
        ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
        for split in (False, True):
            dq = torch.empty_like(d["q_t" if first else "q_s"])
            dk = torch.empty_like(d["k_t" if first else "k_s"])
            args = [d["q_t"].data_ptr(), d["k_t"].data_ptr(), d["q_s"].data_ptr(), d["k_s"].data_ptr(),
                    skl.STREAMKL_BF16, B, H, n, n, 128, 128, strides, ctypes.byref(lay), t, t, int(causal),
                    lt.data_ptr(), ls.data_ptr()]
            wsp = (ws.data_ptr(), wsb) if split else (None, 0)
            stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            if first:
                rc = lib.streamkl_bwd_teacher_ex(*args, kl.data_ptr(), gt.data_ptr(), 1.0, dq.data_ptr(),
                                                 dk.data_ptr(), *wsp, stream)
            else:
                rc = lib.streamkl_bwd_ex(*args, gt.data_ptr(), 1.0, dq.data_ptr(), dk.data_ptr(), *wsp, stream)
            assert rc == 0, skl.status_string(rc)
            torch.cuda.synchronize()
            outs[(first, split)] = (dq.float().cpu().numpy().astype(np.float64),
                                    dk.float().cpu().numpy().astype(np.float64))
    for first, (nq_, nk_) in ((0, ("dq_s", "dk_s")), (1, ("dq_t", "dk_t"))):
        for split in (False, True):
            check_grad(outs[(first, split)][0], ref[nq_], "bf16", f"{nq_} split={split}")
            check_grad(outs[(first, split)][1], ref[nk_], "bf16", f"{nk_} split={split}")
        a, b = outs[(first, False)][1], outs[(first, True)][1]
        assert np.linalg.norm(a - b) <= 4e-3 * np.linalg.norm(a)


def _identities_grouped(xo, dq, dk, hq, hk):
    """At any size: sum_j dK_s[j] = 0 per key head, and per key head the sum
    over its query heads of <Q_s, dQ_s> equals <K_s, dK_s>."""
    B = dq.shape[0]
    g = hq // hk
    for b in range(B):
        for j in range(hk):
            nrm = np.linalg.norm(dk[b, j])
            assert np.linalg.norm(dk[b, j].sum(axis=0)) <= 1e-2 * nrm + 1e-12
            lhs = sum(float(np.sum(xo["q_s"][b, h] * dq[b, h])) for h in range(j * g, (j + 1) * g))
            rhs = float(np.sum(xo["k_s"][b, j] * dk[b, j]))
            scale = sum(np.linalg.norm(xo["q_s"][b, h]) * np.linalg.norm(dq[b, h]) for h in range(j * g, (j + 1) * g))
            scale += np.linalg.norm(xo["k_s"][b, j]) * nrm
            assert abs(lhs - rhs) <= 1e-2 * scale


@pytest.mark.parametrize("name,kv,resize", [
    ("corr_16k", 4, None),                                   # the benchmark's --student-kv-heads 4 launch
    ("corr_4k", 1, dict(B=1, n_q=2048, n_k=2048, seed=77)),  # one shared key head: split groups
])
def test_grouped_full_size_sampled(name, kv, resize):
    """Student keys shared by groups of query heads at the measured sizes:
    sampled KL rows and dQ_s rows (and, for the smaller shape, sampled dK_s
    keys summed over their KL heads) against the oracle on the expanded heads,
    plus the identities that hold at any size."""
    from attention_kl_divergence_amd import inputs
    w = inputs.WORKLOADS[name]
    if resize:
        w = w.resized(**resize)
    print(f"[grouped full] {w.name} {w.B}x{w.H}x{w.n_q} with {kv} student key heads", flush=True)
    x = inputs.make(w)
    x["k_s"] = np.ascontiguousarray(x["k_s"][:, :kv])
    d = {k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in x.items()}
    kl, lt, ls, tot = skl.streamkl_fwd(d["q_t"], d["k_t"], d["q_s"], d["k_s"])
    dq, dk = skl.streamkl_bwd(d["q_t"], d["k_t"], d["q_s"], d["k_s"], lt, ls)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    kl, lt, ls, dq, dk = f(kl), f(lt), f(ls), f(dq), f(dk)
    xo = {k: v.astype(np.float64) for k, v in x.items()}
    del x, d
    xe = dict(xo)
    xe["k_s"] = np.repeat(xo["k_s"], w.H // kv, axis=1)
    rng = np.random.default_rng(w.seed + 9)
    n_rows = w.B * w.H * w.n_q
    rows = np.array(sorted(set(rng.choice(n_rows, 40, replace=False).tolist()) | {0, n_rows - 1}), dtype=np.int64)
    rkl, rlt, rls = oracle.fwd_rows(xe["q_t"], xe["k_t"], xe["q_s"], xe["k_s"], w.tau_t, w.tau_s, False, rows)
    check_kl(kl.ravel()[rows], rkl, "bf16", "grouped full kl")
    check_lse(lt.ravel()[rows], rlt, "bf16", "grouped full lse_t")
    check_lse(ls.ravel()[rows], rls, "bf16", "grouped full lse_s")
    qrows = rows[::3]
    rdq = oracle.dq_rows(xe["q_t"], xe["k_t"], xe["q_s"], xe["k_s"], w.tau_t, w.tau_s, False, qrows)
    check_grad(dq.reshape(-1, w.d_s)[qrows], rdq, "bf16", "grouped full dq_s rows")
    if resize:
        keys = np.array(sorted(set(rng.choice(w.n_k, 6, replace=False).tolist()) | {0, w.n_k - 1}), dtype=np.int64)
        b = w.B - 1
        rdk = sum(oracle.dk_keys(xe["q_t"], xe["k_t"], xe["q_s"], xe["k_s"], w.tau_t, w.tau_s, False, b, h, keys)
                  for h in range(w.H))
        check_grad(dk[b, 0][keys], rdk, "bf16", "grouped full dk_s keys (summed over the group)")
    assert abs(float(tot.item()) - float(np.sum(kl))) <= 1e-6 * float(np.sum(np.abs(kl)))
    _identities_grouped(xo, dq, dk, w.H, kv)


@pytest.mark.parametrize("causal", [False, True])
def test_packed_sequences_match_padded_lengths(causal):
    """Packed sequences (cu_seqlens offsets) give the same bits as the same
    data laid out padded with per-batch lengths: per-row outputs, and the
    student and teacher gradients on every valid row; grouped student keys."""
    lq, lk = [100, 37, 200], [150, 37, 260]
    if causal:
        lk = [max(a, b) for a, b in zip(lq, lk)]
    B, n_q, n_k = 3, max(lq), max(lk)
    heads = (4, 4, 4, 2)
    x = _draw(41 + causal, B, heads, n_q, n_k, 128, 64, "bf16")
    for b in range(B):  # padding rows hold garbage the kernels must not read
        for k, n in (("q_t", lq[b]), ("q_s", lq[b]), ("k_t", lk[b]), ("k_s", lk[b])):
            x[k][b, :, n:] = 1e3
    d = {k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in x.items()}
    sq = torch.tensor(lq, dtype=torch.int32, device="cuda")
    sk = torch.tensor(lk, dtype=torch.int32, device="cuda")
    cq = torch.tensor(np.concatenate([[0], np.cumsum(lq)]), dtype=torch.int32, device="cuda")
    ck = torch.tensor(np.concatenate([[0], np.cumsum(lk)]), dtype=torch.int32, device="cuda")

    def pack(t, lens):
        return torch.cat([t[b, :, :lens[b]].transpose(0, 1) for b in range(B)]).contiguous()
    pk = {k: pack(d[k], lq if k.startswith("q") else lk) for k in d}
    args = (d["q_t"], d["k_t"], d["q_s"], d["k_s"])
    pargs = (pk["q_t"], pk["k_t"], pk["q_s"], pk["k_s"], cq, ck, n_q, n_k)
    kl, lt, ls, tot = skl.streamkl_fwd(*args, causal=causal, seqlen_q=sq, seqlen_k=sk)
    pkl, plt, pls, ptot = skl.streamkl_fwd_varlen(*pargs, causal=causal)
    g = torch.from_numpy(np.random.default_rng(9).standard_normal((B, 4, n_q)).astype(np.float32)).cuda()
    dq, dk = skl.streamkl_bwd(*args, lt, ls, grad_rows=g, causal=causal, seqlen_q=sq, seqlen_k=sk)
    pdq, pdk = skl.streamkl_bwd_varlen(*pargs, plt, pls, grad_rows=g, causal=causal)
    tdq, tdk = skl.streamkl_bwd_teacher(*args, lt, ls, kl, grad_rows=g, causal=causal, seqlen_q=sq, seqlen_k=sk)
    ptdq, ptdk = skl.streamkl_bwd_varlen(*pargs, plt, pls, grad_rows=g, causal=causal, teacher=True, kl_rows=pkl)
    torch.cuda.synchronize()
    for a, b_ in ((kl, pkl), (lt, plt), (ls, pls), (tot, ptot)):
        assert torch.equal(a, b_)
    for padded, packed, lens in ((dq, pdq, lq), (tdq, ptdq, lq), (tdk, ptdk, lk)):
        assert torch.equal(pack(padded, lens), packed)
    # the grouped dK_s: the padded launch splits its head groups over blocks
    # (fp32 partial sums added afterwards), the packed one never does, so the
    # two agree to rounding rather than bit for bit
    a, b_ = pack(dk, lk).float(), pdk.float()
    assert (a - b_).norm() <= 2e-3 * a.norm()
    # and the padded results match the oracle
    t_t, t_s = float(np.float32(1 / np.sqrt(128))), float(np.float32(1 / np.sqrt(64)))
    ref = _reference(x, 4, t_t, t_s, causal, lq, lk, g=g.cpu().numpy())
    check_kl(kl.cpu().numpy(), ref["kl"], "bf16", "packed kl")
    check_grad(dk.float().cpu().numpy(), ref["dk_s"], "bf16", "packed dk_s")
    check_grad(tdq.float().cpu().numpy(), ref["dq_t"], "bf16", "packed dq_t")


def test_packed_sequences_autograd():
    """attention_kl_varlen under autograd gives the gradients of the explicit
    packed calls, for student and teacher tensors."""
    lq, lk = [50, 90], [70, 90]
    cq = torch.tensor(np.concatenate([[0], np.cumsum(lq)]), dtype=torch.int32, device="cuda")
    ck = torch.tensor(np.concatenate([[0], np.cumsum(lk)]), dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(50)
    mk = lambda n, h, d: torch.from_numpy(rng.standard_normal((n, h, d), dtype=np.float32)).cuda()
    q_t, k_t, q_s, k_s = mk(sum(lq), 4, 64), mk(sum(lk), 2, 64), mk(sum(lq), 4, 64), mk(sum(lk), 1, 64)
    leaves = [t.clone().requires_grad_(True) for t in (q_t, k_t, q_s, k_s)]
    kl = skl.attention_kl_varlen(*leaves, cq, ck, max(lq), max(lk), causal=True)
    w = torch.linspace(0.5, 1.5, kl.numel(), device="cuda").reshape(kl.shape)
    (kl * w).sum().backward()
    torch.cuda.synchronize()
    _, lt, ls, _ = skl.streamkl_fwd_varlen(q_t, k_t, q_s, k_s, cq, ck, max(lq), max(lk), causal=True)
    ref_s = skl.streamkl_bwd_varlen(q_t, k_t, q_s, k_s, cq, ck, max(lq), max(lk), lt, ls, grad_rows=w.contiguous(),
                                    causal=True)
    kl2, _, _, _ = skl.streamkl_fwd_varlen(q_t, k_t, q_s, k_s, cq, ck, max(lq), max(lk), causal=True)
    ref_t = skl.streamkl_bwd_varlen(q_t, k_t, q_s, k_s, cq, ck, max(lq), max(lk), lt, ls, grad_rows=w.contiguous(),
                                    causal=True, teacher=True, kl_rows=kl2)
    torch.cuda.synchronize()
    for got, ref in ((leaves[2].grad, ref_s[0]), (leaves[3].grad, ref_s[1]), (leaves[0].grad, ref_t[0]),
                     (leaves[1].grad, ref_t[1])):
        assert torch.equal(got, ref)


def test_packed_rows_no_sequence_owns_get_zero_gradients():
    """Packed buffers with rows before the first offset and after the last one
    (owned by no sequence): those rows of both packed gradients are exactly 0
    for student and teacher gradients, under autograd too, and the owned rows
    match a launch on the trimmed buffers bit for bit."""
    lq, lk = [40, 70], [60, 70]
    lead, tail = 5, 9  # unowned rows before cu[0] and after cu[B]
    cq = torch.tensor(np.concatenate([[lead], lead + np.cumsum(lq)]), dtype=torch.int32, device="cuda")
    ck = torch.tensor(np.concatenate([[lead], lead + np.cumsum(lk)]), dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(51)
    tq, tk = lead + sum(lq) + tail, lead + sum(lk) + tail
    mk = lambda n, h, d: torch.from_numpy(rng.standard_normal((n, h, d), dtype=np.float32)).to(torch.bfloat16).cuda()
    q_t, k_t, q_s, k_s = mk(tq, 2, 64), mk(tk, 2, 64), mk(tq, 2, 64), mk(tk, 2, 64)
    args = (q_t, k_t, q_s, k_s, cq, ck, max(lq), max(lk))
    _, lt, ls, _ = skl.streamkl_fwd_varlen(*args)
    kl = skl.streamkl_fwd_varlen(*args)[0]
    dq, dk = skl.streamkl_bwd_varlen(*args, lt, ls)
    tdq, tdk = skl.streamkl_bwd_varlen(*args, lt, ls, teacher=True, kl_rows=kl)
    # the same sequences without the unowned rows
    c0q = cq - lead
    c0k = ck - lead
    trim = (q_t[lead:lead + sum(lq)], k_t[lead:lead + sum(lk)], q_s[lead:lead + sum(lq)], k_s[lead:lead + sum(lk)])
    targs = (*[t.contiguous() for t in trim], c0q, c0k, max(lq), max(lk))
    _, lt0, ls0, _ = skl.streamkl_fwd_varlen(*targs)
    rdq, rdk = skl.streamkl_bwd_varlen(*targs, lt0, ls0)
    leaves = [t.clone().requires_grad_(True) for t in (q_t, k_t, q_s, k_s)]
    skl.attention_kl_varlen(*leaves, cq, ck, max(lq), max(lk), check_lengths=True).sum().backward()
    torch.cuda.synchronize()
    for g_q, g_k in ((dq, dk), (tdq, tdk), (leaves[2].grad, leaves[3].grad), (leaves[0].grad, leaves[1].grad)):
        for g, n in ((g_q, sum(lq)), (g_k, sum(lk))):
            assert torch.count_nonzero(g[:lead]) == 0
            assert torch.count_nonzero(g[lead + n:]) == 0
            assert torch.count_nonzero(g[lead:lead + n]) > 0
    assert torch.equal(dq[lead:lead + sum(lq)], rdq)
    assert torch.equal(dk[lead:lead + sum(lk)], rdk)


def test_packed_offsets_checked_on_request():
    """check_lengths=True rejects a sequence longer than max_seqlen, decreasing
    offsets and offsets past the packed rows; without it the kernels cut the
    long sequence to max_seqlen rows (documented behaviour)."""
    lq = [30, 50]
    cq = torch.tensor(np.concatenate([[0], np.cumsum(lq)]), dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(52)
    mk = lambda n: torch.from_numpy(rng.standard_normal((n, 1, 64), dtype=np.float32)).cuda()
    x = (mk(80), mk(80), mk(80), mk(80))
    with pytest.raises(ValueError, match="exceeds max_seqlen"):
        skl.streamkl_fwd_varlen(*x, cq, cq, 40, 40, check_lengths=True)
    with pytest.raises(ValueError, match="decrease"):
        bad = torch.tensor([0, 50, 30], dtype=torch.int32, device="cuda")
        skl.streamkl_fwd_varlen(*x, bad, bad, 50, 50, check_lengths=True)
    with pytest.raises(ValueError, match="past the"):
        far = torch.tensor([0, 30, 90], dtype=torch.int32, device="cuda")
        skl.streamkl_fwd_varlen(*x, far, far, 60, 60, check_lengths=True)
    kl, _, _, _ = skl.streamkl_fwd_varlen(*x, cq, cq, 50, 50, check_lengths=True)
    cut, _, _, _ = skl.streamkl_fwd_varlen(*x, cq, cq, 40, 40)
    torch.cuda.synchronize()
    assert kl.shape == (2, 1, 50) and cut.shape == (2, 1, 40)
