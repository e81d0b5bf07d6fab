"""GPU parity of the vocabulary-logit KL (streamkl_vocab_fwd / _bwd / _fwd_bwd)
against the fp64 oracle, through the C ABI: small and ragged shapes element by
element on both the 16-byte vector path and the element-wise path, strided
rows, both dtypes, several temperatures, student and teacher gradients with
per-row and scalar upstream weights, the fused launch against the separate
ones, autograd, and the full-size workload on sampled rows plus identities that
hold at any size."""
import numpy as np
import pytest

import attention_kl_divergence_amd as skl
import oracle
from attention_kl_divergence_amd import inputs
from tests.gpu_util import check_grad, check_kl, check_lse, check_sum, rel_l2

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

VW = inputs.VOCAB_WORKLOADS

CASES = [
    ("bf16_37x32000_T2", VW["kd_logits_small"]),
    ("f32_9x50257_odd", VW["kd_logits_odd_f32"]),
    ("bf16_70x1000_short", VW["kd_logits_short"]),
    ("bf16_5x999_short_odd", VW["kd_logits_short"].resized(rows=5, V=999, seed=41)),
    ("bf16_6x4095", VW["kd_logits_small"].resized(rows=6, V=4095, seed=42)),
    ("bf16_6x4096", VW["kd_logits_small"].resized(rows=6, V=4096, seed=43)),
    ("bf16_3x8", VW["kd_logits_small"].resized(rows=3, V=8, seed=44)),
    ("f32_20x32000_T0.7", VW["kd_logits_small"].resized(rows=20, dtype="f32", temperature=0.7, seed=45)),
    ("bf16_11x20000_T0.05", VW["kd_logits_small"].resized(rows=11, V=20000, temperature=0.05, seed=46)),
    ("bf16_11x20000_T50", VW["kd_logits_small"].resized(rows=11, V=20000, temperature=50.0, seed=47)),
    ("f32_13x7777_iid", VW["kd_logits_short"].resized(rows=13, V=7777, dtype="f32", seed=48)),
]


def _dev(a, dtype):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.from_numpy(np.ascontiguousarray(a)).to(tdt).cuda()


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
def test_vocab_forward_matches_oracle(name, w):
    print(f"[vocab fwd] {w}", flush=True)
    zt, zs = inputs.make_vocab(w)
    kl, lt, ls, tot = skl.streamkl_vocab_fwd(_dev(zt, w.dtype), _dev(zs, w.dtype), w.temperature)
    torch.cuda.synchronize()
    rkl, rlt, rls, _ = oracle.vocab_fwd(zt.astype(np.float64), zs.astype(np.float64), w.temperature)
    check_kl(_np(kl), rkl, w.dtype, f"{name} kl")
    check_lse(_np(lt), rlt, w.dtype, f"{name} lse_t")
    check_lse(_np(ls), rls, w.dtype, f"{name} lse_s")
    check_sum(float(tot.item()), rkl, w.dtype)


@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
def test_vocab_gradients_match_oracle(name, w):
    print(f"[vocab bwd] {w}", flush=True)
    zt, zs = inputs.make_vocab(w)
    g = np.random.default_rng(w.seed + 500).uniform(-1.0, 2.0, size=w.rows).astype(np.float32)
    dt, ds = _dev(zt, w.dtype), _dev(zs, w.dtype)
    kl, lt, ls, _ = skl.streamkl_vocab_fwd(dt, ds, w.temperature)
    gt = torch.from_numpy(g).cuda()
    dzs, dzt = skl.streamkl_vocab_bwd(dt, ds, lt, ls, kl, w.temperature, grad_rows=gt, teacher=True)
    dzs1 = skl.streamkl_vocab_bwd(dt, ds, lt, ls, None, w.temperature, grad_scalar=0.75)
    torch.cuda.synchronize()
    rs, rt = oracle.vocab_bwd(zt.astype(np.float64), zs.astype(np.float64), w.temperature, g=g.astype(np.float64),
                              teacher=True)
    check_grad(_np(dzs), rs, w.dtype, f"{name} dz_s")
    check_grad(_np(dzt), rt, w.dtype, f"{name} dz_t")
    rs1 = oracle.vocab_bwd(zt.astype(np.float64), zs.astype(np.float64), w.temperature, g=0.75)
    check_grad(_np(dzs1), rs1, w.dtype, f"{name} dz_s scalar")


@pytest.mark.parametrize("name,w", [CASES[0], CASES[1], CASES[2], CASES[3]], ids=[c[0] for c in CASES[:4]])
def test_vocab_fused_launch_equals_separate_launches(name, w):
    zt, zs = inputs.make_vocab(w)
    g = np.random.default_rng(w.seed + 600).uniform(0.5, 1.5, size=w.rows).astype(np.float32)
    dt, ds = _dev(zt, w.dtype), _dev(zs, w.dtype)
    gt = torch.from_numpy(g).cuda()
    kl, lt, ls, tot = skl.streamkl_vocab_fwd(dt, ds, w.temperature)
    dzs, dzt = skl.streamkl_vocab_bwd(dt, ds, lt, ls, kl, w.temperature, grad_rows=gt, teacher=True)
    fkl, flt, fls, ftot, fdzs, fdzt = skl.streamkl_vocab_fwd_bwd(dt, ds, w.temperature, grad_rows=gt, teacher=True)
    _, _, _, _, sdzs, none = skl.streamkl_vocab_fwd_bwd(dt, ds, w.temperature, grad_scalar=2.0)
    torch.cuda.synchronize()
    assert none is None
    # the same arithmetic, compiled into another kernel: equal up to the last
    # bits of fp32 rounding (the compiler may contract and schedule the sums
    # differently), which bf16 outputs can carry over as one-ulp differences
    # (KL is a difference of log-normalisers: its rounding scales with |LSE|)
    scale = 1.0 + lt.abs() + ls.abs()
    assert torch.all((kl - fkl).abs() <= 4e-6 * scale), (kl - fkl).abs().max()
    assert torch.all((lt - flt).abs() <= 2e-6 * scale) and torch.all((ls - fls).abs() <= 2e-6 * scale)
    assert abs(tot.item() - ftot.item()) <= 4e-6 * scale.sum().item()
    gtol = 1e-5 if w.dtype == "f32" else 4e-3
    for a, b in ((dzs, fdzs), (dzt, fdzt)):
        assert rel_l2(_np(b), _np(a)) <= gtol
    ref = skl.streamkl_vocab_bwd(dt, ds, lt, ls, None, w.temperature, grad_scalar=2.0)
    torch.cuda.synchronize()
    assert rel_l2(_np(sdzs), _np(ref)) <= gtol


@pytest.mark.parametrize("dtype,pad", [("bf16", 8), ("bf16", 3), ("f32", 4), ("f32", 1)])
def test_vocab_strided_rows(dtype, pad):
    """Rows of a wider buffer (leading dimension V + pad): the vector path when
    the rows stay 16-byte aligned, the element path otherwise; and logits given
    as [B, S, V] with leading dims flattened."""
    w = VW["kd_logits_small"].resized(rows=12, V=3000, dtype=dtype, seed=60 + pad)
    zt, zs = inputs.make_vocab(w)
    wide_t = np.zeros((w.rows, w.V + pad), np.float32); wide_t[:, :w.V] = zt
    wide_s = np.full((w.rows, w.V + pad), 7.0, np.float32); wide_s[:, :w.V] = zs
    dt = _dev(wide_t, dtype)[:, :w.V]
    ds = _dev(wide_s, dtype)[:, :w.V]
    assert dt.stride(0) == w.V + pad
    kl, lt, ls, _ = skl.streamkl_vocab_fwd(dt.view(3, 4, w.V), ds.view(3, 4, w.V), w.temperature)
    dzs = skl.streamkl_vocab_bwd(dt, ds, lt.reshape(-1), ls.reshape(-1), None, w.temperature)
    torch.cuda.synchronize()
    assert tuple(kl.shape) == (3, 4)
    rkl, rlt, _, _ = oracle.vocab_fwd(zt.astype(np.float64), zs.astype(np.float64), w.temperature)
    check_kl(_np(kl).reshape(-1), rkl, dtype, "strided kl")
    check_lse(_np(lt).reshape(-1), rlt, dtype, "strided lse_t")
    check_grad(_np(dzs), oracle.vocab_bwd(zt.astype(np.float64), zs.astype(np.float64), w.temperature), dtype,
               "strided dz_s")


def test_vocab_degenerate_cases():
    # a single logit per row: both distributions are a point mass, KL = 0, LSE = z / T, no gradient
    z = torch.tensor([[3.0], [-2.5], [0.0]], device="cuda")
    kl, lt, ls, tot = skl.streamkl_vocab_fwd(z, z * 2, 2.0)
    dzs, dzt = skl.streamkl_vocab_bwd(z, z * 2, lt, ls, kl, 2.0, teacher=True)
    torch.cuda.synchronize()
    assert torch.all(kl.abs() <= 1e-6)
    assert torch.allclose(lt, z[:, 0] / 2.0) and torch.allclose(ls, z[:, 0])
    assert torch.all(dzs.abs() <= 1e-6) and torch.all(dzt.abs() <= 1e-6)
    # identical teacher and student: zero KL and zero student gradient, on both paths
    for V in (4096 * 3, 1001):
        w = VW["kd_logits_small"].resized(rows=5, V=V, seed=70 + V)
        zt, _ = inputs.make_vocab(w)
        d = _dev(zt, "bf16")
        kl, lt, ls, _ = skl.streamkl_vocab_fwd(d, d.clone(), 1.5)
        dzs = skl.streamkl_vocab_bwd(d, d.clone(), lt, ls, None, 1.5)
        torch.cuda.synchronize()
        assert kl.abs().max().item() <= 1e-6 and (lt - ls).abs().max().item() <= 1e-6
        assert dzs.float().abs().max().item() <= 1e-6
    # a large common shift of one side's logits leaves KL unchanged and moves its LSE by shift / T
    w = VW["kd_logits_small"].resized(rows=8, V=5000, dtype="f32", seed=77)
    zt, zs = inputs.make_vocab(w)
    a = skl.streamkl_vocab_fwd(_dev(zt, "f32"), _dev(zs, "f32"), 2.0)
    b = skl.streamkl_vocab_fwd(_dev(zt + 1000.0, "f32"), _dev(zs - 300.0, "f32"), 2.0)
    torch.cuda.synchronize()
    rkl, _, _, _ = oracle.vocab_fwd((zt + np.float32(1000.0)).astype(np.float64),
                                    (zs - np.float32(300.0)).astype(np.float64), 2.0)
    check_kl(_np(b[0]), rkl, "f32", "shifted kl")
    assert np.max(np.abs(_np(b[0]) - _np(a[0]))) <= 1e-3
    assert np.max(np.abs(_np(b[1]) - _np(a[1]) - 500.0)) <= 1e-3


def test_vocab_autograd_matches_oracle():
    w = VW["kd_logits_small"].resized(rows=6, V=2048 + 8, seed=80)
    zt, zs = inputs.make_vocab(w)
    dt = _dev(zt, "bf16").requires_grad_(True)
    ds = _dev(zs, "bf16").requires_grad_(True)
    wts = torch.linspace(0.5, 2.0, w.rows, device="cuda")
    T = w.temperature
    loss = (skl.vocab_kl(dt, ds, T) * wts).sum() * (T * T)
    loss.backward()
    torch.cuda.synchronize()
    g = (wts * T * T).cpu().numpy().astype(np.float64)
    rs, rt = oracle.vocab_bwd(zt.astype(np.float64), zs.astype(np.float64), T, g=g, teacher=True)
    check_grad(_np(ds.grad), rs, "bf16", "autograd dz_s")
    check_grad(_np(dt.grad), rt, "bf16", "autograd dz_t")
    # student-only: the teacher takes no gradient and none is computed
    ds2 = _dev(zs, "bf16").requires_grad_(True)
    skl.vocab_kl(_dev(zt, "bf16"), ds2, T).sum().backward()
    torch.cuda.synchronize()
    check_grad(_np(ds2.grad), oracle.vocab_bwd(zt.astype(np.float64), zs.astype(np.float64), T), "bf16",
               "autograd dz_s only")


@pytest.fixture(scope="module")
def full_vocab():
    w = VW["kd_logits_4k_128k"]
    print(f"[vocab full] drawing {w}", flush=True)
    zt, zs = inputs.make_vocab(w)
    return w, _dev(zt, w.dtype), _dev(zs, w.dtype)


def test_vocab_full_size_sampled_rows(full_vocab):
    """The measured configuration (4096 rows x 128256 logits, bf16, T = 2), in
    the launches the benchmark times: sampled rows against the oracle, and the
    identities every row satisfies."""
    w, dt, ds = full_vocab
    kl, lt, ls, tot = skl.streamkl_vocab_fwd(dt, ds, w.temperature)
    fkl, _, _, _, fdzs, _ = skl.streamkl_vocab_fwd_bwd(dt, ds, w.temperature, grad_scalar=1.0 / w.rows)
    torch.cuda.synchronize()
    assert torch.all((kl - fkl).abs() <= 4e-6 * (1.0 + lt.abs() + ls.abs()))
    rows = np.random.default_rng(90).choice(w.rows, size=48, replace=False)
    rows[:2] = [0, w.rows - 1]
    zt, zs = inputs.make_vocab(w, rows=rows)
    rkl, rlt, rls, _ = oracle.vocab_fwd(zt.astype(np.float64), zs.astype(np.float64), w.temperature)
    check_kl(_np(kl)[rows], rkl, w.dtype, "full kl (sampled)")
    check_lse(_np(lt)[rows], rlt, w.dtype, "full lse_t (sampled)")
    check_lse(_np(ls)[rows], rls, w.dtype, "full lse_s (sampled)")
    rg = oracle.vocab_bwd(zt.astype(np.float64), zs.astype(np.float64), w.temperature, g=1.0 / w.rows)
    check_grad(_np(fdzs[torch.from_numpy(rows).cuda()]), rg, w.dtype, "full dz_s (sampled)")
    # every row: KL >= 0 up to the tolerance, the sum is the sum of the rows, and
    # each gradient row sums to ~0 (softmax gradients are shift invariant)
    a, r = 2e-3, 1e-2
    k = _np(kl)
    assert np.all(k >= -a) and np.all(np.isfinite(k))
    assert abs(float(tot.item()) - float(np.sum(k))) <= 1e-3 * max(1.0, float(np.sum(np.abs(k))))
    rowsum = fdzs.float().sum(dim=1).abs().max().item()
    assert rowsum <= 1e-5, rowsum


def test_vocab_rows_beyond_one_launch():
    """More rows than one launch covers (2^20): the host splits the rows over
    consecutive launches; rows on both sides of the boundary match the oracle,
    and the sum covers every row."""
    rows, V = (1 << 20) + 37, 16
    rng = np.random.default_rng(95)
    zt = _round_bf16_np(rng.standard_normal((rows, V), dtype=np.float32) * 2.0)
    zs = _round_bf16_np(zt + 0.5 * rng.standard_normal((rows, V), dtype=np.float32))
    dt, ds = _dev(zt, "bf16"), _dev(zs, "bf16")
    kl, lt, ls, tot, dzs, _ = skl.streamkl_vocab_fwd_bwd(dt, ds, 1.5, grad_scalar=0.5)
    torch.cuda.synchronize()
    pick = np.array([0, 1, (1 << 20) - 2, (1 << 20) - 1, 1 << 20, (1 << 20) + 1, rows - 1], dtype=np.int64)
    rkl, rlt, _, _ = oracle.vocab_fwd(zt[pick].astype(np.float64), zs[pick].astype(np.float64), 1.5)
    check_kl(_np(kl)[pick], rkl, "bf16", "many rows kl")
    check_lse(_np(lt)[pick], rlt, "bf16", "many rows lse_t")
    rg = oracle.vocab_bwd(zt[pick].astype(np.float64), zs[pick].astype(np.float64), 1.5, g=0.5)
    check_grad(_np(dzs[torch.from_numpy(pick).cuda()]), rg, "bf16", "many rows dz_s")
    k = _np(kl)
    assert abs(float(tot.item()) - float(np.sum(k))) <= 1e-4 * max(1.0, float(np.sum(np.abs(k))))


def _round_bf16_np(a):
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)).view(np.float32)
