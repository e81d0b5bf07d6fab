"""GPU parity of the split forward (key ranges run separately, partial online
states merged) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest

import attention_kl_divergence_amd as skl
import oracle
from attention_kl_divergence_amd import inputs
from tests.gpu_util import as_f64, check_grad, check_kl, check_lse, check_sum, to_device

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

W = inputs.WORKLOADS

CASES = [
    ("tiny_f32", W["tiny_f32"]),
    ("bf16_corr_300x700", W["corr_4k"].resized(B=2, H=2, n_q=300, n_k=700, seed=401)),
    ("bf16_causal_500", W["corr_4k"].resized(B=1, H=2, n_q=500, n_k=500, causal=True, seed=402)),
    ("bf16_mixed_200x1100", W["mixed_dims_2k"].resized(B=2, H=3, n_q=200, n_k=1100, seed=403)),
    ("bf16_causal_rect_130x900", W["corr_4k"].resized(B=1, H=2, n_q=130, n_k=900, causal=True, seed=404)),
]


def _oracle(w, x):
    xo = as_f64(x)
    return oracle.fwd(xo["q_t"], xo["k_t"], xo["q_s"], xo["k_s"], w.tau_t, w.tau_s, w.causal)


def _check(w, out, ref):
    kl, lt, ls, tot = (t.cpu().double().numpy() if t is not None else None for t in out)
    rkl, rlt, rls, _ = ref
    check_kl(kl, rkl, w.dtype)
    check_lse(lt, rlt, w.dtype, "lse_t")
    check_lse(ls, rls, w.dtype, "lse_s")
    check_sum(float(tot[0]), rkl, w.dtype)


@pytest.mark.parametrize("n_split", [2, 3, 7])
@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
def test_split_forward_matches_oracle(name, w, n_split):
    print(f"[split] {name} n_split={n_split}", flush=True)
    x = inputs.make(w)
    d = to_device(x, w.dtype)
    out = skl.streamkl_fwd(d["q_t"], d["k_t"], d["q_s"], d["k_s"], w.tau_t, w.tau_s, w.causal, split=n_split)
    torch.cuda.synchronize()
    _check(w, out, _oracle(w, x))
    # and the unsplit forward agrees to rounding
    ref = skl.streamkl_fwd(d["q_t"], d["k_t"], d["q_s"], d["k_s"], w.tau_t, w.tau_s, w.causal, split=1)
    torch.cuda.synchronize()
    assert torch.allclose(out[0], ref[0], rtol=1e-4, atol=1e-5)
    assert torch.allclose(out[1], ref[1], rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("name,w", [CASES[1], CASES[2], CASES[4]], ids=["bf16_corr", "bf16_causal", "bf16_causal_rect"])
def test_partial_states_over_uneven_ranges_merge_to_the_forward(name, w):
    """Context-parallel use: disjoint, uneven key ranges computed one call each
    (some of them empty for some rows under a causal mask), merged afterwards."""
    x = inputs.make(w)
    d = to_device(x, w.dtype)
    cuts = [0, 96, 224, 320, w.n_k]
    states = [skl.streamkl_fwd_partial(d["q_t"], d["k_t"], d["q_s"], d["k_s"], a, b, w.tau_t, w.tau_s, w.causal)
              for a, b in zip(cuts[:-1], cuts[1:])]
    out = skl.streamkl_fwd_merge(states, w.tau_t, w.tau_s)
    torch.cuda.synchronize()
    _check(w, out, _oracle(w, x))


def test_backward_on_split_forward_statistics():
    """The log-normalisers from the split forward drive the backward as well."""
    w = W["mixed_dims_2k"].resized(B=2, H=2, n_q=160, n_k=900, seed=405)
    x = inputs.make(w)
    d = to_device(x, w.dtype)
    kl, lt, ls, _ = skl.streamkl_fwd(d["q_t"], d["k_t"], d["q_s"], d["k_s"], w.tau_t, w.tau_s, w.causal, split=4)
    dq, dk = skl.streamkl_bwd(d["q_t"], d["k_t"], d["q_s"], d["k_s"], lt, ls, tau_t=w.tau_t, tau_s=w.tau_s)
    torch.cuda.synchronize()
    xo = as_f64(x)
    rdq, rdk = oracle.bwd(xo["q_t"], xo["k_t"], xo["q_s"], xo["k_s"], w.tau_t, w.tau_s, w.causal)
    check_grad(dq.float().cpu().numpy(), rdq, w.dtype, "dq_s")
    check_grad(dk.float().cpu().numpy(), rdk, w.dtype, "dk_s")


@pytest.mark.parametrize("name", ["corr_4k", "cross_512x16k"])
def test_auto_split_full_size_sampled(name):
    """The full workloads the split is suggested for, on sampled oracle rows."""
    w = W[name]
    lib = skl.load_library()
    n_split = lib.streamkl_fwd_split_count(w.B, w.H, w.n_q, w.n_k, int(w.causal))
    print(f"[split full] {name}: n_split {n_split}", flush=True)
    assert n_split > 1
    x = inputs.make(w)
    d = to_device(x, w.dtype)
    kl, lt, ls, tot = skl.streamkl_fwd(d["q_t"], d["k_t"], d["q_s"], d["k_s"], w.tau_t, w.tau_s, w.causal)
    torch.cuda.synchronize()
    xo = as_f64(x)
    rng = np.random.default_rng(w.seed + 31)
    n_rows = w.B * w.H * w.n_q
    rows = np.array(sorted(set(rng.choice(n_rows, 40, replace=False).tolist()) | {0, n_rows - 1}), dtype=np.int64)
    rkl, rlt, rls = oracle.fwd_rows(xo["q_t"], xo["k_t"], xo["q_s"], xo["k_s"], w.tau_t, w.tau_s, w.causal, rows)
    check_kl(kl.cpu().double().numpy().ravel()[rows], rkl, w.dtype)
    check_lse(lt.cpu().double().numpy().ravel()[rows], rlt, w.dtype, "lse_t")
    check_lse(ls.cpu().double().numpy().ravel()[rows], rls, w.dtype, "lse_s")
