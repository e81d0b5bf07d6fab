"""Oracle against stored fixtures: hand-derived closed forms, and a frozen copy of
its own tiny-workload output (written by tests/golden/make_oracle_regression.py)."""
import json
import os

import numpy as np

import oracle
from attention_kl_divergence_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_closed_form_cases():
    with open(os.path.join(GOLDEN, "closed_form_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        arr = [np.array(c[k], dtype=np.float64)[None, None] for k in ("q_t", "k_t", "q_s", "k_s")]
        kl, _, _, _ = oracle.fwd(*arr, c["tau_t"], c["tau_s"], c["causal"])
        np.testing.assert_allclose(kl[0, 0], c["kl"], rtol=1e-14, atol=1e-15, err_msg=c["name"])


def test_tiny_workload_regression():
    with open(os.path.join(GOLDEN, "tiny_f32_oracle.json")) as f:
        ref = json.load(f)
    w = inputs.WORKLOADS["tiny_f32"]
    x = inputs.make(w)
    kl, lt, ls, tot = oracle.fwd(x["q_t"], x["k_t"], x["q_s"], x["k_s"], w.tau_t, w.tau_s, w.causal)
    np.testing.assert_allclose(kl.ravel()[:16], ref["kl_rows_0_16"], rtol=1e-13)
    np.testing.assert_allclose(lt.ravel()[:16], ref["lse_t_0_16"], rtol=1e-14)
    np.testing.assert_allclose(ls.ravel()[:16], ref["lse_s_0_16"], rtol=1e-14)
    assert abs(tot - ref["kl_sum"]) <= 1e-12 * abs(ref["kl_sum"])
    dq, dk = oracle.bwd(x["q_t"], x["k_t"], x["q_s"], x["k_s"], w.tau_t, w.tau_s, w.causal)
    np.testing.assert_allclose(dq[0, 0, 0], ref["dq_s_row0"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(dk[0, 0, 0], ref["dk_s_row0"], rtol=1e-12, atol=1e-15)
