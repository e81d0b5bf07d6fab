"""Pins for the oracle's gradients with respect to the first (teacher)
distribution of L = sum_r g_r KL(P_t || P_s)_r.

The derivative follows from the forward KL definition ("Lecture 05 - Where It
All Lands", section 3.1) alone; these checks tie the oracle's closed form to
that definition without reusing it: central finite differences of the oracle's
own forward, the two-key (Bernoulli) closed form, the translation and scale
invariances of the teacher scores, the exact zero at the minimum (identical
distributions), and the reverse divergence KL(P_s || P_t), whose student
gradient is the same first-argument formula with the distributions swapped.
"""
import math

import numpy as np
import pytest

import oracle


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def _loss(qt, kt, qs, ks, tt, ts, causal, g):
    kl, _, _, _ = oracle.fwd(qt, kt, qs, ks, tt, ts, causal)
    return math.fsum((g * kl).ravel())


@pytest.mark.parametrize("causal", [False, True])
def test_teacher_gradients_match_central_differences(causal):
    rng = np.random.default_rng(121 + causal)
    B, H, n_q, n_k, d_t, d_s = 1, 2, 5, 7, 3, 4
    qt, kt = _rand(rng, B, H, n_q, d_t), _rand(rng, B, H, n_k, d_t)
    qs, ks = _rand(rng, B, H, n_q, d_s), _rand(rng, B, H, n_k, d_s)
    g = rng.uniform(-1.5, 2.0, size=(B, H, n_q))
    tt, ts = 0.8, 0.6
    dq, dk = oracle.bwd_teacher(qt, kt, qs, ks, tt, ts, causal, g=g)
    h = 1e-6
    fd_q = np.zeros_like(qt); fd_k = np.zeros_like(kt)
    for idx in np.ndindex(qt.shape):
        a, b = qt.copy(), qt.copy(); a[idx] += h; b[idx] -= h
        fd_q[idx] = (_loss(a, kt, qs, ks, tt, ts, causal, g) - _loss(b, kt, qs, ks, tt, ts, causal, g)) / (2 * h)
    for idx in np.ndindex(kt.shape):
        a, b = kt.copy(), kt.copy(); a[idx] += h; b[idx] -= h
        fd_k[idx] = (_loss(qt, a, qs, ks, tt, ts, causal, g) - _loss(qt, b, qs, ks, tt, ts, causal, g)) / (2 * h)
    assert np.all(np.abs(fd_q - dq) <= 1e-7 + 1e-5 * np.abs(dq))
    assert np.all(np.abs(fd_k - dk) <= 1e-7 + 1e-5 * np.abs(dk))
    assert np.linalg.norm(fd_q - dq) <= 1e-6 * np.linalg.norm(dq)
    assert np.linalg.norm(fd_k - dk) <= 1e-6 * np.linalg.norm(dk)


def test_two_keys_bernoulli_closed_form():
    """One query, two keys, d = 1: KL = p ln(p/q) + (1-p) ln((1-p)/(1-q)) with
    p = sigmoid(s_t0 - s_t1), q = sigmoid(s_s0 - s_s1); dKL/ds_t0 =
    p (1 - p) [ln(p/q) - ln((1-p)/(1-q))] = -dKL/ds_t1, so
    dq_t = tau_t dKL/ds_t0 (k_t0 - k_t1) and dk_t[j] = +-tau_t dKL/ds_t0 q_t."""
    qt = np.array([[[[1.3]]]]); kt = np.array([[[[0.7], [-0.4]]]])
    qs = np.array([[[[0.5]]]]); ks = np.array([[[[-0.2], [0.9]]]])
    tt, ts = 0.9, 1.1
    st = tt * qt[0, 0, 0, 0] * kt[0, 0, :, 0]
    ss = ts * qs[0, 0, 0, 0] * ks[0, 0, :, 0]
    p = 1.0 / (1.0 + math.exp(-(st[0] - st[1])))
    q = 1.0 / (1.0 + math.exp(-(ss[0] - ss[1])))
    dds0 = p * (1 - p) * (math.log(p / q) - math.log((1 - p) / (1 - q)))
    dq, dk = oracle.bwd_teacher(qt, kt, qs, ks, tt, ts, False)
    assert abs(dq[0, 0, 0, 0] - tt * dds0 * (kt[0, 0, 0, 0] - kt[0, 0, 1, 0])) <= 1e-15
    assert abs(dk[0, 0, 0, 0] - tt * dds0 * qt[0, 0, 0, 0]) <= 1e-15
    assert abs(dk[0, 0, 1, 0] + tt * dds0 * qt[0, 0, 0, 0]) <= 1e-15


@pytest.mark.parametrize("causal", [False, True])
def test_teacher_gradient_invariants(causal):
    """sum_j dK_t[j] = 0 (a common shift of every teacher key moves a row's
    teacher scores by a constant) and <Q_t, dQ_t> = <K_t, dK_t> per head
    (Q_t (1+e), K_t / (1+e) leaves the scores unchanged)."""
    rng = np.random.default_rng(131)
    B, H, n_q, n_k = 2, 2, 11, 16
    qt, kt = _rand(rng, B, H, n_q, 5), _rand(rng, B, H, n_k, 5)
    qs, ks = _rand(rng, B, H, n_q, 6), _rand(rng, B, H, n_k, 6)
    g = rng.uniform(0.5, 1.5, size=(B, H, n_q))
    dq, dk = oracle.bwd_teacher(qt, kt, qs, ks, 0.6, 0.5, causal, g=g)
    scale = np.max(np.abs(dk))
    assert scale > 1e-3
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-13 * scale * n_k)
    lhs = np.einsum("bhnd,bhnd->bh", qt, dq)
    rhs = np.einsum("bhnd,bhnd->bh", kt, dk)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_distributions_give_zero_teacher_gradient(causal):
    rng = np.random.default_rng(141)
    q, k = _rand(rng, 1, 2, 6, 4), _rand(rng, 1, 2, 9, 4)
    dq, dk = oracle.bwd_teacher(q, k, q, k, 0.5, 0.5, causal)
    assert not np.any(dq) and not np.any(dk)


def test_swapped_distributions_give_reverse_kl_student_gradient():
    """KL(P_s || P_t) is the forward KL with the distributions swapped; its
    gradient in the student queries, from finite differences, equals the
    first-argument gradient of the swapped call."""
    rng = np.random.default_rng(151)
    qt, kt = _rand(rng, 1, 1, 4, 3), _rand(rng, 1, 1, 6, 3)
    qs, ks = _rand(rng, 1, 1, 4, 3), _rand(rng, 1, 1, 6, 3)
    tt, ts = 0.7, 0.9
    dq_rev, dk_rev = oracle.bwd_teacher(qs, ks, qt, kt, ts, tt, False)

    def rev(qs_):
        kl, _, _, _ = oracle.fwd(qs_, ks, qt, kt, ts, tt, False)
        return math.fsum(kl.ravel())
    h = 1e-6
    for idx in np.ndindex(qs.shape):
        a, b = qs.copy(), qs.copy(); a[idx] += h; b[idx] -= h
        fd = (rev(a) - rev(b)) / (2 * h)
        assert abs(fd - dq_rev[idx]) <= 1e-7 + 1e-5 * abs(dq_rev[idx])
    # and it differs from the forward-KL student gradient (the divergence is asymmetric)
    dq_fwd, _ = oracle.bwd(qt, kt, qs, ks, tt, ts, False)
    assert np.linalg.norm(dq_fwd - dq_rev) > 1e-3 * np.linalg.norm(dq_rev)


def test_teacher_sampled_entry_points_agree_with_full():
    rng = np.random.default_rng(161)
    B, H, n_q, n_k = 2, 3, 10, 15
    qt, kt = _rand(rng, B, H, n_q, 4), _rand(rng, B, H, n_k, 4)
    qs, ks = _rand(rng, B, H, n_q, 3), _rand(rng, B, H, n_k, 3)
    g = rng.normal(size=(B, H, n_q))
    for causal in (False, True):
        dq, dk = oracle.bwd_teacher(qt, kt, qs, ks, 0.5, 0.7, causal, g=g)
        rows = np.array([0, 7, 11, 29, 59], dtype=np.int64)
        dq2 = oracle.dqt_rows(qt, kt, qs, ks, 0.5, 0.7, causal, rows, g=g)
        np.testing.assert_allclose(dq2, dq.reshape(-1, 4)[rows], rtol=1e-13, atol=1e-15)
        keys = np.array([0, 4, 14], dtype=np.int64)
        dk2 = oracle.dkt_keys(qt, kt, qs, ks, 0.5, 0.7, causal, 1, 2, keys, g=g)
        np.testing.assert_allclose(dk2, dk[1, 2, keys], rtol=1e-12, atol=1e-15)
