"""Pins for the fp64 CPU oracle, checked against what the definition and the mathematics fix.

The pages print no worked example for the attention KL, so every pin here is a
brute-force evaluation, a closed form, an identity or an invariance that the
definition implies (forward KL, teacher first, natural log: "Lecture 05 - Where
It All Lands", sections 1 and 3.1; the per-row attention-KL reduction:
"StreamKL: Fast and Memory-Efficient KL Divergence for Boosting Attention
Distillation", abstract).  Each is chosen so that a plausible slip in the
oracle (a swapped argument order, a dropped tau, a causal off-by-one, a wrong
sign or a transposed operand in a gradient) fails at least one of them.
"""
import math

import numpy as np
import pytest
import scipy.special as sp

import oracle
from tests import brute


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def _softmax_rows(s, n_allowed):
    out = []
    for i, n in enumerate(n_allowed):
        out.append(sp.softmax(s[i, :n]))
    return out


def _allowed(n_q, n_k, causal):
    if not causal:
        return [n_k] * n_q
    return [min(n_k, i + (n_k - n_q) + 1) for i in range(n_q)]


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("shape", [(3, 5, 4, 2), (4, 4, 3, 3), (2, 7, 2, 4), (1, 1, 2, 2), (4, 8, 4, 4)])
@pytest.mark.parametrize("causal", [False, True])
def test_matches_decimal_brute_force(shape, causal):
    n_q, n_k, d_t, d_s = shape
    rng = np.random.default_rng(hash((shape, causal)) % 2**32)
    B, H = 1, 2
    qt = _rand(rng, B, H, n_q, d_t, scale=1.5); kt = _rand(rng, B, H, n_k, d_t, scale=1.5)
    qs = _rand(rng, B, H, n_q, d_s, scale=1.5); ks = _rand(rng, B, H, n_k, d_s, scale=1.5)
    tau_t, tau_s = 0.7, 1.1
    kl, lt, ls, tot = oracle.fwd(qt, kt, qs, ks, tau_t, tau_s, causal)
    for h in range(H):
        bk, bl, bs = brute.kl_rows(qt[0, h].tolist(), kt[0, h].tolist(), qs[0, h].tolist(), ks[0, h].tolist(),
                                   tau_t, tau_s, causal)
        for i in range(n_q):
            assert abs(kl[0, h, i] - float(bk[i])) <= 1e-14 + 1e-12 * abs(float(bk[i]))
            assert abs(lt[0, h, i] - float(bl[i])) <= 1e-14 * (1 + abs(float(bl[i])))
            assert abs(ls[0, h, i] - float(bs[i])) <= 1e-14 * (1 + abs(float(bs[i])))
    assert abs(tot - math.fsum(kl.ravel())) <= 1e-15 * (1 + abs(tot))


def test_argument_order_is_teacher_first():
    """KL is asymmetric; swapping teacher and student must change the value and
    the brute force must agree with the teacher-first orientation."""
    rng = np.random.default_rng(7)
    qt, kt, qs, ks = (_rand(rng, 1, 1, 3, 4, scale=2.0) for _ in range(4))
    kl, _, _, _ = oracle.fwd(qt, kt, qs, ks, 0.9, 0.9)
    kl_sw, _, _, _ = oracle.fwd(qs, ks, qt, kt, 0.9, 0.9)
    bk, _, _ = brute.kl_rows(qt[0, 0].tolist(), kt[0, 0].tolist(), qs[0, 0].tolist(), ks[0, 0].tolist(), 0.9, 0.9, False)
    assert np.max(np.abs(kl_sw - kl)) > 1e-3
    np.testing.assert_allclose(kl[0, 0], [float(x) for x in bk], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- exact / closed forms
@pytest.mark.parametrize("causal", [False, True])
def test_identical_inputs_give_exact_zero(causal):
    rng = np.random.default_rng(11)
    q = _rand(rng, 2, 3, 9, 8); k = _rand(rng, 2, 3, 13, 8)
    kl, lt, ls, tot = oracle.fwd(q, k, q, k, 0.35, 0.35, causal)
    assert np.all(kl == 0.0) and tot == 0.0
    np.testing.assert_array_equal(lt, ls)
    dq, dk = oracle.bwd(q, k, q, k, 0.35, 0.35, causal, g=np.linspace(-2, 3, 2 * 3 * 9))
    assert np.all(dq == 0.0) and np.all(dk == 0.0)


def test_two_keys_bernoulli_closed_form():
    """With two keys each softmax is a Bernoulli: p = sigmoid(s0 - s1)."""
    rng = np.random.default_rng(3)
    qt, qs = _rand(rng, 1, 1, 6, 3), _rand(rng, 1, 1, 6, 3)
    kt, ks = _rand(rng, 1, 1, 2, 3), _rand(rng, 1, 1, 2, 3)
    tt, ts = 0.8, 1.3
    kl, _, _, _ = oracle.fwd(qt, kt, qs, ks, tt, ts)
    for i in range(6):
        st = [tt * math.fsum(qt[0, 0, i] * kt[0, 0, j]) for j in range(2)]
        ss = [ts * math.fsum(qs[0, 0, i] * ks[0, 0, j]) for j in range(2)]
        p = 1.0 / (1.0 + math.exp(-(st[0] - st[1])))
        q = 1.0 / (1.0 + math.exp(-(ss[0] - ss[1])))
        ref = p * math.log(p / q) + (1 - p) * math.log((1 - p) / (1 - q))
        assert abs(kl[0, 0, i] - ref) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_student_gives_log_n_minus_teacher_entropy(causal):
    """Q_s = 0 (or tau_s = 0) makes the student uniform over the allowed keys:
    KL = ln|J_i| - H(P_t).  Entropy from scipy's entr on scipy's softmax."""
    rng = np.random.default_rng(5)
    n_q, n_k = 7, 11
    qt, kt = _rand(rng, 1, 1, n_q, 5), _rand(rng, 1, 1, n_k, 5)
    ks = _rand(rng, 1, 1, n_k, 3)
    qs0 = np.zeros((1, 1, n_q, 3))
    tt = 0.6
    kl0, _, ls0, _ = oracle.fwd(qt, kt, qs0, ks, tt, 0.5, causal)
    kl1, _, ls1, _ = oracle.fwd(qt, kt, _rand(rng, 1, 1, n_q, 3), ks, tt, 0.0, causal)
    s = tt * (qt[0, 0] @ kt[0, 0].T)
    n_allowed = _allowed(n_q, n_k, causal)
    for i, p in enumerate(_softmax_rows(s, n_allowed)):
        ref = math.log(n_allowed[i]) - float(np.sum(sp.entr(p)))
        assert abs(kl0[0, 0, i] - ref) <= 1e-13
        assert abs(kl1[0, 0, i] - ref) <= 1e-13
        assert abs(ls0[0, 0, i] - math.log(n_allowed[i])) <= 1e-14
        assert abs(ls1[0, 0, i] - math.log(n_allowed[i])) <= 1e-14


def test_causal_square_first_row_is_zero():
    rng = np.random.default_rng(8)
    qt, kt, qs, ks = (_rand(rng, 1, 2, 6, 4) for _ in range(4))
    kl, lt, _, _ = oracle.fwd(qt, kt, qs, ks, 0.5, 0.5, True)
    assert np.all(kl[:, :, 0] == 0.0)
    np.testing.assert_allclose(lt[0, :, 0], 0.5 * np.sum(qt[0, :, 0] * kt[0, :, 0], axis=-1), rtol=0, atol=1e-14)


def test_cross_entropy_minus_entropy_identity():
    """H(p, q) = H(p) + D_KL(p || q) ("Lecture 05", section 1), with both sides
    from scipy's log_softmax on numpy score matrices."""
    rng = np.random.default_rng(9)
    n_q, n_k = 8, 19
    qt, kt = _rand(rng, 1, 1, n_q, 6), _rand(rng, 1, 1, n_k, 6)
    qs, ks = _rand(rng, 1, 1, n_q, 4), _rand(rng, 1, 1, n_k, 4)
    for causal in (False, True):
        kl, _, _, _ = oracle.fwd(qt, kt, qs, ks, 0.4, 0.7, causal)
        st, ss = 0.4 * (qt[0, 0] @ kt[0, 0].T), 0.7 * (qs[0, 0] @ ks[0, 0].T)
        for i, n in enumerate(_allowed(n_q, n_k, causal)):
            lp, lq = sp.log_softmax(st[i, :n]), sp.log_softmax(ss[i, :n])
            p = np.exp(lp)
            ce, ent = -np.sum(p * lq), -np.sum(p * lp)
            assert abs(kl[0, 0, i] - (ce - ent)) <= 1e-12


def test_kl_nonnegative_on_random_rows():
    rng = np.random.default_rng(10)
    qt, kt, qs, ks = (_rand(rng, 2, 2, 24, 6, scale=2.0) for _ in range(4))
    for causal in (False, True):
        kl, _, _, _ = oracle.fwd(qt, kt, qs, ks, 0.9, 0.6, causal)
        assert np.all(kl >= -1e-12)
        assert np.count_nonzero(kl > 1e-3) > 0


# ---------------------------------------------------------------- invariances
def test_row_shift_and_key_permutation_invariance():
    rng = np.random.default_rng(12)
    n_q, n_k = 9, 14
    qt, kt = _rand(rng, 1, 1, n_q, 5), _rand(rng, 1, 1, n_k, 5)
    qs, ks = _rand(rng, 1, 1, n_q, 4), _rand(rng, 1, 1, n_k, 4)
    kl, _, _, _ = oracle.fwd(qt, kt, qs, ks, 0.5, 0.8)
    # shift every student score of row i by tau_s * c_i via an appended column
    c = _rand(rng, 1, 1, n_q, 1, scale=3.0)
    qs2 = np.concatenate([qs, c], axis=-1)
    ks2 = np.concatenate([ks, np.ones((1, 1, n_k, 1))], axis=-1)
    kl2, _, _, _ = oracle.fwd(qt, kt, qs2, ks2, 0.5, 0.8)
    np.testing.assert_allclose(kl2, kl, rtol=0, atol=1e-12)
    # jointly permute the keys of teacher and student (non-causal)
    perm = rng.permutation(n_k)
    kl3, _, _, _ = oracle.fwd(qt, kt[:, :, perm], qs, ks[:, :, perm], 0.5, 0.8)
    np.testing.assert_allclose(kl3, kl, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_log_count(causal):
    rng = np.random.default_rng(13)
    n_q, n_k = 5, 9
    z = np.zeros((1, 1, n_q, 4))
    k = _rand(rng, 1, 1, n_k, 4)
    _, lt, ls, _ = oracle.fwd(z, k, z, k, 1.0, 1.0, causal)
    ref = np.log(np.array(_allowed(n_q, n_k, causal), dtype=np.float64))
    np.testing.assert_allclose(lt[0, 0], ref, rtol=0, atol=1e-15)


# ---------------------------------------------------------------- gradients
def _loss(qt, kt, qs, ks, tt, ts, causal, g):
    kl, _, _, _ = oracle.fwd(qt, kt, qs, ks, tt, ts, causal)
    return math.fsum((g * kl).ravel())


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_central_differences(causal):
    rng = np.random.default_rng(21 + causal)
    B, H, n_q, n_k, d_t, d_s = 1, 2, 5, 7, 4, 3
    qt, kt = _rand(rng, B, H, n_q, d_t), _rand(rng, B, H, n_k, d_t)
    qs, ks = _rand(rng, B, H, n_q, d_s), _rand(rng, B, H, n_k, d_s)
    g = rng.uniform(-1.5, 2.0, size=(B, H, n_q))
    tt, ts = 0.6, 0.9
    dq, dk = oracle.bwd(qt, kt, qs, ks, tt, ts, causal, g=g)
    h = 1e-6
    fd_q = np.zeros_like(qs); fd_k = np.zeros_like(ks)
    for idx in np.ndindex(qs.shape):
        a, b = qs.copy(), qs.copy(); a[idx] += h; b[idx] -= h
        fd_q[idx] = (_loss(qt, kt, a, ks, tt, ts, causal, g) - _loss(qt, kt, b, ks, tt, ts, causal, g)) / (2 * h)
    for idx in np.ndindex(ks.shape):
        a, b = ks.copy(), ks.copy(); a[idx] += h; b[idx] -= h
        fd_k[idx] = (_loss(qt, kt, qs, a, tt, ts, causal, g) - _loss(qt, kt, qs, b, tt, ts, causal, g)) / (2 * h)
    assert np.all(np.abs(fd_q - dq) <= 1e-7 + 1e-5 * np.abs(dq))
    assert np.all(np.abs(fd_k - dk) <= 1e-7 + 1e-5 * np.abs(dk))
    assert np.linalg.norm(fd_q - dq) <= 1e-6 * np.linalg.norm(dq)
    assert np.linalg.norm(fd_k - dk) <= 1e-6 * np.linalg.norm(dk)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    """sum_j dK_s[j] = 0 (adding one vector to every student key leaves every
    row's student softmax unchanged) and <Q_s, dQ_s> = <K_s, dK_s> per head
    (scaling Q_s by (1+e) and K_s by 1/(1+e) leaves the scores unchanged)."""
    rng = np.random.default_rng(31)
    B, H, n_q, n_k = 2, 2, 12, 17
    qt, kt = _rand(rng, B, H, n_q, 6), _rand(rng, B, H, n_k, 6)
    qs, ks = _rand(rng, B, H, n_q, 5), _rand(rng, B, H, n_k, 5)
    g = rng.uniform(0.5, 1.5, size=(B, H, n_q))
    dq, dk = oracle.bwd(qt, kt, qs, ks, 0.5, 0.7, causal, g=g)
    scale = np.max(np.abs(dk))
    assert scale > 1e-3
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-13 * scale * n_k)
    lhs = np.einsum("bhnd,bhnd->bh", qs, dq)
    rhs = np.einsum("bhnd,bhnd->bh", ks, dk)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-13)


def test_sampled_entry_points_agree_with_full():
    rng = np.random.default_rng(41)
    B, H, n_q, n_k = 2, 3, 10, 15
    qt, kt = _rand(rng, B, H, n_q, 4), _rand(rng, B, H, n_k, 4)
    qs, ks = _rand(rng, B, H, n_q, 3), _rand(rng, B, H, n_k, 3)
    g = rng.normal(size=(B, H, n_q))
    for causal in (False, True):
        kl, lt, ls, _ = oracle.fwd(qt, kt, qs, ks, 0.5, 0.7, causal)
        dq, dk = oracle.bwd(qt, kt, qs, ks, 0.5, 0.7, causal, g=g)
        rows = np.array([0, 7, 11, 29, 59], dtype=np.int64)
        k2, l2, s2 = oracle.fwd_rows(qt, kt, qs, ks, 0.5, 0.7, causal, rows)
        np.testing.assert_array_equal(k2, kl.ravel()[rows])
        np.testing.assert_array_equal(l2, lt.ravel()[rows])
        np.testing.assert_array_equal(s2, ls.ravel()[rows])
        dq2 = oracle.dq_rows(qt, kt, qs, ks, 0.5, 0.7, causal, rows, g=g)
        np.testing.assert_allclose(dq2, dq.reshape(-1, 3)[rows], rtol=1e-13, atol=1e-15)
        keys = np.array([0, 4, 14], dtype=np.int64)
        dk2 = oracle.dk_keys(qt, kt, qs, ks, 0.5, 0.7, causal, 1, 2, keys, g=g)
        np.testing.assert_allclose(dk2, dk[1, 2, keys], rtol=1e-12, atol=1e-15)
