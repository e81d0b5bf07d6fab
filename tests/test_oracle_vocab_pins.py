"""Pins for the oracle's vocabulary-logit KL (distillation loss at temperature
T between the teacher and student output distributions: "Lecture 05 - Where It
All Lands", sections 3.1 and 3.3).

A vocabulary row is the attention case with one query q = [1], keys
k_v = z[v] (d = 1) and tau = 1/T, so the attention oracle -- a separate code
path, itself pinned by 50-digit brute force -- fixes the values; the decimal
brute force is applied here directly as well.  Gradients are pinned by central
finite differences, and the sum-to-zero and temperature identities hold.
"""
import math

import numpy as np
import pytest

import oracle
from tests import brute


def test_vocab_rows_equal_the_single_query_attention_case():
    rng = np.random.default_rng(201)
    rows, V, T = 5, 37, 1.7
    zt = rng.standard_normal((rows, V)) * 2.0
    zs = rng.standard_normal((rows, V)) * 2.0
    kl, lt, ls, tot = oracle.vocab_fwd(zt, zs, T)
    for r in range(rows):
        one = np.ones((1, 1, 1, 1))
        akl, alt, als, _ = oracle.fwd(one, zt[r].reshape(1, 1, V, 1), one, zs[r].reshape(1, 1, V, 1),
                                      1.0 / T, 1.0 / T, False)
        assert abs(kl[r] - akl[0, 0, 0]) <= 1e-14 * (1 + abs(akl[0, 0, 0]))
        assert abs(lt[r] - alt[0, 0, 0]) <= 1e-14 * (1 + abs(alt[0, 0, 0]))
        assert abs(ls[r] - als[0, 0, 0]) <= 1e-14 * (1 + abs(als[0, 0, 0]))
    assert abs(tot - math.fsum(kl)) <= 1e-14 * (1 + abs(tot))


def test_vocab_matches_decimal_brute_force():
    rng = np.random.default_rng(202)
    zt = rng.standard_normal((3, 6)) * 1.5
    zs = rng.standard_normal((3, 6)) * 1.5
    T = 0.8
    kl, lt, ls, _ = oracle.vocab_fwd(zt, zs, T)
    for r in range(3):
        bk, bl, bs = brute.kl_rows([[1.0]], [[v] for v in zt[r]], [[1.0]], [[v] for v in zs[r]], 1.0 / T, 1.0 / T,
                                   False)
        assert abs(kl[r] - float(bk[0])) <= 1e-14 + 1e-12 * abs(float(bk[0]))
        assert abs(lt[r] - float(bl[0])) <= 1e-14 * (1 + abs(float(bl[0])))


def test_vocab_shift_invariance_and_identical_rows():
    rng = np.random.default_rng(203)
    zt = rng.standard_normal((4, 50)); zs = rng.standard_normal((4, 50))
    kl, _, _, _ = oracle.vocab_fwd(zt, zs, 1.3)
    kl2, _, _, _ = oracle.vocab_fwd(zt + rng.standard_normal((4, 1)) * 5, zs - 3.0, 1.3)
    np.testing.assert_allclose(kl2, kl, rtol=1e-12, atol=1e-14)
    z0, _, _, _ = oracle.vocab_fwd(zt, zt, 2.0)
    assert not np.any(z0)
    assert np.all(kl >= 0)


@pytest.mark.parametrize("teacher", [False, True])
def test_vocab_gradients_match_central_differences(teacher):
    rng = np.random.default_rng(204 + teacher)
    rows, V, T = 3, 9, 1.6
    zt = rng.standard_normal((rows, V)); zs = rng.standard_normal((rows, V))
    g = rng.uniform(-1.0, 2.0, size=rows)
    out = oracle.vocab_bwd(zt, zs, T, g=g, teacher=True)
    an = out[1] if teacher else out[0]

    def loss(a, b):
        kl, _, _, _ = oracle.vocab_fwd(a, b, T)
        return math.fsum(g * kl)
    h = 1e-6
    fd = np.zeros_like(an)
    for idx in np.ndindex(an.shape):
        if teacher:
            a, b = zt.copy(), zt.copy(); a[idx] += h; b[idx] -= h
            fd[idx] = (loss(a, zs) - loss(b, zs)) / (2 * h)
        else:
            a, b = zs.copy(), zs.copy(); a[idx] += h; b[idx] -= h
            fd[idx] = (loss(zt, a) - loss(zt, b)) / (2 * h)
    assert np.all(np.abs(fd - an) <= 1e-8 + 1e-5 * np.abs(an))
    # shifting a row's logits leaves KL unchanged, so each gradient row sums to 0
    np.testing.assert_allclose(an.sum(axis=1), 0.0, atol=1e-14 * V)


def test_vocab_two_classes_closed_form():
    """Two logits: KL = p ln(p/q) + (1-p) ln((1-p)/(1-q)), p = sigmoid((a0-a1)/T)."""
    zt = np.array([[1.2, -0.7]]); zs = np.array([[0.1, 0.4]]); T = 1.4
    p = 1 / (1 + math.exp(-(zt[0, 0] - zt[0, 1]) / T))
    q = 1 / (1 + math.exp(-(zs[0, 0] - zs[0, 1]) / T))
    ref = p * math.log(p / q) + (1 - p) * math.log((1 - p) / (1 - q))
    kl, _, _, _ = oracle.vocab_fwd(zt, zs, T)
    assert abs(kl[0] - ref) <= 1e-15
    dzs = oracle.vocab_bwd(zt, zs, T)
    assert abs(dzs[0, 0] - (q - p) / T) <= 1e-15 and abs(dzs[0, 1] - (p - q) / T) <= 1e-15
