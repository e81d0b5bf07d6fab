"""50-digit decimal brute force of the attention KL, for pinning the oracle on tiny inputs.

Written independently of oracle/: it forms the two softmax distributions as
explicit ratios p_j = e^{s_j} / sum_k e^{s_k} and sums p_j ln(p_j / q_j)
(forward KL, teacher first, natural log; "Lecture 05 - Where It All Lands",
section 3.1), with every step in 50-digit decimal arithmetic.
"""
from decimal import Decimal, getcontext

getcontext().prec = 50


def _dec(x) -> Decimal:
    return Decimal(float(x))  # exact: a binary float converts to decimal exactly


def kl_rows(q_t, k_t, q_s, k_s, tau_t, tau_s, causal):
    """q_*: [n_q][d], k_*: [n_k][d] nested sequences of floats. Returns (kl, lse_t, lse_s) lists of Decimal."""
    n_q, n_k = len(q_t), len(k_t)
    tt, ts = _dec(tau_t), _dec(tau_s)
    out_kl, out_lt, out_ls = [], [], []
    for i in range(n_q):
        keys = [j for j in range(n_k) if (not causal) or j <= i + (n_k - n_q)]
        st = [tt * sum(_dec(a) * _dec(b) for a, b in zip(q_t[i], k_t[j])) for j in keys]
        ss = [ts * sum(_dec(a) * _dec(b) for a, b in zip(q_s[i], k_s[j])) for j in keys]
        et = [x.exp() for x in st]
        es = [x.exp() for x in ss]
        zt, zs = sum(et), sum(es)
        p = [e / zt for e in et]
        q = [e / zs for e in es]
        kl = sum(pj * (pj / qj).ln() for pj, qj in zip(p, q))
        out_kl.append(kl)
        out_lt.append(zt.ln())
        out_ls.append(zs.ln())
    return out_kl, out_lt, out_ls
