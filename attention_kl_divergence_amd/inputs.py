"""Seeded synthetic inputs for the fused attention-KL primitive.

This module holds none of the method's arithmetic: it only draws the teacher
and student query/key tensors with the shapes and value distributions of the
workloads the primitive is measured on, rounds them once to the compute dtype,
and hands the same bits to every consumer (the HIP path, the CPU oracle, the
benchmark).  The pages name no dataset for this primitive; every input is
synthetic.

Recipe (all draws are numpy PCG64 standard normals in float32, taken in the
order listed; every transform is done in float32; bf16 inputs are then rounded
once, round-to-nearest-even):
  iid        Q_t, K_t, Q_s, K_s independent N(0, 1)
  perturbed  Q_t, K_t ~ N(0, 1); Q_s = Q_t + sigma*N(0, 1); K_s = K_t + sigma*N(0, 1)
  peaked     Q, K ~ N(0, 1); Q_t = 3 Q, K_t = K; Q_s = Q + 0.3 N(0, 1); K_s = K + 0.3 N(0, 1)
Scales default to tau = 1/sqrt(d) per side, rounded to float32.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    n_q: int
    n_k: int
    d_t: int
    d_s: int
    dtype: str          # "bf16" or "f32"
    causal: bool
    recipe: str         # "iid" | "perturbed" | "peaked"
    sigma: float        # noise scale for "perturbed"
    seed: int

    @property
    def tau_t(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d_t)))

    @property
    def tau_s(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d_s)))

    def resized(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def pairs(self) -> int:
        """Unmasked (query, key) pairs."""
        if not self.causal:
            return self.B * self.H * self.n_q * self.n_k
        return self.B * self.H * _causal_pairs(self.n_q, self.n_k)


def _causal_pairs(n_q: int, n_k: int) -> int:
    off = n_k - n_q
    # sum_{i=0}^{n_q-1} (i + off + 1), all <= n_k when n_q <= n_k
    return n_q * (off + 1) + n_q * (n_q - 1) // 2


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 1, 128, 128, 64, 64, "f32", False, "iid", 0.0, 1),
    "corr_4k": Workload("corr_4k", 2, 16, 4096, 4096, 128, 128, "bf16", False, "perturbed", 0.3, 2),
    "causal_32k": Workload("causal_32k", 1, 8, 32768, 32768, 128, 128, "bf16", True, "perturbed", 0.5, 3),
    "mixed_dims_2k": Workload("mixed_dims_2k", 4, 12, 2048, 2048, 128, 64, "bf16", False, "iid", 0.0, 4),
    "cross_512x16k": Workload("cross_512x16k", 8, 16, 512, 16384, 128, 128, "bf16", False, "peaked", 0.3, 5),
    "corr_16k": Workload("corr_16k", 2, 16, 16384, 16384, 128, 128, "bf16", False, "perturbed", 0.3, 16),
    "corr_16k_causal": Workload("corr_16k_causal", 2, 16, 16384, 16384, 128, 128, "bf16", True, "perturbed", 0.3, 17),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32 holding bf16 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs: the sum stays below 2^32 (largest finite pattern 0xFF7FFFFF)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32).reshape(x.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are exactly representable in bf16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def make(w: Workload, seed: int | None = None) -> dict:
    """Draw the four tensors of workload ``w``.

    Returns a dict with float32 arrays 'q_t', 'k_t', 'q_s', 'k_s' ([B, H, N, d]),
    whose values are exactly representable in ``w.dtype``.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    qshape_t = (w.B, w.H, w.n_q, w.d_t)
    kshape_t = (w.B, w.H, w.n_k, w.d_t)
    qshape_s = (w.B, w.H, w.n_q, w.d_s)
    kshape_s = (w.B, w.H, w.n_k, w.d_s)

    def draw(shape):
        return rng.standard_normal(shape, dtype=np.float32)

    if w.recipe == "iid":
        q_t, k_t, q_s, k_s = draw(qshape_t), draw(kshape_t), draw(qshape_s), draw(kshape_s)
    elif w.recipe == "perturbed":
        if w.d_t != w.d_s:
            raise ValueError("perturbed recipe needs d_t == d_s")
        q_t, k_t = draw(qshape_t), draw(kshape_t)
        sig = np.float32(w.sigma)
        q_s = q_t + sig * draw(qshape_s)
        k_s = k_t + sig * draw(kshape_s)
    elif w.recipe == "peaked":
        if w.d_t != w.d_s:
            raise ValueError("peaked recipe needs d_t == d_s")
        q, k = draw(qshape_t), draw(kshape_t)
        q_t = np.float32(3.0) * q
        k_t = k
        q_s = q + np.float32(0.3) * draw(qshape_s)
        k_s = k + np.float32(0.3) * draw(kshape_s)
    else:
        raise ValueError(f"unknown recipe {w.recipe}")
    out = {"q_t": q_t, "k_t": k_t, "q_s": q_s, "k_s": k_s}
    if w.dtype == "bf16":
        out = {n: round_bf16(a) for n, a in out.items()}
    elif w.dtype == "f32":
        out = {n: np.ascontiguousarray(a, dtype=np.float32) for n, a in out.items()}
    else:
        raise ValueError(f"unknown dtype {w.dtype}")
    return out


def upstream_grad(B: int, H: int, n_q: int, seed: int) -> np.ndarray:
    """Random per-row upstream gradients dL/dKL_r (float32, N(0, 1))."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((B, H, n_q), dtype=np.float32)


# ----------------------------------------------------------------------------
# Vocabulary-logit workloads (distillation loss over output logits).  The pages
# name no dataset or model for them; the logits are synthetic with the
# character of language-model outputs: a broad Gaussian body plus a few
# strongly preferred tokens per row, and a student that is a noisy copy of the
# teacher.  Each row is drawn from its own generator (seed, row), so any subset
# of rows can be regenerated on its own.
#
# Recipe "lm" (float32, in this order per row): z_t = 2.5 N(0, 1) over V; 16
# token indices uniform in [0, V) (repeats allowed) each get + U(4, 12); then
# z_s = z_t + sigma N(0, 1).  "iid": z_t, z_s independent 2.5 N(0, 1).
# bf16 workloads round both once (ties to even).

@dataclasses.dataclass(frozen=True)
class VocabWorkload:
    name: str
    rows: int
    V: int
    dtype: str          # "bf16" or "f32"
    temperature: float
    recipe: str         # "lm" | "iid"
    sigma: float
    seed: int

    def resized(self, **kw) -> "VocabWorkload":
        return dataclasses.replace(self, **kw)


VOCAB_WORKLOADS = {
    "kd_logits_small": VocabWorkload("kd_logits_small", 37, 32000, "bf16", 2.0, "lm", 0.5, 31),
    "kd_logits_odd_f32": VocabWorkload("kd_logits_odd_f32", 9, 50257, "f32", 1.0, "lm", 0.5, 32),
    "kd_logits_short": VocabWorkload("kd_logits_short", 70, 1000, "bf16", 4.0, "iid", 0.0, 33),
    "kd_logits_4k_128k": VocabWorkload("kd_logits_4k_128k", 4096, 128256, "bf16", 2.0, "lm", 0.5, 34),
    "kd_logits_8k_50257": VocabWorkload("kd_logits_8k_50257", 8192, 50257, "bf16", 2.0, "lm", 0.5, 35),
}


def make_vocab(w: VocabWorkload, rows=None, threads: int = 8) -> tuple:
    """Teacher and student logits of ``w`` as float32 arrays [n, V] exactly
    representable in ``w.dtype``; ``rows`` (an iterable of row indices) selects
    a subset, default all rows.  Rows are drawn on ``threads`` threads (each
    row from its own generator, so the result does not depend on it)."""
    from concurrent.futures import ThreadPoolExecutor

    idx = list(range(w.rows)) if rows is None else [int(r) for r in rows]
    if w.recipe not in ("lm", "iid"):
        raise ValueError(f"unknown vocab recipe {w.recipe}")
    if w.dtype not in ("bf16", "f32"):
        raise ValueError(f"unknown dtype {w.dtype}")
    zt = np.empty((len(idx), w.V), dtype=np.float32)
    zs = np.empty((len(idx), w.V), dtype=np.float32)
    body = np.float32(2.5)

    def one(n):
        rng = np.random.Generator(np.random.PCG64([w.seed, idx[n]]))
        t = zt[n]
        rng.standard_normal(out=t, dtype=np.float32)
        t *= body
        s = zs[n]
        if w.recipe == "lm":
            hot = rng.integers(0, w.V, size=16)
            t[hot] += rng.uniform(4.0, 12.0, size=16).astype(np.float32)
            rng.standard_normal(out=s, dtype=np.float32)
            s *= np.float32(w.sigma)
            s += t
        else:
            rng.standard_normal(out=s, dtype=np.float32)
            s *= body
        if w.dtype == "bf16":
            zt[n] = round_bf16(t)
            zs[n] = round_bf16(s)

    with ThreadPoolExecutor(max_workers=max(1, int(threads))) as ex:
        list(ex.map(one, range(len(idx))))
    return zt, zs
