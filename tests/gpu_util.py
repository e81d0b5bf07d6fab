"""Helpers shared by the GPU parity tests: device copies of the seeded inputs and
the tolerance checks.

Tolerances (per-row KL, gradients) are the ones stated for this primitive:
per-row KL |err| <= 1e-4 + 1e-3 |KL| for fp32 inputs and <= 2e-3 + 1e-2 |KL| for
bf16 inputs; gradients relative L2 <= 1e-2 for bf16.  For fp32 gradients
(relative L2 <= 1e-4), log-normalisers (<= 1e-5 (1 + |LSE|) fp32, <= 1e-4 (1 + |LSE|)
bf16) and the summed KL (the per-row bounds summed over rows) the bounds are
derived from fp32 accumulation and are listed with the other readings in the
design notes.
"""
import numpy as np

KL_TOL = {"f32": (1e-4, 1e-3), "bf16": (2e-3, 1e-2)}
LSE_TOL = {"f32": 1e-5, "bf16": 1e-4}
GRAD_TOL = {"f32": 1e-4, "bf16": 1e-2}


def to_device(x: dict, dtype: str):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(tdt).cuda() for k, v in x.items()}


def as_f64(x: dict):
    return {k: np.ascontiguousarray(v, dtype=np.float64) for k, v in x.items()}


def check_kl(gpu, ref, dtype, what="kl"):
    a, r = KL_TOL[dtype]
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref)
    bound = a + r * np.abs(ref)
    worst = int(np.argmax(err - bound))
    assert np.all(err <= bound), f"{what}: worst at {worst}: gpu {gpu.ravel()[worst]} ref {ref.ravel()[worst]}"
    return float(np.max(err))


def check_lse(gpu, ref, dtype, what="lse"):
    t = LSE_TOL[dtype]
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref)
    assert np.all(err <= t * (1 + np.abs(ref))), f"{what}: max err {err.max()}"
    return float(np.max(err))


def check_sum(gpu_sum, ref_rows, dtype):
    a, r = KL_TOL[dtype]
    ref = float(np.sum(ref_rows, dtype=np.float64))
    bound = ref_rows.size * a + r * float(np.sum(np.abs(ref_rows)))
    assert abs(float(gpu_sum) - ref) <= bound, f"sum gpu {gpu_sum} ref {ref} bound {bound}"


def rel_l2(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(gpu - ref) / (den if den > 0 else 1.0))


def check_grad(gpu, ref, dtype, what="grad"):
    e = rel_l2(gpu, ref)
    assert e <= GRAD_TOL[dtype], f"{what}: relative L2 {e}"
    return e
