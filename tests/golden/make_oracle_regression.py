"""Write tests/golden/tiny_f32_oracle.json: the oracle's outputs on the first rows of
the tiny fp32 workload (B=1, H=1, N_Q=N_K=128, d=64, i.i.d. N(0,1), seed 1).

Calls only oracle/ and the seeded input generator; it freezes the oracle and the
generator together so an unintended change in either shows up as a test failure.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from attention_kl_divergence_amd import inputs  # noqa: E402

w = inputs.WORKLOADS["tiny_f32"]
x = inputs.make(w)
kl, lt, ls, tot = oracle.fwd(x["q_t"], x["k_t"], x["q_s"], x["k_s"], w.tau_t, w.tau_s, w.causal)
dq, dk = oracle.bwd(x["q_t"], x["k_t"], x["q_s"], x["k_s"], w.tau_t, w.tau_s, w.causal)
out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_f32_oracle.json")
with open(out, "w") as f:
    json.dump({"workload": "tiny_f32", "kl_rows_0_16": kl.ravel()[:16].tolist(),
               "lse_t_0_16": lt.ravel()[:16].tolist(), "lse_s_0_16": ls.ravel()[:16].tolist(),
               "kl_sum": tot, "dq_s_row0": dq[0, 0, 0].tolist(), "dk_s_row0": dk[0, 0, 0].tolist()}, f, indent=1)
print(out)
