"""Write tests/golden/closed_form_cases.json: tiny attention-KL cases whose value is
fixed by hand-derived closed forms (no oracle or GPU output is used).

KL here is forward KL, teacher first, natural log ("Lecture 05 - Where It All
Lands", section 3.1); for one row with scores s_t, s_s over the allowed keys,
KL = sum_j P_t[j] (s_t[j] - s_s[j]) - LSE(s_t) + LSE(s_s).
"""
import json
import math
import os

e = math.e
cases = [
    dict(name="two_keys", q_t=[[1.0]], k_t=[[1.0], [0.0]], q_s=[[0.0]], k_s=[[1.0], [0.0]],
         tau_t=1.0, tau_s=1.0, causal=False,
         derivation="s_t=(1,0), s_s=(0,0): KL = ln2 - ln(1+e) + e/(1+e)",
         kl=[math.log(2) - math.log(1 + e) + e / (1 + e)]),
    dict(name="three_keys", q_t=[[2.0]], k_t=[[1.0], [0.0], [0.0]], q_s=[[1.0]], k_s=[[0.0], [1.0], [0.0]],
         tau_t=1.0, tau_s=1.0, causal=False,
         derivation="s_t=(2,0,0), s_s=(0,1,0): KL = (2e^2-1)/(e^2+2) - ln(e^2+2) + ln(e+2)",
         kl=[(2 * e * e - 1) / (e * e + 2) - math.log(e * e + 2) + math.log(e + 2)]),
    dict(name="causal_two_rows", q_t=[[1.0], [1.0]], k_t=[[0.0], [1.0]], q_s=[[1.0], [1.0]], k_s=[[1.0], [0.0]],
         tau_t=1.0, tau_s=1.0, causal=True,
         derivation="row 0 sees one key: KL=0; row 1: s_t=(0,1), s_s=(1,0): KL=(e-1)/(e+1)",
         kl=[0.0, (e - 1) / (e + 1)]),
    dict(name="temperature_half", q_t=[[1.0]], k_t=[[1.0], [0.0]], q_s=[[0.0]], k_s=[[1.0], [0.0]],
         tau_t=0.5, tau_s=0.5, causal=False,
         derivation="s_t=(1/2,0), s_s=(0,0): KL = ln2 - ln(1+sqrt(e)) + sqrt(e)/(2(1+sqrt(e)))",
         kl=[math.log(2) - math.log(1 + math.sqrt(e)) + 0.5 * math.sqrt(e) / (1 + math.sqrt(e))]),
]
out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "closed_form_cases.json")
with open(out, "w") as f:
    json.dump({"source": "hand-derived closed forms of forward KL between two softmax rows; "
                         "definition: 'Lecture 05 - Where It All Lands', section 3.1",
               "cases": cases}, f, indent=1)
print(out)
