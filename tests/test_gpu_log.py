"""STREAMKL_LOG=1 prints one line per launch on stderr, with the chosen
configuration and grid; without it the library prints nothing."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import torch
import attention_kl_divergence_amd as skl
g = torch.Generator(device="cuda").manual_seed(3)
q = torch.randn(1, 2, 70, 64, device="cuda", generator=g).bfloat16()
k = torch.randn(1, 2, 90, 64, device="cuda", generator=g).bfloat16()
kl, lt, ls, tot = skl.streamkl_fwd(q, k, q, k)
skl.streamkl_bwd(q, k, q, k, lt, ls)
z = torch.randn(5, 1000, device="cuda", generator=g).bfloat16()
skl.streamkl_vocab_fwd(z, z)
torch.cuda.synchronize()
print("done")
"""


def test_log_lines_name_the_launch_configuration():
    env = dict(os.environ, STREAMKL_LOG="1")
    res = subprocess.run([sys.executable, "-c", SCRIPT], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l for l in res.stderr.splitlines() if l.startswith("[streamkl]")]
    fwd = [l for l in lines if l.startswith("[streamkl] fwd ")]
    bwd = [l for l in lines if l.startswith("[streamkl] bwd ")]
    voc = [l for l in lines if l.startswith("[streamkl] vocab fwd ")]
    assert len(fwd) == 1 and "B=1 H=2 n_q=70 n_k=90 d_t=64 d_s=64 causal=0" in fwd[0] and "grid 2 x 256" in fwd[0]
    assert len(bwd) == 1 and "grid 4 x 256" in bwd[0] and "1 query-major + 1 key-major" in bwd[0]
    assert len(voc) == 1 and "rows=5 V=1000" in voc[0]


def test_silent_without_the_variable(capfd):
    if os.environ.get("STREAMKL_LOG", "0") not in ("", "0"):
        pytest.skip("STREAMKL_LOG is set in this environment")
    import attention_kl_divergence_amd as skl
    q = torch.randn(1, 1, 40, 64, device="cuda").bfloat16()
    skl.streamkl_fwd(q, q, q, q)
    torch.cuda.synchronize()
    assert "[streamkl]" not in capfd.readouterr().err
