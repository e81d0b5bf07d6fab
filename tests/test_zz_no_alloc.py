"""GPU test of the allocation-free split forward (streamkl_fwd_split_noalloc,
for callers that cannot allocate device memory): called through the C ABI, it
gives the same bits as streamkl_fwd_split with a caller workspace, on two calls
in a row (the second smaller, reusing the scratch array the first wrote), and
rejects states that would not fit in its scratch array."""
import ctypes

import numpy as np
import pytest

import attention_kl_divergence_amd as skl
from attention_kl_divergence_amd import inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

W = inputs.WORKLOADS


def _run(lib, w, n_split, noalloc):
    x = inputs.make(w)
    d = {k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in x.items()}
    B, H, n_q, n_k, d_t, d_s = w.B, w.H, w.n_q, w.n_k, w.d_t, w.d_s
    kl = torch.full((B, H, n_q), float("nan"), dtype=torch.float32, device="cuda")
    lt, ls = torch.full_like(kl, float("nan")), torch.full_like(kl, float("nan"))
    tot = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = (d["q_t"].data_ptr(), d["k_t"].data_ptr(), d["q_s"].data_ptr(), d["k_s"].data_ptr(), skl.STREAMKL_BF16,
            B, H, n_q, n_k, d_t, d_s, None, w.tau_t, w.tau_s, int(w.causal), n_split)
    outs = (kl.data_ptr(), lt.data_ptr(), ls.data_ptr(), tot.data_ptr(), stream)
    if noalloc:
        code = lib.streamkl_fwd_split_noalloc(*args, *outs)
    else:
        nbytes = int(lib.streamkl_fwd_split_workspace_size(B, H, n_q, n_split))
        ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
        code = lib.streamkl_fwd_split(*args, ws.data_ptr(), nbytes, *outs)
    assert code == skl.STREAMKL_OK, skl.status_string(code)
    torch.cuda.synchronize()
    return kl.cpu(), lt.cpu(), ls.cpu(), tot.cpu()


def test_noalloc_split_forward_matches_workspace_entry_point():
    lib = skl.load_library()
    cases = [(W["cross_512x16k"].resized(B=2, H=4, n_q=300, n_k=2000, seed=301), 4),
             (W["corr_4k"].resized(B=1, H=2, n_q=100, n_k=700, causal=True, seed=302), 3)]
    for w, n_split in cases:  # the second call is smaller and reuses the scratch array
        print(f"[noalloc] {w} split {n_split}", flush=True)
        got = _run(lib, w, n_split, noalloc=True)
        ref = _run(lib, w, n_split, noalloc=False)
        for g, r in zip(got, ref):
            assert not torch.isnan(g).any()
            assert torch.equal(g, r)


def test_noalloc_split_forward_rejects_states_past_its_scratch():
    lib = skl.load_library()
    A = 0x7f0000000000  # never dereferenced: the size is rejected before any launch
    B, H, n_q, n_split = 64, 16, 4096, 8  # 8 x 64 x 16 x 4096 rows x 24 B = 768 MiB of states
    assert lib.streamkl_fwd_split_workspace_size(B, H, n_q, n_split) > skl.NOALLOC_SCRATCH_BYTES
    code = lib.streamkl_fwd_split_noalloc(A, A + 0x100000, A + 0x200000, A + 0x300000, skl.STREAMKL_BF16, B, H,
                                          n_q, 8192, 128, 128, None, 0.088, 0.088, 0, n_split, A + 0x400000,
                                          A + 0x500000, A + 0x600000, None, None)
    assert code == skl.STREAMKL_ERR_WORKSPACE
