"""Properties of the generated gfx950 code that the kernels' correctness rests on
(CPU only: the device code is compiled to assembly here, nothing runs).

Streamed tiles are written into LDS by direct buffer->LDS loads, which count on
the issuing wave's vmcnt.  A workgroup barrier does not wait for them by
itself, so every s_barrier in the forward and backward kernels must directly
follow an s_waitcnt that drains vmcnt; otherwise a wave could pass the barrier
with its share of a tile still in flight and other waves would read stale LDS.
"""
import os
import re
import shutil
import subprocess

import pytest

from attention_kl_divergence_amd import build as hip_build

HIPCC = hip_build.HIPCC


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "streamkl.s"
    flags = [f for f in hip_build.FLAGS if f not in ("-shared",)]
    res = subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", "-o", str(out), hip_build.SRC],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text().split("\n")


def _kernels(lines):
    starts = [(i, l.split(":")[0]) for i, l in enumerate(lines)
              if re.match(r"^_ZN12_GLOBAL__N_1\d+streamkl_(fwd|bwd)_kernel\w*:", l)]
    for i, name in starts:
        end = next(j for j in range(i, len(lines)) if lines[j].startswith(".Lfunc_end"))
        yield name, lines[i:end]


def test_every_kernel_barrier_drains_vmcnt_first(asm):
    """Walking back from each s_barrier, the nearest s_waitcnt drains vmcnt and
    no vector-memory load is issued between it and the barrier."""
    kernels = list(_kernels(asm))
    # {bf16, f32} x {64, 128}^2 x {causal, not}: 16 forward kernels, 32 student
    # backward kernels ({scalar, per-row} upstream gradient), 16 teacher ones,
    # and 32 grouped-head backward kernels (student and teacher)
    assert len(kernels) == 96
    for name, body in kernels:
        nbar = 0
        for k, line in enumerate(body):
            if not line.strip().startswith("s_barrier"):
                continue
            nbar += 1
            j = k - 1
            while j > 0 and not body[j].strip().startswith("s_waitcnt"):
                op = body[j].strip().split(" ")[0]
                assert not op.startswith(("global_load", "buffer_load", "flat_load")), \
                    f"{name}: load {body[j]!r} between the last wait and the barrier at +{k}"
                assert not re.match(r"^\.LBB|^; %bb", body[j]), f"{name}: barrier at +{k} starts a block without a wait"
                j -= 1
            assert "vmcnt(0)" in body[j], f"{name}: barrier at +{k} after {body[j]!r}"
        assert nbar >= 2, name


def test_no_spills_in_the_mfma_loops(asm):
    """Register spills inside the hot loops would make them memory-bound: no
    basic block that issues MFMAs touches scratch, the kernels with one KL head
    per output head do not spill at all, and the grouped-head ones spill only
    a few registers (at their head boundaries)."""
    text = "\n".join(asm)
    found = list(re.finditer(r"\.name:\s+(_ZN12_GLOBAL__N_1\d+streamkl_\w+)[\s\S]*?"
                             r"\.private_segment_fixed_size:\s+(\d+)", text))
    # 96 forward/backward instantiations + the sum, merge and two split-reduce kernels
    assert len(found) == 100
    for m in found:
        # grouped-head backward kernels (last template flag GRP = 1) keep more
        # state across their head loop and spill at the head boundaries
        grouped = m.group(1).endswith("Lb1EEEvNS_9BwdParamsES1_")
        assert int(m.group(2)) <= (128 if grouped else 0), m.group(1)
    for name, body in _kernels(asm):
        block, mfma, scratch = "entry", 0, 0
        for line in body + [".LBBend:"]:
            if re.match(r"^\.LBB\d+_\d+:|^\.LBBend:|^; %bb", line):
                assert not (mfma and scratch), f"{name}: scratch access in MFMA block {block}"
                block, mfma, scratch = line.split(":")[0], 0, 0
            elif "v_mfma" in line:
                mfma += 1
            elif "scratch_" in line:
                scratch += 1


def test_streamed_tiles_use_buffer_loads_into_lds(asm):
    """Every forward and backward kernel moves its streamed tiles with 16-byte
    buffer->LDS loads (one wave-uniform descriptor per tile, per-lane 32-bit
    offsets) and has no per-lane 64-bit global addressing left for them."""
    for name, body in _kernels(asm):
        ops = [l.strip() for l in body]
        assert any(o.startswith("buffer_load_dwordx4") and o.endswith(" lds") for o in ops), name
        assert not any(o.startswith("global_load_lds") for o in ops), name


def test_forward_fast_path_keeps_its_fmas_beside_the_exponentials(asm):
    """In every bf16 forward kernel, the block of the steady-state update (the
    tile's 32 exponentials, before the wave votes on a rebase) also holds all
    64 FMAs of the tile (32 scale-shifts, 32 teacher-weighted sums): none is
    sunk past the rebase branch into a serial tail of its own."""
    starts = [(i, l.split(":")[0]) for i, l in enumerate(asm)
              if re.match(r"^_ZN12_GLOBAL__N_1\d+streamkl_fwd_kernelIDF16b\w*:", l)]
    assert len(starts) == 8
    for i, name in starts:
        end = next(j for j in range(i, len(asm)) if asm[j].startswith(".Lfunc_end"))
        best, ops = 0, []
        for line in asm[i:end] + [".LBBend:"]:
            if re.match(r"^\.LBB\d+_\d+:|^\.LBBend:|^; %bb", line):
                # exactly 32: the rebase paths add two for the rescale factors
                if sum(o == "v_exp_f32_e32" for o in ops) == 32:
                    best = max(best, sum(o in ("v_fma_f32", "v_fmac_f32_e32") for o in ops))
                ops = []
            elif line.startswith("\t"):
                ops.append(line.strip().split(" ")[0])
        assert best >= 64, f"{name}: {best} FMAs beside the exponentials"


def test_vocab_kernels_do_not_spill_and_stay_vectorised(tmp_path):
    """The vocabulary-logit kernels stream HBM: no register spills (private
    segment 0) in any instantiation, and the vector paths move the logits with
    16-byte loads."""
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path / "vocab.s"
    flags = [f for f in hip_build.FLAGS if f not in ("-shared",)]
    res = subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", "-o", str(out), hip_build.SRCS[1]],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    text = out.read_text()
    found = re.findall(r"\.name:\s+(_ZN12_GLOBAL__N_1\d+streamkl_vocab_\w+)[\s\S]*?"
                       r"\.private_segment_fixed_size:\s+(\d+)", text)
    # {bf16, f32} x {vector, element} x (forward {1,4,8,16} waves per row + backward and fused
    # {student, teacher} x {1,4,8,16})
    assert len(found) == 2 * 2 * (4 + 2 * 2 * 4)
    for name, priv in found:
        assert int(priv) == 0, name
    lines = text.split("\n")
    starts = [i for i, l in enumerate(lines) if re.match(r"^_ZN12_GLOBAL__N_1\d+streamkl_vocab_fwd_kernelIDF16bLb1E", l)]
    assert starts
    for i in starts:
        end = next(j for j in range(i, len(lines)) if lines[j].startswith(".Lfunc_end"))
        assert any("global_load_dwordx4" in l for l in lines[i:end])
