"""Compile the HIP library (gfx950 only) into attention_kl_divergence_amd/libstreamkl.so.

Two translation units, csrc/streamkl.hip (attention KL) and csrc/streamkl_vocab.hip
(vocabulary-logit KL), compiled in parallel with hipcc for --offload-arch=gfx950
into objects under a temporary folder, then linked into one shared library.
Packed fp32 VALU instructions are disabled for the device code (the host pass
warns that it does not know the feature; that warning is harmless).
"""
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "streamkl.hip")
SRCS = [SRC, os.path.join(HERE, "csrc", "streamkl_vocab.hip")]
LIB = os.path.join(HERE, "libstreamkl.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-mllvm", "--amdgpu-mfma-vgpr-form",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _filtered(stderr: str) -> str:
    noise = "is not a recognized feature for this target"
    return "\n".join(l for l in stderr.splitlines() if noise not in l)


def build(verbose: bool = False, extra=()) -> str:
    with tempfile.TemporaryDirectory(prefix="streamkl_build_") as tmp:
        objs, procs = [], []
        for src in SRCS:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [HIPCC, *FLAGS, *extra, "-c", "-o", obj, src]
            if verbose:
                print(" ".join(cmd))
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
            objs.append(obj)
        for cmd, proc in procs:
            _, err = proc.communicate()
            err = _filtered(err)
            if proc.returncode != 0:
                raise RuntimeError(f"hipcc failed ({proc.returncode}) on {cmd[-1]}:\n{err}")
            if verbose and err.strip():
                print(err)
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
        if verbose:
            print(" ".join(cmd))
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc link failed ({res.returncode}):\n{_filtered(res.stderr)}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
