"""Build libsdpa_bwd.so for gfx950 in-tree with hipcc.

    python -m sdpa_backward_fa2_amd.build        # or build() from Python

Every HIP source under csrc/ is compiled into one shared library next to this
file.  Packed fp32 instructions are disabled for device code
(``-packed-fp32-ops``); hipcc's host pass warns that it does not know that
feature, which is harmless.  Matrix-core results are allocated in ordinary
vector registers (``-amdgpu-mfma-vgpr-form``): the score tiles feed vector-ALU
code right after their products, and with accumulation registers the compiler
copies every element across (about 130 copies per step of the D=128 dK/dV
kernel); the dK/dV accumulators still land in accumulation registers when the
vector file is full.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsdpa_bwd.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


# Machine-scheduler strategy per source file, chosen by measurement on
# MI355X: the D=128 kernels (bwd128.hip) ran 3 % faster with iterative-ilp and
# the selected-attention kernels (nsa.hip) 2 % faster with max-memory-clause;
# the D=64 kernel (bwd.hip) was fastest with the default.  The D=192 kernels
# (bwd192.hip, at 512 registers) take the default: iterative-ilp crashes the
# compiler on them.  The selected-attention dK/dV kernel (nsa_kv.hip) also
# uses the AMDGPU register-pressure trackers, which took it 3 % faster and the
# selected dQ pass 4 % slower.
FILE_FLAGS = {
    "bwd128.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
    "nsa.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"],
    "nsa_kv.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause", "-mllvm", "-amdgpu-use-amdgpu-trackers"],
}


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every HIP source in parallel, then link the shared library."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    flags = [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Wno-unused-result", "-Wno-unused-command-line-argument",
    ] + list(extra or [])
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC, *flags, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write("\n".join(lines) + "\n")
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError(f"hipcc failed for: {', '.join(os.path.basename(f) for f in failed)}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
