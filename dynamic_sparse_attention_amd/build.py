"""Build libvs.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage: python -m dynamic_sparse_attention_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libvs.so")
SOURCES = ["vs_api.cpp", "vs_fwd.hip", "vs_bwd.hip", "vs_bwd_kv.hip", "vs_bwd_dq.hip", "vs_estimate.hip", "vs_misc.hip", "vs_moba.hip",
           "vs_xattn.hip"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def flags(arch: str = "gfx950"):
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={arch}",
            # packed fp32 VALU ops stay off: only scalar/vector fp32 code is generated
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-result", "-munsafe-fp-atomics"]


# Per-source extra flags.  The attention kernels keep their matrix-core
# accumulators in the VGPR file: the softmax works on the score tiles with
# vector ALU instructions right after the products, and with AGPR results the
# compiler copied whole tiles back and forth on every iteration (measured
# slower for all three).
EXTRA = {"vs_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "vs_bwd_kv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "vs_bwd_dq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source for gfx950 and link libvs.so next to this file."""
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="vs_build_")
    try:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            lang = ["-x", "hip"] if src.endswith(".cpp") else []
            cmd = [cc, *flags(), *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
            if len(procs) >= jobs:
                _wait(procs.pop(0))
        for pr in procs:
            _wait(pr)
        out_tmp = LIB + ".tmp"
        cmd = [cc, *flags(), "-shared", *objs, "-o", out_tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(out_tmp, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


def _wait(pr):
    src, p = pr
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{text}")
    warn = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if warn:
        sys.stderr.write(f"[{src}]\n" + "\n".join(warn) + "\n")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
