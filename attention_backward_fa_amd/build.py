"""Compile ``libfa_bwd.so`` in place with hipcc for gfx950.

    python -m attention_backward_fa_amd.build

Three translation units, compiled in parallel and linked into one library that
lands next to this file, where the binding looks for it:
  fa_bwd.hip       the C ABI and the kernels for head dims up to 128, with MFMA
                   accumulators in VGPRs (two waves per SIMD, 256 registers each);
  fa_bwd_wide.hip, fa_bwd_wide192.hip
                   the kernels for head dims above 128 (one wave per SIMD), whose
                   accumulators need the AGPRs as well.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libfa_bwd.so")
CSRC = os.path.join(HERE, "csrc")
# (source, extra flags)
UNITS = [
    ("fa_bwd.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form"]),  # the softmax reads S and dP without AGPR copies
    ("fa_bwd_wide.hip", []),
    ("fa_bwd_wide192.hip", []),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa_bwd.so)")


def compile_command(src: str, extra: list, obj: str) -> list:
    return [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-c",
            # packed fp32 VALU forms are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-munsafe-fp-atomics", "-Wno-unused-result",
            *extra,
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            os.path.join(CSRC, src), "-o", obj]


def link_command(objs: list, out: str) -> list:
    return [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out]


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="fa_bwd_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(src)[0] + ".o") for src, _ in UNITS]
        cmds = [compile_command(src, extra, obj) for (src, extra), obj in zip(UNITS, objs)]
        procs = []
        for cmd in cmds:
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
        errors = []
        for cmd, p in zip(cmds, procs):
            _, err = p.communicate()
            if p.returncode != 0:
                errors.append(f"hipcc failed ({p.returncode}) on {cmd[-3]}:\n{err[-4000:]}")
        if errors:
            raise RuntimeError("\n".join(errors))
        tmp = LIB + ".tmp"
        cmd = link_command(objs, tmp)
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed ({res.returncode}):\n{res.stderr[-4000:]}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
