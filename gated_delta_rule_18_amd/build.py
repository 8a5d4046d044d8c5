"""Build libkla.so for gfx950, in-tree, with hipcc.

Every HIP source under csrc/ is compiled for gfx950 only, with packed-fp32 VALU
instructions turned off, and linked into gated_delta_rule_18_amd/libkla.so.
Objects go to <repo>/_build/. Run as ``python -m gated_delta_rule_18_amd.build``.
"""
from __future__ import annotations

import os
import pathlib
import shutil
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libkla.so"
SOURCES = ["kla_abi.hip", "device_info.hip", "decode.hip", "prepare_beta.hip", "chunk_prep.hip", "chunk_scan.hip",
           "chunk_seg.hip", "chunk_bwd_scan.hip", "chunk_bwd_grad.hip", "chunk_bwd_grad_kda.hip",
           "chunk_bwd_grad_f32.hip"]
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", str(ROOT / "include"), "-I", str(CSRC),
    "-Wno-unused-command-line-argument",
]
# Per-source extra flags. The scan kernels keep their MFMA accumulators in ordinary VGPRs (the
# default places them in AGPRs and copies every value the VALU touches).
EXTRA = {"chunk_scan.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "chunk_bwd_scan.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose: bool = False) -> pathlib.Path:
    objdir = ROOT / "_build"
    objdir.mkdir(exist_ok=True)
    procs = []
    for src in SOURCES:
        obj = objdir / (src.rsplit(".", 1)[0] + ".o")
        cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", str(CSRC / src), "-o", str(obj)]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    objs, errors = [], []
    for src, obj, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            errors.append(f"--- {src} ---\n{out}")
        elif verbose and out.strip():
            print(out)
        objs.append(str(obj))
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", str(tmp)]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
