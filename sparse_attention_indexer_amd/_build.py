"""Compile libdsa.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdsa.so")
SOURCES = ["api.hip", "indexer.hip", "topk.hip", "mla.hip", "proj.hip", "prep.hip", "mha.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdsa.so)")


def command(out: str = LIB, extra=()) -> list:
    return [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-fvisibility=hidden",
            # keep the compiler from emitting packed fp32 math (v_pk_*_f32)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA results in ordinary VGPRs rather than accumulation registers:
            # the epilogues that read them (the indexer's ReLU and head sum) then
            # need no v_accvgpr_read per element (8192-query prefill indexer
            # 501 -> 475 us; no kernel spills either way)
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *extra, *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


def build(out: str = LIB, verbose: bool = False) -> str:
    tmp = out + ".tmp"
    res = subprocess.run(command(tmp), capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
