"""Build libmla.so in-tree with hipcc for gfx950 (cross-compiles without a GPU).

    python -m mla_latent_kv_40_amd.build [--save-temps DIR]
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["libmla.cpp", "append.hip", "absorb.hip", "decode.hip"]
LIB = os.path.join(HERE, "libmla.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 ops stay off: the compiler is told not to form v_pk_{add,mul,fma}_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]
# Per-source extras.  The MFMA builtins select their VGPR form (accumulators in VGPRs); the
# decode kernel places its output tiles in the accumulation registers itself.
EXTRA = {
    "append.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "absorb.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "libmla.cpp": [],
}


def _run(cmd, cwd=None, verbose=False, remarks=False):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}")
    if verbose or remarks:
        sys.stderr.write(r.stderr)


def build(verbose: bool = False, save_temps: str | None = None) -> str:
    """Compile every source to an object (own flags) and link libmla.so; always recompiles."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmd = [HIPCC, *FLAGS, *EXTRA[src], "-c", os.path.join(CSRC, src), "-o", obj]
        if save_temps:
            cmd.insert(1, "-save-temps=cwd")
            cmd += ["-Rpass-analysis=kernel-resource-usage"]
        _run(cmd, cwd=save_temps, verbose=verbose, remarks=bool(save_temps))
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose=verbose)
    os.replace(tmp, LIB)
    return LIB


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--save-temps", default=None, help="keep intermediate files (ISA) in this folder")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(verbose=a.verbose, save_temps=a.save_temps))


if __name__ == "__main__":
    main()
