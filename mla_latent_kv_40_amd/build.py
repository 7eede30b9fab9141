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
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 ops stay off: the compiler is told not to form v_pk_{add,mul,fma}_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # select the VGPR form of MFMA: accumulators stay in VGPRs and the accumulation register
    # file is only spill space (otherwise the decode kernel shuttles its whole output tile
    # between the two register files around its rarely-taken rescale branch every page)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, save_temps: str | None = None) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd.insert(1, "-save-temps=cwd")
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    if verbose:
        print(" ".join(cmd), flush=True)
    cwd = save_temps if save_temps else None
    if save_temps:
        cmd[cmd.index("-o") + 1] = os.path.abspath(tmp)
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode})")
    if verbose or save_temps:
        sys.stderr.write(r.stderr)
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
