"""Compile the HIP sources into libgemma_attn.so for gfx950 (in-tree).

    python -m global_gqa_rope_amd.build [--jobs N] [--verbose]

hipcc cross-compiles without a GPU.  Packed fp32 VALU ops are disabled for
every device pass.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB_NAME = "libgemma_attn.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["api.hip", "prep.hip", "prefill.hip", "decode.hip", "calibrate.hip"]
ARCH = "gfx950"
# Per-source device flags.  MFMAs in VGPR form: the decode kernel keeps its
# 128 fp32 output accumulators in VGPRs and rescales them with VALU ops; the
# prefill kernel keeps its QK^T scores in VGPRs, and its output accumulators
# in AGPRs through MFMAs written out with AGPR operands.  Either way nothing is
# copied between the two register files every tile.
SOURCE_FLAGS = {"decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")
    return path


def common_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


def build(jobs: int = 8, verbose: bool = False, extra: list[str] | None = None) -> str:
    cc = hipcc()
    extra = extra or []
    tmp = tempfile.mkdtemp(prefix="gemma_attn_build_")
    try:
        def compile_one(src: str) -> str:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [cc, *common_flags(), *SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
            if verbose and res.stderr.strip():
                print(res.stderr, file=sys.stderr)
            return obj

        with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        out_tmp = LIB_PATH + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
        os.replace(out_tmp, LIB_PATH)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB_PATH


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    main()
