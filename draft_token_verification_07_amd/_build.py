"""Build libspecverify.so (HIP, gfx950) in-tree, next to this file.

    python -m draft_token_verification_07_amd._build

Compiles every HIP source under csrc/ with hipcc for gfx950 only.  Packed
FP32 instructions are switched off for the device code (-packed-fp32-ops).
Extra -D flags (tuning sweeps) can be passed through SV_HIPCC_DEFS.
"""
from __future__ import annotations

import os
import shlex
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libspecverify.so")
SOURCES = ["sv_host.cpp", "sv_api.hip", "sv_greedy.hip", "sv_sample.hip", "sv_draft.hip", "sv_fanout.hip", "sv_trim.hip", "sv_lmhead.hip"]
HEADERS = ["sv_host.h", "sv_common.h", "sv_internal.h", "sv_rows.h"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(out: str = LIB, extra: list[str] | None = None, verbose: bool = False) -> str:
    defs = shlex.split(os.environ.get("SV_HIPCC_DEFS", ""))
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function",
           "-I", os.path.join(HERE, "..", "include")]
    cmd += defs + (extra or [])
    cmd += ["-o", out + ".tmp"] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(shlex.quote(c) for c in cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
