"""Build libkda.so in-tree with hipcc for gfx950 (no GPU needed)."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkda.so")
SOURCES = ["kda_api.hip", "kda_prep.hip", "kda_state.hip", "kda_fused.hip", "kda_segment.hip", "kda_decode.hip",
           "kda_attn.hip", "kda_bwd.hip", "kda_bwd_bf16.hip", "kda_bwd_tok.hip"]
HEADERS = ["kda_device.hpp", "kda_internal.hpp", "kda_solve.hpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    # Packed fp32 instructions stay off: the compiler would otherwise form them
    # from plain float code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build_library(force: bool = True, verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    deps = srcs + [os.path.join(CSRC, h) for h in HEADERS] + [
        os.path.join(os.path.dirname(PKG), "include", "kda.h")]
    if not force and os.path.exists(LIB) and all(os.path.getmtime(LIB) >= os.path.getmtime(d)
                                                 for d in deps):
        return LIB
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + ["-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-8000:]}")
    # hipcc's host pass warns about the packed-fp32 feature it does not know; anything else is shown.
    other = [ln for ln in res.stderr.splitlines() if ln.strip() and "packed-fp32-ops" not in ln]
    if other and verbose:
        print("\n".join(other[-50:]))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(force=True, verbose=True))
