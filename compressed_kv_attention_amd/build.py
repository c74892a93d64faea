"""Builds libada.so (the gfx950 HIP library) in place with hipcc.

    python -m compressed_kv_attention_amd.build
    python -m compressed_kv_attention_amd.build --phase-trace

The second builds libada_trace.so instead: the same sources with
ADA_PHASE_TRACE defined, whose page-stream kernel records per-wave phase
timestamps (ada_phase_trace), for profiling only.
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libada.so")
OUT_TRACE = os.path.join(PKG, "libada_trace.so")
BUILD = os.path.join(PKG, "_build")

SOURCES = ["ada_abi.cpp", "decode.hip", "encode.hip", "pack.hip", "rdr.hip", "append.hip"]

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # no packed-fp32 instructions (v_pk_*_f32) anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division and square root (the value quantiser divides)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-function",
]


def source_digest() -> str:
    """SHA-256 over the library's sources (every file under csrc/ and the
    public header), names and contents, in name order.  The build stamps it
    into the library (ada_build_id) so that a stale libada.so is refused at
    load time."""
    h = hashlib.sha256()
    files = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp", ".h")))
    paths = [os.path.join(CSRC, f) for f in files] + [os.path.join(ROOT, "include", "ada.h")]
    for path in paths:
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()


def build(verbose: bool = False, phase_trace: bool = False) -> str:
    bdir = os.path.join(BUILD, "trace") if phase_trace else BUILD
    out = OUT_TRACE if phase_trace else OUT
    os.makedirs(bdir, exist_ok=True)
    digest = source_digest()
    extra = ["-DADA_PHASE_TRACE"] if phase_trace else []

    def compile_one(src: str) -> str:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        cmd = ["hipcc", *FLAGS, *extra, f'-DADA_BUILD_ID="{digest}"', "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out + ".tmp"
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, phase_trace="--phase-trace" in sys.argv))
