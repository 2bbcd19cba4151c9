"""Compile the HIP sources into ``libring_attn.so`` next to this file (gfx950),
and the measurement aid ``mfma_stream.hip`` into ``libmfma_stream.so`` (a
separate library: it is no part of the attention ABI)."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libring_attn.so")
SOURCES = ["api.cpp", "partition.hip", "fwd_f32.hip", "fwd_bf16.hip", "merge.hip", "decode.hip", "noalloc.hip"]
STREAM_LIB = os.path.join(HERE, "libmfma_stream.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-Wno-unused-command-line-argument",
]


def _compile(src: str, obj: str, extra: list) -> None:
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")


def build(out: str = LIB, extra: list | None = None, verbose: bool = False) -> str:
    extra = list(extra or [])
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        futs = [ex.submit(_compile, s, o, extra) for s, o in zip(SOURCES, objs)]
        for f in futs:
            f.result()
    tmp = out + ".tmp"
    # --no-undefined: a missing kernel launch stub must fail the build, not the load.
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def build_stream(out: str = STREAM_LIB, verbose: bool = False) -> str:
    """The matrix-core stream used by bench.py --power."""
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, "-shared", "-Wl,--no-undefined", os.path.join(CSRC, "mfma_stream.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for mfma_stream.hip:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(extra=sys.argv[1:], verbose=True)
    build_stream(verbose=True)
