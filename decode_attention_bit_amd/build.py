"""Compile libuq.so for gfx950 in-tree with hipcc (no JIT cache)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["uq_store.hip", "uq_decode.hip", "uq_prefill.hip", "uq_probe.hip", "uq_api.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-FP32 instructions anywhere in the library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False) -> str:
    out = os.path.join(HERE, "libuq.so")
    tmp = out + ".tmp"
    cmd = ["hipcc", *FLAGS, "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libuq.so")
    if verbose:
        sys.stderr.write(r.stderr)
    # every symbol must resolve (a kernel whose host stub was not emitted
    # links but does not load); checked in a child so no handle stays open
    chk = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({tmp!r})"],
                         capture_output=True, text=True)
    if chk.returncode != 0:
        os.remove(tmp)
        sys.stderr.write(chk.stderr)
        raise RuntimeError("libuq.so built but does not load")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
