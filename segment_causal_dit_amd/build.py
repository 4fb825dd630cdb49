"""Build libsegcausal.so (gfx950) in-tree with hipcc.

Usage: python -m segment_causal_dit_amd.build   (or build() from Python)
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsegcausal.so")
SOURCES = ["api.cpp", "rope.hip", "append.hip", "dequant.hip", "attn.hip", "attn_bwd.hip", "gemm_w8.hip",
           "camera.hip", "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wextra", "-Werror", "-Wno-unused-function",
    # packed fp32 arithmetic stays off: code generation must not emit it
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose=False, extra=(), out=LIB):
    """Compile every HIP source into `out` (by default
    segment_causal_dit_amd/libsegcausal.so); `extra` flags follow the standard
    ones."""
    tmp = out + ".tmp"
    cmd = [HIPCC] + FLAGS + list(extra) + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
