"""Build libkda.so (the gfx950 HIP library behind include/kda.h) in-tree with hipcc."""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("kda_api.hip", "kda_intra.hip", "kda_inter.hip", "kda_kcp.hip", "kda_decode.hip", "kda_bwd.hip")]
LIB = os.path.join(HERE, "libkda.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # keep the compiler from forming packed fp32 (v_pk_*_f32) arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(extra_flags=(), out=LIB) -> str:
    """Compile every HIP source into ``out`` and return its path."""
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra_flags, *SOURCES, "-o", tmp]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + proc.stdout + proc.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
