"""Build libkda.so (the gfx950 HIP library behind include/kda.h) in-tree with hipcc."""

import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("kda_api.hip", "kda_intra.hip", "kda_inter.hip", "kda_kcp.hip", "kda_decode.hip", "kda_bwd.hip",
                                                     "kda_bwd_grad.hip", "kda_noalloc.hip", "kda_chain.hip")]
LIB = os.path.join(HERE, "libkda.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # keep the compiler from forming packed fp32 (v_pk_*_f32) arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# Per-source flags.  The two recurrence kernels (forward inter-chunk, backward
# state gradient) keep their MFMA accumulators in arch VGPRs, where the VALU
# scales and converts them without accumulator-register moves; their operand
# prefetch sets, which only feed MFMAs, then go to the accumulator registers.
SOURCE_FLAGS = {"kda_inter.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "kda_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(extra_flags=(), out=LIB, sources=None) -> str:
    """Compile every HIP source (in parallel, one object each) and link them
    into ``out``; return its path."""
    sources = list(sources or SOURCES)
    with tempfile.TemporaryDirectory(prefix="kda_build_") as tmpdir:
        procs = []
        for src in sources:
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []), *extra_flags, "-c", src, "-o", obj]
            procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        errors = []
        for src, _, p in procs:
            so, se = p.communicate()
            if p.returncode != 0:
                errors.append(f"{src}:\n{so}{se}")
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
        tmp = out + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for _, o, _ in procs], "-o", tmp]
        proc = subprocess.run(cmd, capture_output=True, text=True)
        if proc.returncode != 0:
            raise RuntimeError("hipcc link failed:\n" + proc.stdout + proc.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
