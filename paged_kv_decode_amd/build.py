"""Build libpa_decode.so (gfx950) in-tree with hipcc.

Run as ``python -m paged_kv_decode_amd.build``.  The library is written next to
this file so it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libpa_decode.so")
SOURCES = [
    os.path.join(HERE, "csrc", "pa_decode_kernels.hip"),
    os.path.join(HERE, "csrc", "pa_decode_balanced.hip"),
    os.path.join(HERE, "csrc", "pa_decode_api.cpp"),
    os.path.join(HERE, "csrc", "planner.cpp"),
    os.path.join(HERE, "csrc", "validate.cpp"),
    os.path.join(HERE, "csrc", "pa_decode_scratch.hip"),
]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # Packed fp32 VALU ops stay off: the compiler emits plain fp32 ops.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the decode loop rescales them on the
    # vector ALUs, which cannot touch AGPRs (AGPR accumulators cost two moves
    # per element per rescale).
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I" + os.path.join(ROOT, "include"),
    "-I" + os.path.join(HERE, "csrc"),
]


def build(verbose: bool = False) -> str:
    """Compile the library (always recompiles) and return its path.

    Each source compiles to an object in its own hipcc process (all at
    once: the two kernel translation units dominate), then one link."""
    tag = ".tmp%d" % os.getpid()
    objs = [os.path.join(tempfile.gettempdir(), os.path.basename(src) + tag + ".o")
            for src in SOURCES]
    cmds = [[HIPCC] + FLAGS + ["-c", src, "-o", obj] for src, obj in zip(SOURCES, objs)]
    try:
        procs = []
        for cmd in cmds:
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                          text=True))
        failed = False
        for p in procs:
            out, _ = p.communicate()
            if p.returncode != 0:
                sys.stderr.write(out)
                failed = True
        if failed:
            raise RuntimeError("hipcc failed building libpa_decode.so")
        tmp = LIB_PATH + tag
        link = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        res = subprocess.run(link, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError("hipcc failed linking libpa_decode.so")
        os.replace(tmp, LIB_PATH)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
