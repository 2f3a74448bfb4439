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


# Comparison builds (measurement only, never loaded by the package itself):
# name -> (library file, extra defines).  qk_valu: the scores on the vector
# ALUs (packed dot products, lane-swap sums) instead of the score MFMA.
# fused_merge: no merge kernel for fixed partitions; the last workgroup of a
# (sequence, KV head) merges its states.
VARIANTS = {"qk_valu": ("libpa_decode_qk_valu.so", ["-DPA_QK_VALU=1"]),
            "fused_merge": ("libpa_decode_fused_merge.so", ["-DPA_FUSED_MERGE=1"])}


def build(verbose: bool = False, variant: str = None) -> str:
    """Compile the library (always recompiles) and return its path.

    Each source compiles to an object in its own hipcc process (all at
    once: the two kernel translation units dominate), then one link.
    variant: a key of VARIANTS, for a comparison build written next to the
    library under its own name."""
    lib_path = LIB_PATH
    extra = []
    if variant is not None:
        name, extra = VARIANTS[variant]
        lib_path = os.path.join(HERE, name)
    tag = ".tmp%d" % os.getpid() + ("." + variant if variant else "")
    objs = [os.path.join(tempfile.gettempdir(), os.path.basename(src) + tag + ".o")
            for src in SOURCES]
    cmds = [[HIPCC] + FLAGS + extra + ["-c", src, "-o", obj] for src, obj in zip(SOURCES, objs)]
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
        tmp = lib_path + tag
        link = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        res = subprocess.run(link, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError("hipcc failed linking libpa_decode.so")
        os.replace(tmp, lib_path)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    return lib_path


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="build libpa_decode.so for gfx950")
    ap.add_argument("--variant", choices=sorted(VARIANTS), default=None,
                    help="a comparison build (measurement only)")
    print(build(verbose=True, variant=ap.parse_args().variant))
