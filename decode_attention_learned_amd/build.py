"""Build libdms.so in-tree with hipcc for gfx950.

    python -m decode_attention_learned_amd.build

Every call recompiles.  The libraries land next to this file, where
``decode_attention_learned_amd.lib`` looks for them: ``libdms.so`` (the
product) and ``libdms_generic.so``, a test build of the same sources whose
one-query decode of bf16 caches runs the vector kernel (decode_mfma.hip
compiled with DMS_DECODE_BF16_GENERIC), against which tests check the
matrix-core kernel.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libdms.so")
LIB_GENERIC = os.path.join(HERE, "libdms_generic.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "cache_kernels.hip", "decode_f32.hip", "decode_kernels.hip", "decode_mfma.hip",
           "decode_scratch.hip", "prefill.hip", "prefill_f32.hip"]

# Packed fp32 instructions are switched off for all device code; hipcc's host
# pass warns that it does not know the feature, which is harmless.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", "-Wno-pass-failed",
]


# The attention kernels mask with -inf and never rely on NaN semantics; without
# NaN honouring the compiler drops the NaN-quieting copies before every max.
PER_FILE_FLAGS = {
    "decode_f32.hip": ["-fno-honor-nans"],
    "decode_mfma.hip": ["-fno-honor-nans"],
    "prefill.hip": ["-fno-honor-nans"],
}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


# the test build differs in one object
GENERIC_VARIANT = ("decode_mfma.hip", ["-DDMS_DECODE_BF16_GENERIC"])


def build(verbose: bool = False) -> str:
    objs = []
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    procs = []
    jobs = [(src, os.path.join(build_dir, src.replace(".hip", ".o")), []) for src in SOURCES]
    gsrc, gflags = GENERIC_VARIANT
    gobj = os.path.join(build_dir, gsrc.replace(".hip", "_generic.o"))
    jobs.append((gsrc, gobj, gflags))
    for src, obj, extra in jobs:
        cmd = [hipcc(), *[f for f in FLAGS if f != "-shared"], *PER_FILE_FLAGS.get(src, []), *extra,
               "-c", "-I", INCLUDE, "-I", CSRC, os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if not extra:
            objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        errors = [ln for ln in text.splitlines() if "error" in ln]
        if p.returncode != 0:
            failed.append((src, text))
        elif verbose and errors:
            print(text)
    if failed:
        for src, text in failed:
            sys.stderr.write(f"--- {src}\n{text}\n")
        raise RuntimeError("hipcc failed for " + ", ".join(s for s, _ in failed))
    gobjs = [gobj if o.endswith(gsrc.replace(".hip", ".o")) else o for o in objs]
    for lib, members in ((LIB, objs), (LIB_GENERIC, gobjs)):
        tmp = lib + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *members, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
