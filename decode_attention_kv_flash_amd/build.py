"""Compile the dattn HIP library in-tree for gfx950.

    python -m decode_attention_kv_flash_amd.build

Produces ``decode_attention_kv_flash_amd/libdattn.so`` from ``csrc/`` (object
files under ``_build/``).  DATTN_LIB_OUT / DATTN_BUILD_DIR redirect the output
and DATTN_EXTRA_CFLAGS adds compiler flags (for tuning builds).  Always recompiles: the result must match the
sources.  All HIP code is built with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.environ.get("DATTN_BUILD_DIR", os.path.join(PKG, "_build"))
LIB = os.environ.get("DATTN_LIB_OUT", os.path.join(PKG, "libdattn.so"))
SOURCES = ["api.cpp", "gqa_decode.hip", "mla_decode.hip", "indexer.hip", "topk.hip", "kv_append.hip", "quest.hip", "probe.hip"]
ARCH = os.environ.get("DATTN_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
    *os.environ.get("DATTN_EXTRA_CFLAGS", "").split(),
]


# Per-file device-code flags.  The MLA kernel keeps its output accumulator in
# AGPRs through inline assembly; its score MFMAs must then take VGPRs.
FILE_FLAGS = {
    "mla_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"]
        cmd = [HIPCC, *lang, *CFLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature flag: harmless
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if p.returncode != 0:
            failed.append(src)
            print("\n".join(lines), file=sys.stderr)
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
