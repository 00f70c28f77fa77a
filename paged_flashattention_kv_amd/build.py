"""Build libpagedattn.so for gfx950 in-tree with hipcc.

    python -m paged_flashattention_kv_amd.build

Every source is compiled on each call (objects under ``_build/``), then
linked into ``paged_flashattention_kv_amd/libpagedattn.so``. Device code is
built with packed-fp32 instructions disabled.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libpagedattn.so")

SOURCES = ["pa_plan.cpp", "paged_attention.cpp", "pa_decode.hip", "pa_prefill.hip", "pa_append.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    path = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError(f"hipcc not found at {path}")
    return path


def common_flags():
    return [
        "-O3",
        "-std=c++17",
        "-fPIC",
        f"--offload-arch={ARCH}",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall",
        "-Wno-unused-function",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; return its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        objs.append(obj)
        cmd = [cc, *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd.insert(1, "-xhip")
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, cmd, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature; that note is harmless
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text)
    if failed:
        msg = "\n".join(f"--- {s} ---\n{t}" for s, t in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    fd, tmp = tempfile.mkstemp(prefix="libpagedattn.", suffix=".so.tmp", dir=HERE)
    os.close(fd)
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        os.unlink(tmp)
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
