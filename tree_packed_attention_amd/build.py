"""Builds libtreeattn.so (all HIP kernels and the C ABI) for gfx950 in place.

    python tree_packed_attention_amd/build.py [-v]

Each source compiles to its own object in parallel, then one link. Extra
hipcc flags (build-time knobs such as -DTA_LA_DKDV=2) may be given in the
TREEATTN_HIPCC_FLAGS environment variable; TREEATTN_LIB names another output
file than the in-place libtreeattn.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shlex
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libtreeattn.so")
NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm install missing?)")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if NOISE not in l)
    return res.returncode, msgs


def build(verbose: bool = False) -> str:
    out = os.environ.get("TREEATTN_LIB") or LIB
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")) + glob.glob(os.path.join(HERE, "csrc", "*.cpp")))
    flags = [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-result",
        "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(HERE, "csrc"),
        *shlex.split(os.environ.get("TREEATTN_HIPCC_FLAGS", "")),
    ]
    with tempfile.TemporaryDirectory(prefix="treeattn_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(src) + ".o") for src in srcs]
        cmds = [[hipcc(), *flags, "-c", src, "-o", obj] for src, obj in zip(srcs, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with cf.ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1, 16)) as ex:
            results = list(ex.map(_run, cmds))
        errs = [m for rc, m in results if rc != 0]
        if errs:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
        if verbose:
            for rc, m in results:
                if m.strip():
                    print(m)
        tmp_lib = out + ".tmp"
        rc, msgs = _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_lib])
        if rc != 0:
            raise RuntimeError("link failed:\n" + msgs)
    os.replace(tmp_lib, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
