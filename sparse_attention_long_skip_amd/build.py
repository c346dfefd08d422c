"""Build libssa.so (the HIP kernels and the C ABI) in-tree for gfx950."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libssa.so")

SOURCES = ["ssa_api.cpp", "prefill.hip", "decode.hip", "mask.hip", "vslash.hip", "calibrate.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 instructions stay off: plain scalar fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
]

# Per-source extra flags. decode.hip: the split kernel takes a work ticket
# with one atomic add from lane 0 and reads the result a tile later; the
# compiler's atomic optimizer would rewrite it into a wave-aggregated add
# whose result is waited for at once.
EXTRA_FLAGS = {
    "decode.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
}


def build(verbose: bool = False, jobs: int = 4, lib_path: str = LIB, overrides: dict | None = None,
          objdir: str | None = None) -> str:
    """Compile every source to an object (in parallel) and link the library
    (libssa.so in the package by default). ``overrides`` maps a source name
    to another file to compile in its place. Always rebuilds. Returns the
    library path."""
    if not lib_path or os.path.isdir(lib_path):
        raise ValueError(f"lib_path must name the library file to write, got {lib_path!r}")
    lib_path = os.path.abspath(lib_path)
    overrides = overrides or {}
    objdir = objdir or os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        path = overrides.get(src, os.path.join(CSRC, src))
        cmd = [HIPCC, *FLAGS, *EXTRA_FLAGS.get(src, []), "-I", INCLUDE, "-I", CSRC, *lang, "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        if len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    failed = []
    for src, p in procs:
        log, _ = p.communicate()
        log = "\n".join(l for l in log.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((src, log))
        elif verbose and log.strip():
            print(log)
    if failed:
        msg = "\n".join(f"--- {s}\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = lib_path + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
