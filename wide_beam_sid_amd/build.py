"""Build libgr.so (host C++ and gfx950 HIP kernels) in-tree with hipcc.

Each source compiles to its own object in parallel (objects under
wide_beam_sid_amd/_build/), then one hipcc link step makes libgr.so.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgr.so")
SOURCES = ["gr_host.cpp", "post.cpp", "cross_attn.hip", "self_attn.hip", "constrain.hip"]
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    f"--offload-arch={ARCH}",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-pthread",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    return r.returncode, r.stdout + r.stderr


def build(verbose: bool = False) -> str:
    """Compile every source into wide_beam_sid_amd/libgr.so (always rebuilds)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJ, exist_ok=True)
    objs = [os.path.join(OBJ, s + ".o") for s in SOURCES]
    # host-only sources need no device pass
    cmds = []
    for s, o in zip(SOURCES, objs):
        lang = [] if s.endswith(".hip") else ["-x", "hip"]
        cmds.append([hipcc, *FLAGS, *lang, "-c", os.path.join(CSRC, s), "-o", o])
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        results = list(ex.map(_run, cmds))
    for (rc, out), cmd in zip(results, cmds):
        if rc != 0:
            sys.stderr.write(" ".join(cmd) + "\n" + out)
            raise RuntimeError("hipcc failed building libgr.so")
        if verbose and out:
            sys.stderr.write(out)
    tmp = LIB + ".tmp"
    rc, out = _run([hipcc, *FLAGS, "-shared", *objs, "-o", tmp])
    if rc != 0:
        sys.stderr.write(out)
        raise RuntimeError("hipcc failed linking libgr.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
