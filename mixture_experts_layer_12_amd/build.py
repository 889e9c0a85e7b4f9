"""Build libmoe.so for gfx950 with hipcc (in-tree, into ``lib/``)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["csrc/api.cpp", "csrc/router.hip", "csrc/decode.hip", "csrc/decode_fused.hip", "csrc/sparse.hip",
           "csrc/prefill.hip", "csrc/probe.hip", "csrc/noalloc.hip", "csrc/cache.cpp"]
HEADERS = ["csrc/common.hpp", "csrc/router_items.hpp", "csrc/decode_items.hpp", "../include/moe.h",
           "../include/moe_probe.h"]
OUT = os.path.join(HERE, "lib", "libmoe.so")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise FileNotFoundError("hipcc not found")


FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-munsafe-fp-atomics",
         # no implicit multiply-add contraction: whether a product and a sum fuse would otherwise
         # depend on how a work item was inlined, and the single- and multi-launch decodes, which
         # share the items, must produce the same bits (explicit fmaf calls are unaffected)
         "-ffp-contract=off",
         # packed fp32 ops are kept out of the generated code on purpose
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def compile_command(src: str, obj: str) -> list:
    return [hipcc(), *FLAGS, "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(HERE, "csrc"),
            "-c", os.path.join(HERE, src), "-o", obj]


def _check(r, what):
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {what} ({r.returncode}):\n{err}")
    return err


def build(verbose: bool = True) -> str:
    """Compile every source (in parallel) and link lib/libmoe.so; always rebuilds."""
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    tmp = OUT + ".tmp"
    with tempfile.TemporaryDirectory(prefix="moe_build_") as d:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(d, os.path.basename(src) + ".o")
            cmd = compile_command(src, obj)
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
            objs.append(obj)
        warnings = []
        for src, p in procs:
            out, err = p.communicate()
            warnings.append(_check(subprocess.CompletedProcess(p.args, p.returncode, out, err), src))
        link = [hipcc(), "--offload-arch=gfx950", "-fPIC", "-shared", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        warnings.append(_check(subprocess.run(link, capture_output=True, text=True), "link"))
    text = "\n".join(w for w in warnings if w.strip())
    if text.strip() and verbose:
        print(text, file=sys.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    build()
