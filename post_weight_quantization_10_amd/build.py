"""Build the gfx950 shared library (libgptq_mi355x.so) in-tree with hipcc, and
the measurement probe (libgptq_peaks.so, csrc/probe/) beside it.

Usage:  python -m post_weight_quantization_10_amd.build   (or build() from Python)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libgptq_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
PROBE_SRC = os.path.join(CSRC, "probe", "peaks.hip")
PROBE_PATH = os.path.join(HERE, "libgptq_peaks.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are kept out of the device code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    if src == PROBE_SRC:
        obj = os.path.join(BUILD_DIR, "probe_" + os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max(1, min(len(srcs) + 1, os.cpu_count() or 1))) as ex:
        objs = list(ex.map(_compile, srcs + [PROBE_SRC]))
    for out, parts in ((LIB_PATH, objs[:-1]), (PROBE_PATH, objs[-1:])):
        tmp = out + ".tmp"
        cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *parts, "-o", tmp]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}")
        os.replace(tmp, out)
        if verbose:
            print(f"built {out}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
