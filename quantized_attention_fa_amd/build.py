"""Build the gfx950 HIP libraries in-tree with hipcc.

    python -m quantized_attention_fa_amd.build

produces ``libfaquant.so`` (the product library: quantization + attention
kernels behind the C ABI of include/fa_quant.h) and ``libfaquant_probe.so``
(single-instruction probes used only by the test suite) next to this file.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
ARCH = os.environ.get("FAQ_OFFLOAD_ARCH", "gfx950")

LIB_SOURCES = ["api.hip", "quant.hip", "attention.hip", "static_ws.hip"]
PROBE_SOURCES = ["probe.hip"]
LIB = os.path.join(PKG, "libfaquant.so")
PROBE_LIB = os.path.join(PKG, "libfaquant_probe.so")

CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


# The attention kernels handle no NaN (codes are finite; masked scores are
# -inf): without NaN semantics max/min need no quieting of their inputs.
EXTRA = {"attention.hip": ["-fno-honor-nans"]}


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *CFLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    noise = ("packed-fp32-ops", "warning: unknown target feature", "generated.")
    warn = "\n".join(l for l in r.stderr.splitlines() if l.strip() and not any(n in l for n in noise))
    return obj, warn


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(out)} failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(_compile, LIB_SOURCES + PROBE_SOURCES))
    for (obj, warn), src in zip(results, LIB_SOURCES + PROBE_SOURCES):
        if warn and verbose:
            print(f"[build] {src}:\n{warn}", file=sys.stderr)
    objs = [o for o, _ in results]
    _link(objs[: len(LIB_SOURCES)], LIB)
    _link(objs[len(LIB_SOURCES):], PROBE_LIB)
    if verbose:
        print(f"[build] {LIB}\n[build] {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build()
