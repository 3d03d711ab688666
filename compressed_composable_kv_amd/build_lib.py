"""Build libc2kv.so (the C2KV C ABI + gfx950 HIP kernels) in-tree with hipcc.

    python -m compressed_composable_kv_amd.build_lib [--jobs N]

Compiles every source under csrc/ for --offload-arch=gfx950 and links the
shared library next to this file.  Also builds libc2kv_probe.so from probe/,
measurement tools the benchmark loads (the achievable MFMA and HBM read
rates); the library does not use them.  Always rebuilds.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libc2kv.so")
PROBE_SRCS = [os.path.join(PKG, "probe", "mfma_peak.hip"), os.path.join(PKG, "probe", "hbm_read.hip")]
PROBE_LIB = os.path.join(PKG, "libc2kv_probe.so")

SOURCES = ["c2kv_attn.hip", "c2kv_decode.hip", "c2kv_aux.hip", "c2kv_layer.hip", "c2kv_abi.cpp", "c2kv_cache.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    # packed fp32 VALU forms stay disabled on this path
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    t = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if warn:
        print(f"[build] {src} warnings:\n{warn}", file=sys.stderr)
    print(f"[build] {src} {time.time() - t:.1f}s", file=sys.stderr)
    return obj


def build(jobs: int = 4) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
           "-Wl,-rpath,/opt/rocm/lib", "-Wl,--no-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    build_probe()
    return LIB


def build_probe() -> str:
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *[f for f in CFLAGS if not f.startswith("-I")], "-shared", "-o", tmp, *PROBE_SRCS,
           "-Wl,-rpath,/opt/rocm/lib", "-Wl,--no-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--clean", action="store_true")
    a = ap.parse_args()
    if a.clean and os.path.isdir(BUILD):
        shutil.rmtree(BUILD)
    print(build(a.jobs))


if __name__ == "__main__":
    main()
