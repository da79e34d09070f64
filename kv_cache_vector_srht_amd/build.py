"""Builds libtq.so (HIP kernels for gfx950 + host code) in-tree with hipcc,
and libtq_checked.so, the same sources with TQ_DEVICE_CHECKS=1 (the kernels
verify their index invariants as they run; tq_device_checks reads the result).

Packed FP32 instructions are disabled for the device code
(``-target-feature -packed-fp32-ops``): the kernels use plain FP32 VALU.
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libtq.so")
CHECKED_LIB = os.path.join(LIB_DIR, "libtq_checked.so")
ARCH = os.environ.get("TQ_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


SOURCES = ("tq_encode.hip", "tq_pages.hip", "tq_decode.hip", "tq_dequant.hip", "tq_host.cpp")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd))


def build(verbose: bool = False) -> str:
    """Compiles each source to an object (in parallel, release and checked),
    then links libtq.so and libtq_checked.so; returns libtq.so's path."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(LIB_DIR, exist_ok=True)
    chk_dir = os.path.join(LIB_DIR, "checked")
    os.makedirs(chk_dir, exist_ok=True)
    links, cmds = [], []
    for lib_path, obj_dir, extra in ((LIB, LIB_DIR, []), (CHECKED_LIB, chk_dir, ["-DTQ_DEVICE_CHECKS=1"])):
        objs = []
        for src in SOURCES:
            obj = os.path.join(obj_dir, src.replace(".", "_") + ".o")
            objs.append(obj)
            cmds.append([hipcc(), f"--offload-arch={ARCH}", *FLAGS, *extra, "-I", os.path.join(ROOT, "include"),
                         "-c", os.path.join(SRC, src), "-o", obj])
        links.append((lib_path, objs))
    with ThreadPoolExecutor(max_workers=min(len(cmds), max(1, os.cpu_count() or 1))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    for lib_path, objs in links:
        tmp = lib_path + ".tmp"
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, lib_path)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
