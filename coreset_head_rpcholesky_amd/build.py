"""Build the WildCat HIP library (libwc.so) in-tree for gfx950.

    python -m coreset_head_rpcholesky_amd.build

Each source under csrc/ is compiled with hipcc to an object in _build/, then linked into
coreset_head_rpcholesky_amd/libwc.so next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libwc.so")
LIB_DEBUG = os.path.join(HERE, "libwc_debug.so")
ARCH = os.environ.get("WC_OFFLOAD_ARCH", "gfx950")

# (source, object name, extra defines): the resident kernel is built once per (d, dv).
SOURCES = [("wc_api.cpp", "wc_api", []), ("wc_stream.hip", "wc_stream", []),
           ("wc_weights.hip", "wc_weights", []), ("wc_union.hip", "wc_union", []),
           ("wc_center.hip", "wc_center", []), ("wc_noalloc.hip", "wc_noalloc", []),
           ("wc_attend.hip", "wc_attend", []), ("wc_calibrate.hip", "wc_calibrate", [])] + [
    ("wc_resident.hip", f"wc_resident_{d}_{dv}", [f"-DWC_RES_D={d}", f"-DWC_RES_DV={dv}"])
    for d in (64, 128) for dv in (64, 128)]

# the objects with WC_DEBUG index checks (the kernels that read caller-supplied pivot indices)
DEBUG_CHECKED = ("wc_attend", "wc_union", "wc_weights")

# Packed fp32 instructions stay off: the compiler would otherwise emit v_pk_* fp32 ops.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
          "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the WildCat library)")


def _compile(spec, verbose: bool) -> str:
    src, name, defs = spec
    obj = os.path.join(BUILD, name + ".o")
    cmd = [hipcc(), "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj] + COMMON + DEVICE_FLAGS + defs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    noise = "is not a recognized feature for this target"
    errs = [ln for ln in res.stderr.splitlines() if ln.strip() and noise not in ln]
    if verbose and errs:
        print("\n".join(errs), file=sys.stderr)
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)


def build(verbose: bool = False, debug: bool = True) -> str:
    """Build libwc.so and, unless debug is False, libwc_debug.so: the same library with the
    sources that read pivot indices from device memory compiled with WC_DEBUG=1 (those
    indices are checked before use and reported through WC_FLAG_BOUNDS)."""
    os.makedirs(BUILD, exist_ok=True)
    specs = list(SOURCES)
    if debug:
        specs += [(src, name + "_debug", defs + ["-DWC_DEBUG=1"]) for src, name, defs in SOURCES
                  if name in DEBUG_CHECKED]
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        objs = dict(zip([s[1] for s in specs], ex.map(lambda s: _compile(s, verbose), specs)))
    _link([objs[name] for _, name, _ in SOURCES], LIB, verbose)
    if debug:
        _link([objs[name + "_debug" if name in DEBUG_CHECKED else name] for _, name, _ in SOURCES],
              LIB_DEBUG, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
