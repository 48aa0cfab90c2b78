"""Build the HIP decode library for gfx950 in-tree: csrc/* -> libkvdecode.so.

Usage:  python kv_cache_decode_02_amd/build.py  [--jobs N] [--save-temps]

(Run it as a script: importing the package would load the library it builds.)

Every source is compiled with hipcc for gfx950 only.  Packed fp32 vector
instructions are disabled for the device code (``-packed-fp32-ops``).
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libkvdecode.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["api.cpp", "block_pool.cpp", "validate.cpp", "append.hip", "decode_paged.hip", "decode_merge.hip",
           "decode_mla.hip", "prefill_paged.hip", "scratch.hip",
           "stream_read.hip", "lds_read.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"-I{os.path.join(ROOT, 'include')}"]
DEVICE = [f"--offload-arch={ARCH}", "-x", "hip",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


def _compile(src, obj, save_temps):
    cmd = [_hipcc()] + COMMON
    if src.endswith(".hip"):
        cmd += DEVICE
        if save_temps:
            cmd += ["-save-temps=obj"]
    else:
        cmd += ["-D__HIP_PLATFORM_AMD__"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return res.stderr


def build(jobs=None, save_temps=False, verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, s, o, save_temps) for s, o in zip(SOURCES, objs)]
        for f in futs:
            warn = f.result()
            if verbose and warn.strip():
                print(warn, file=sys.stderr)
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--save-temps", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(args.jobs, args.save_temps, args.verbose))


if __name__ == "__main__":
    main()
