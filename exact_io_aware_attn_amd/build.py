"""Build libmiattn.so for gfx950 with hipcc (in-tree, next to this file).

    python -m exact_io_aware_attn_amd.build [--jobs N]

Each attention source under csrc/ is compiled to an object in _build/ (in
parallel), then linked into exact_io_aware_attn_amd/libmiattn.so; the engine
clock probe (csrc/clock_probe.hip, include/miclock.h) becomes
exact_io_aware_attn_amd/libmiclock.so. Always rebuilds.
"""

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmiattn.so")
SOURCES = ["api.cpp", "fwd_bf16.hip", "fwd_f32.hip", "kstats.hip", "decode.hip", "segments.hip", "bwd_bf16.hip"]
CLOCK_LIB = os.path.join(PKG, "libmiclock.so")
CLOCK_SOURCES = ["clock_probe.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# packed fp32 VALU ops are disabled for every HIP translation unit
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-result"]


def _compile(src):
    out = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC] + CFLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{msg}")
    return out, msg


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)


def build(jobs=None, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CLOCK_SOURCES
    jobs = jobs or min(len(srcs), os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = dict(zip(srcs, ex.map(_compile, srcs)))
    for _, msg in results.values():
        if verbose and msg.strip():
            print(msg)
    _link([results[s][0] for s in SOURCES], LIB)
    _link([results[s][0] for s in CLOCK_SOURCES], CLOCK_LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    sys.exit(main())
