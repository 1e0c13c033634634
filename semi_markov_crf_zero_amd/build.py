"""Build libsemicrf.so (gfx950) in-tree with hipcc.

    python -m semi_markov_crf_zero_amd.build [--asm]

Every .hip file under csrc/ is compiled to an object in _build/ (in
parallel) and linked into semi_markov_crf_zero_amd/libsemicrf.so; the
peak microbenchmarks under probe/ (used by the benchmark only) become
semi_markov_crf_zero_amd/libsemicrf_peaks.so.
Packed FP32 instructions are disabled for all device code.  --asm also keeps
the gfx950 assembly (_build/*.s) for inspection.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsemicrf.so")
PROBE = os.path.join(PKG, "probe")
PEAKS_LIB = os.path.join(PKG, "libsemicrf_peaks.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    "-Wall", "-Wno-unused-result",
]


def _compile(src: str, asm: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(os.path.dirname(src)) + "_" +
                       os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + ["-c", src, "-o", obj]
    if asm:
        cmd += ["--save-temps"]
    r = subprocess.run(cmd, cwd=BUILD, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed for %s" % src)
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.check_call(cmd)
    os.replace(tmp, lib)


def build(asm: bool = False, jobs: int = 4) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    probes = sorted(glob.glob(os.path.join(PROBE, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, asm), srcs + probes))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    print(build(asm="--asm" in sys.argv))
