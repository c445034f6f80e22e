"""Ahead-of-time build of the gfx950 HIP library `libmla_fp8.so` (in-tree).

Usage: python -m mla_latent_kv_fp8_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla_fp8.so")
# measurement probe (bench.py --gather-probe), a library of its own: not the path's C ABI
PROBE_LIB = os.path.join(HERE, "libmla_probe.so")
PROBE_SRC = "probe_gather.hip"
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")
SOURCES = ["kv_write.hip", "decode_partial.hip", "merge_lse.hip", "value_gate.hip", "merge_value.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-FP32 instructions are generated
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    return obj


def build() -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, *FLAGS, "-shared", os.path.join(CSRC, PROBE_SRC), "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (PROBE_SRC, r.stderr))
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
