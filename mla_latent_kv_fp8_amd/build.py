"""Ahead-of-time build of the gfx950 HIP library `libmla_fp8.so` (in-tree).

Usage: python -m mla_latent_kv_fp8_amd.build [--timeline]

--timeline builds the measurement variant `libmla_fp8_timeline.so` (in-tree):
the same library with the partial kernel's per-workgroup wall-clock marks
compiled in (MLA_WG_TIMELINE) and read by `mla_latent_kv_fp8_amd.timeline`.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla_fp8.so")
TIMELINE_LIB = os.path.join(HERE, "libmla_fp8_timeline.so")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")
SOURCES = ["kv_write.hip", "absorb_q.hip", "decode_partial.hip", "merge_lse.hip", "value_gate.hip",
           "merge_value.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-FP32 instructions are generated
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# per-source flags: the partial kernel keeps its query in accumulation
# registers and its MFMA accumulators (O, S) in arch registers, which the
# compiler's default heuristic does not choose for it
SOURCE_FLAGS = {"decode_partial.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

# host code (argument checks, the host-built split partition, launches)
# instrumented with AddressSanitizer and UndefinedBehaviorSanitizer; the
# device code is built as usual
SANITIZE_FLAGS = ["-g", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address",
                  "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all"]
SANITIZED_LIB = os.path.join(BUILD_DIR, "asan", "libmla_fp8_asan.so")


def _compile(src: str, sanitize: bool = False, timeline: bool = False) -> str:
    out_dir = os.path.join(BUILD_DIR, "asan" if sanitize else "timeline") if sanitize or timeline else BUILD_DIR
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    marks = ["-DMLA_WG_TIMELINE"] if timeline and src == "decode_partial.hip" else []
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), *(SANITIZE_FLAGS if sanitize else []), *marks, "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    return obj


def build(sanitize: bool = False, timeline: bool = False) -> str:
    """Build the library in-tree; or (sanitize=True) the host-sanitizer build
    under _build/asan, which a process loads with the clang ASan runtime
    preloaded; or (timeline=True) the measurement build
    libmla_fp8_timeline.so, in-tree."""
    out = SANITIZED_LIB if sanitize else (TIMELINE_LIB if timeline else LIB)
    os.makedirs(os.path.dirname(SANITIZED_LIB) if sanitize else
                os.path.join(BUILD_DIR, "timeline") if timeline else BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize, timeline), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    link_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-shared-libsan"] if sanitize else []
    r = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *link_san, *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(timeline="--timeline" in sys.argv[1:]))
    sys.exit(0)
