"""Build libdetk.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
# the host API and one translation unit per tile size's kernels, compiled in parallel
SOURCES = [os.path.join(CSRC, n) for n in ("detk_api.hip", "inst_4096.hip", "inst_8192.hip", "inst_16384.hip",
                                           "inst_32768.hip", "indexer.hip")]
DEPS = SOURCES + [os.path.join(CSRC, "topk_device.hpp"), os.path.join(CSRC, "kernels.hpp"),
                  os.path.join(CSRC, "indexer.hpp"),
                  os.path.join(ROOT, "include", "detk.h")]
OUT = os.path.join(HERE, "libdetk.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # Packed FP32 instructions are kept out of the code object on purpose.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build_library(force: bool = True, extra_flags=()) -> str:
    if not force and os.path.exists(OUT) and all(os.path.getmtime(OUT) >= os.path.getmtime(d) for d in DEPS):
        return OUT
    import concurrent.futures
    tag = "%d" % os.getpid()
    objs = [os.path.join(CSRC, os.path.basename(src) + ".%s.o" % tag) for src in SOURCES]

    def compile_one(pair):
        src, obj = pair
        subprocess.check_call([hipcc()] + HIPCC_FLAGS + list(extra_flags) + ["-c", src, "-o", obj])

    try:
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            list(ex.map(compile_one, zip(SOURCES, objs)))
        tmp = OUT + ".tmp" + tag
        subprocess.check_call([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp])
        os.replace(tmp, OUT)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return OUT


if __name__ == "__main__":
    print(build_library(force=True, extra_flags=sys.argv[1:]))
