"""Build the gfx950 shared library libmoe_mx.so in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_mx.so")

SOURCES = ["quant.hip", "route.hip", "ffn.hip", "ffn_mfma.hip", "layer_m1.hip", "verify.hip", "qk_rope.hip",
           "util.hip", "capi.cpp"]
HIPCC = os.environ.get("HIPCC", "hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + INCLUDE, "-I" + CSRC]


# Host-side checking build (CPU tests only): AddressSanitizer and UndefinedBehaviorSanitizer on
# the host code (argument validation, workspace layout, launch set-up); the device code is built
# as usual.  Its process must preload clang's ASan runtime (sanitizer_runtime()).
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
                  "-fno-omit-frame-pointer"]


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, src + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(out: str = LIB, sanitize_host: bool = False) -> str:
    """Compile every source for gfx950 and link libmoe_mx.so (or `out`).  With sanitize_host,
    the host-only checking build described above."""
    build_dir = BUILD if not sanitize_host else os.path.join(BUILD, "host_sanitized")
    os.makedirs(build_dir, exist_ok=True)
    extra = SANITIZE_FLAGS if sanitize_host else []
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), SOURCES))
    tmp = out + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)
    return out


def sanitizer_runtime() -> str:
    """Path of the ASan runtime of the compiler that built the host-sanitized library."""
    r = subprocess.run([HIPCC, "--print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang's ASan runtime not found")
    return path


if __name__ == "__main__":
    print(build())
