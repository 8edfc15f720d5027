"""Build the host side of libtpla under AddressSanitizer and UBSan (CPU only).

    python -m tensor_latent_decode_amd.build_sanitize

Compiles every source of the library with the address and undefined-
behaviour sanitizers on the host side only (the device code is built as
usual; its kernels are not launched on a host without a GPU), into
_build/sanitize/libtpla.so.  The
argument checks, split planning and the split cost model then run under the
sanitizers when a process loads that library (TPLA_LIB=<path>) with the
sanitizer runtime preloaded (runtime_path()).
"""

from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

from tensor_latent_decode_amd import build as _b

OUT = os.path.join(_b.OBJ, "sanitize")
LIB = os.path.join(OUT, "libtpla.so")

# host-side sanitizer flags, each behind -Xarch_host so no device code is
# built with them
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["-O1", "-g", "--offload-arch=gfx950", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", _b.INCLUDE, "-I", _b.CSRC]


def runtime_path() -> str:
    """The sanitizer runtime a non-instrumented interpreter must preload."""
    res = subprocess.run([_b.hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True)
    return res.stdout.strip().splitlines()[-1]


def _compile(src: str) -> str:
    obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
    cmd = [_b.hipcc(), *FLAGS, *SAN, "-c", os.path.join(_b.CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build() -> str:
    os.makedirs(OUT, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(_b.SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, _b.SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_b.hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, *SAN, "-shared-libsan",
           "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking the sanitizer build failed:\n{' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(f"built {build()}")
