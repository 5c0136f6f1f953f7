"""Host-sanitised build of libspectree, for CPU tests of the host side of the C ABI.

    python -m tree_attention_verification_spec_amd.asan_build

Compiles every ``csrc/*.hip`` with AddressSanitizer and UndefinedBehaviorSanitizer on the host
pass only (each sanitizer flag carries -Xarch_host; the gfx950 device code is built exactly as
in the product library) into ``_build/asan/libspectree_asan.so``.  The CPU tests load it in a
child process with clang's ASan runtime preloaded and drive the argument checks, workspace
queries and status strings through ctypes; nothing in it is ever launched on a GPU.
"""

import concurrent.futures as cf
import os
import subprocess
import sys

from . import build as _b

OUT_DIR = os.path.join(_b.BUILD, "asan")
OUT = os.path.join(OUT_DIR, "libspectree_asan.so")
CLANG = "/opt/rocm/llvm/bin/clang"

HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]


def runtime():
    """Path of clang's shared ASan runtime (to preload into the uninstrumented interpreter)."""
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang's ASan runtime was not found")
    return path


def _compile(src):
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    r = subprocess.run([_b.HIPCC, *_b.FLAGS, *HOST_SAN, "-c", src, "-o", obj], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}{r.stderr}")
    return obj


def build():
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = _b.sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    r = subprocess.run([_b.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-shared-libsan",
                        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-o", tmp] + objs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
    sys.exit(0)
