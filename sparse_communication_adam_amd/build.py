"""Build libscape.so (HIP for gfx950) in-tree with hipcc.

Flags that matter for the numerics:
  -ffp-contract=off                          no fused multiply-add: every fp32
                                             operation rounds on its own
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE-correct fp32 '/' and sqrtf
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                             no packed fp32 instructions
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libscape.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["k_elementwise.hip", "k_select.hip", "k_bits.hip", "scape_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
         "-fhip-fp32-correctly-rounded-divide-sqrt", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


# AddressSanitizer and UBSan for the host code only (argument validation,
# layout, tables, launch sequences); the device code is built as usual.
HOST_SANITIZE = ["-g", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                 "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _compile(src: str, build_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False, out: str = None) -> str:
    """Compile every source for gfx950 and link libscape.so next to this file
    (or, with sanitize, a host-sanitizer build to `out`)."""
    out = out or LIB_PATH
    build_dir = BUILD_DIR + ("_sanitize" if sanitize else "")
    extra = HOST_SANITIZE if sanitize else ()
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *(["-Xarch_host", "-fsanitize=address", "-Xarch_host",
                                                                  "-fsanitize=undefined"] if sanitize else []),
           *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
