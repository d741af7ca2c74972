"""The CPU suite under AddressSanitizer and UBSan (CPU only).

Two builds, each run in a child process with its sanitizer runtime preloaded
(the two runtimes cannot share a process):
  - the oracle, built by gcc with -fsanitize=address,undefined, under the
    oracle pins and the checkpoint tests;
  - libscape with its host code built by hipcc under the same sanitizers (the
    device code as usual), under the ABI tests, which drive argument
    validation, the layout, the owner map and context creation without a GPU.
Any sanitizer report fails the child process and so this test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG_RT = "/opt/rocm/lib/llvm/lib/clang"


def _clang_asan_runtime():
    if not os.path.isdir(CLANG_RT):
        return None
    for ver in sorted(os.listdir(CLANG_RT), reverse=True):
        p = os.path.join(CLANG_RT, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def _run(tests, env):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


def _env(preload, **extra):
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    env.update(extra)
    return env


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    import oracle
    lib = oracle.build(sanitize=True, out=str(tmp_path / "liboracle_asan.so"))
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    out = _run(["tests/test_oracle_pins.py", "tests/test_checkpoint.py"], _env(asan, SCAPE_ORACLE_LIB=lib))
    assert "passed" in out


def test_library_host_paths_under_address_and_ub_sanitizers(tmp_path):
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("clang AddressSanitizer runtime not found")
    from sparse_communication_adam_amd.build import build
    lib = build(sanitize=True, out=str(tmp_path / "libscape_asan.so"))
    out = _run(["tests/test_abi.py"], _env(rt, SCAPE_LIB=lib))
    assert "passed" in out
