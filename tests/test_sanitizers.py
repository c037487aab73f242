"""The host code under AddressSanitizer + UndefinedBehaviorSanitizer, on the CPU.

Two sanitized builds are made in a temporary directory:
  * the oracle (oracle/ssm_oracle.c, same fp flags) -- oracle.build_sanitized;
  * libssmscan.so with its host-side C ABI (ssm_abi.cpp: argument validation,
    size and overlap arithmetic) instrumented; GPU code is not sanitized
    (the flags go to the host pass only) -- build.build_host_sanitized.
The oracle's pins, the planted-mistake check and the C-ABI contract tests then
run in a child process with the sanitizer runtime preloaded and both builds
loaded in place of the regular ones; any report aborts that process.  A copy
of the oracle with one planted out-of-bounds read shows the runtime is live."""
import os
import subprocess
import sys

import pytest

import oracle
from selective_scan_ssm_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


def asan_runtime():
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    rt = asan_runtime()
    if rt is None or not os.path.exists(CLANG):
        pytest.skip("no clang AddressSanitizer runtime in this image")
    d = tmp_path_factory.mktemp("sanitized")
    lib = build.build_host_sanitized(str(d / "libssmscan_asan.so"))
    orc = oracle.build_sanitized(str(d / "libssm_oracle_asan.so"), cc=CLANG)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", SSM_SCAN_LIB=lib, SSM_ORACLE_LIB=orc,
               PYTHONDONTWRITEBYTECODE="1")
    return {"env": env, "lib": lib, "oracle": orc, "dir": d}


def test_sanitized_builds_are_the_ones_loaded(sanitized):
    code = ("import ctypes, oracle\n"
            "from selective_scan_ssm_amd import _lib\n"
            "_lib.load(); oracle.load()\n"
            "maps = open('/proc/self/maps').read()\n"
            "ctypes.CDLL(None).__asan_init\n"
            "print('scan' if _lib.LIB_PATH in maps else '-', 'oracle' if oracle._LIB_OVERRIDE in maps else '-')\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=sanitized["env"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.split() == ["scan", "oracle"], r.stdout


def test_pins_and_abi_contract_run_clean(sanitized):
    tests = ["tests/test_abi.py", "tests/test_oracle_pins.py", "tests/test_oracle_mutants.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *tests],
                       cwd=ROOT, env=sanitized["env"], capture_output=True, text=True, timeout=1200)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail


def test_a_planted_out_of_bounds_read_is_caught(sanitized):
    # one read one state past the caller's h0 in a copy of the oracle
    src = open(os.path.join(ROOT, "oracle", "ssm_oracle.c")).read()
    good = "h[n] = h0 ? h0[(b * dim + d) * dstate + n] : 0.0;"
    assert src.count(good) == 1
    bad = src.replace(good, "h[n] = h0 ? h0[(b * dim + d) * dstate + n + dstate] : 0.0;")
    path = sanitized["dir"] / "oob.c"
    path.write_text(bad)
    lib = sanitized["dir"] / "liboob.so"
    subprocess.run([CLANG, *oracle.CFLAGS, "-fsanitize=address,undefined", "-shared-libasan", str(path), "-o",
                    str(lib), "-lm"], check=True)
    code = ("import numpy as np, oracle\n"
            f"lib = oracle.load({str(lib)!r})\n"
            "x = np.ones((1, 3, 2)); B = np.ones((1, 3, 4)); A = -np.ones((2, 4)); h0 = np.ones((1, 2, 4))\n"
            "oracle.selective_scan(x, x, A, B, B, h0=h0, lib=lib)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=sanitized["env"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-2000:]
