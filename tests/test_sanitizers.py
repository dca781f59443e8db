"""Host code under AddressSanitizer + UndefinedBehaviorSanitizer (CPU only).

Two builds, each run in a subprocess with its sanitizer runtime preloaded
(gcc's and clang's runtimes cannot share a process):

  * the C oracle, built with gcc -fsanitize=address,undefined, running every
    oracle pin (tests/oracle_pins.py);
  * the HIP library with its host code instrumented (hipcc, -Xarch_host before
    each sanitizer flag, so device code is built as usual), running the
    host-side validation tests of the C ABI (tests/test_abi_cpu.py) and the
    tiled-layout size calls.  No case there reaches the device.

Each half first runs a small planted out-of-bounds read or signed overflow
under the same setup and requires the sanitizer to report it, so a silent
pass cannot come from a sanitizer that is not active.
"""

import glob
import importlib.util
import os
import subprocess
import sys
import textwrap
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
CSRC = ROOT / "gemm_ternary_linear_amd" / "csrc"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_runtime():
    libs = [subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True,
                           text=True).stdout.strip() for n in ("libasan.so", "libubsan.so")]
    if not all(os.path.isabs(p) and os.path.exists(p) for p in libs):
        pytest.skip("gcc sanitizer runtimes not found")
    return ":".join(libs)


def _clang_runtime():
    hits = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not hits or not os.path.exists(HIPCC):
        pytest.skip("clang sanitizer runtime or hipcc not found")
    return hits[0]


def _run(script: str, preload: str, *args):
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=preload)
    return subprocess.run([sys.executable, "-c", script, *map(str, args)], capture_output=True,
                          text=True, env=env, timeout=600)


PLANTED_C = """
#include <stdlib.h>
int oob(int n) { int *a = (int *)malloc(4 * sizeof(int)); int v = a[n]; free(a); return v; }
int ovf(int a) { return a + 2147483647; }
"""

CALL_PLANTED = textwrap.dedent("""
    import ctypes, sys
    lib = ctypes.CDLL(sys.argv[1])
    print(getattr(lib, sys.argv[2])(int(sys.argv[3])))
""")


def _check_planted(compiler, flags, preload, tmp_path):
    src = tmp_path / "planted.c"
    src.write_text(PLANTED_C)
    so = tmp_path / "libplanted.so"
    subprocess.check_call([compiler, *flags, "-shared", "-fPIC", "-x", "c", str(src), "-o", str(so)])
    r = _run(CALL_PLANTED, preload, so, "oob", 6)
    # gcc's object-size check may report the read before ASan does
    assert r.returncode != 0 and ("AddressSanitizer" in r.stderr or "runtime error" in r.stderr), \
        r.stderr[-2000:]
    r = _run(CALL_PLANTED, preload, so, "ovf", 5)
    assert r.returncode != 0 and "runtime error" in r.stderr, r.stderr[-2000:]


ORACLE_PINS = textwrap.dedent("""
    import sys
    sys.path.insert(0, %r); sys.path.insert(0, %r)
    import oracle
    from oracle_pins import PINS
    o = oracle.Oracle(sys.argv[1])
    for p in PINS:
        p(o)
    print("pins", len(PINS))
""") % (str(ROOT), str(ROOT / "tests"))


def test_oracle_under_asan_ubsan(tmp_path):
    preload = _gcc_runtime()
    flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined"]
    _check_planted("gcc", flags, preload, tmp_path)
    so = tmp_path / "liboracle_san.so"
    subprocess.check_call(["gcc", *flags, "-fopenmp", "-shared", "-fPIC", "-ffp-contract=off",
                           "-std=c11", "-Wall", str(ROOT / "oracle" / "ternary_oracle.c"), "-o",
                           str(so), "-lm"])
    r = _run(ORACLE_PINS, preload, so)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
    assert r.stdout.strip().startswith("pins")


ABI_TESTS = textwrap.dedent("""
    import sys
    from pathlib import Path
    sys.path.insert(0, %r)
    import gemm_ternary_linear_amd as tl
    tl.LIB_PATH = Path(sys.argv[1])
    assert tl.tiled_bytes(17, 260) == 4096
    import pytest
    sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", %r,
                          "-k", "not exported_symbols and not no_oracle_linkage"]))
""") % (str(ROOT), str(ROOT / "tests" / "test_abi_cpu.py"))

HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
            "-fno-omit-frame-pointer"]


def test_host_validation_under_asan_ubsan(tmp_path):
    preload = _clang_runtime()
    clangc = "/opt/rocm/lib/llvm/bin/clang"
    if not os.path.exists(clangc):
        pytest.skip("clang not found")
    _check_planted(clangc, ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                            "-fno-sanitize-recover=undefined", "-shared-libsan"], preload, tmp_path)
    spec = importlib.util.spec_from_file_location("ternary_build",
                                                  ROOT / "gemm_ternary_linear_amd" / "build.py")
    B = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(B)

    def comp(src):
        o = tmp_path / (Path(src).stem + ".o")
        subprocess.check_call([HIPCC, *B.FLAGS, "-O1", "-g", *HOST_SAN, "-c", str(CSRC / src),
                               "-o", str(o)], stderr=subprocess.DEVNULL)
        return o

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        objs = list(ex.map(comp, B.SOURCES))
    so = tmp_path / "libternary_san.so"
    subprocess.check_call([HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC",
                           *map(str, objs), "-o", str(so)])
    r = _run(ABI_TESTS, preload, so)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
    assert "passed" in r.stdout
