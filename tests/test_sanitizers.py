"""Memory and undefined-behaviour checks of the host code: the C oracle and the C-ABI
library's host side (argument validation, sizing, workspace layout), each built with
AddressSanitizer and UndefinedBehaviorSanitizer and driven by the existing CPU tests in a
child process.

The oracle is built by gcc, the library by hipcc with the sanitizers on its host pass only
(``-Xarch_host`` before each option; the gfx950 code objects are built as usual).  A Python
interpreter is not itself instrumented, so each child preloads its compiler's ASan runtime.
Leak checking is off (the interpreter keeps allocations alive at exit); every other report
ends the child with an error.  A planted heap overrun in a throw-away C file, built and loaded
the same way, checks that the harness does catch what it is meant to catch.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:exitcode=86",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=87"}
ORACLE_TESTS = ["test_oracle_attn.py", "test_oracle_cache.py", "test_oracle_fp16.py", "test_oracle_quant.py",
                "test_oracle_quant4.py", "test_oracle_rope.py", "test_layout_golden.py"]

pytestmark = pytest.mark.slow


def _gcc_asan():
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def _clang_asan():
    clang = "/opt/rocm/lib/llvm/bin/clang"
    if not os.path.exists(clang):
        pytest.skip("no ROCm clang")
    return subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                          text=True, check=True).stdout.strip()


def _instrumented(lib):
    """The build calls the ASan and UBSan runtimes."""
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms


def _child(args, preload, extra_env, timeout=900):
    env = dict(os.environ, **ENV, **extra_env, LD_PRELOAD=preload, PYTHONDONTWRITEBYTECODE="1")
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


def test_planted_overrun_is_reported(tmp_path):
    src = tmp_path / "overrun.c"
    src.write_text("#include <stdlib.h>\n"
                   "int poke(int n) { int *a = malloc(n * sizeof(int)); a[n] = 1; int r = a[0]; free(a); return r; }\n")
    lib = tmp_path / "liboverrun.so"
    subprocess.run(["gcc", "-shared", "-fPIC", *SAN, str(src), "-o", str(lib)], check=True)
    r = _child(["-c", f"import ctypes; ctypes.CDLL({str(lib)!r}).poke(4)"], _gcc_asan(), {})
    assert r.returncode == 86 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]


def test_oracle_pins_under_asan_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from oracle import build as oracle_build
    lib = oracle_build.build(out=str(tmp_path / "libkivi_oracle_san.so"), extra_flags=SAN)
    _instrumented(lib)
    probe = "import os; from oracle import ref; assert ref.lib()._name == os.environ['KIVI_ORACLE_LIB']"
    r = _child(["-c", probe], _gcc_asan(), {"KIVI_ORACLE_LIB": lib})
    assert r.returncode == 0, r.stderr[-2000:]
    tests = [os.path.join("tests", t) for t in ORACLE_TESTS]
    r = _child(["-m", "pytest", "-q", "-x", "-m", "not gpu and not slow", "-p", "no:cacheprovider",
                "-n", "8", *tests], _gcc_asan(), {"KIVI_ORACLE_LIB": lib})
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout and "error" not in r.stdout.splitlines()[-1]


def test_library_host_code_under_asan_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from kv_cache_bit_quantize_amd import build as kivi_build
    flags = [x for f in SAN for x in ("-Xarch_host", f)]
    lib = kivi_build.build(out=str(tmp_path / "libkivi_san.so"), extra_flags=flags)
    _instrumented(lib)
    probe = ("import os; from kv_cache_bit_quantize_amd import kivi; "
             "assert kivi._load()._name == os.environ['KIVI_LIBRARY']")
    r = _child(["-c", probe], _clang_asan(), {"KIVI_LIBRARY": lib})
    assert r.returncode == 0, r.stderr[-2000:]
    r = _child(["-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider", "tests/test_abi.py"],
               _clang_asan(), {"KIVI_LIBRARY": lib})
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout
