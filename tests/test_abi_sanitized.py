"""The C ABI's host-side argument checks and error paths under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, no GPU call reaches a kernel).

libqsa is rebuilt with the sanitizers on its host code only (-Xarch_host before each
-fsanitize flag; the gfx950 device code is the usual one) and test_abi_cpu.py runs
against it in a child process with the ASan runtime preloaded. Any heap or stack
overflow, use after free or undefined behaviour in the validation, error reporting or
workspace sizing aborts the child and fails this test.
"""
import glob
import os
import subprocess
import sys

import pytest

from block_sparse_attention_06_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SANITIZE = ("-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
            "-fno-omit-frame-pointer")


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no clang ASan runtime in this ROCm install")
    out = str(tmp_path_factory.mktemp("asan") / "libqsa_asan.so")
    B.build_library(B.SOURCES, out, extra_flags=SANITIZE)
    return out, rt


def test_sanitizers_are_compiled_in(sanitized_lib):
    # the host code calls the ASan and UBSan runtimes (undefined dynamic symbols)
    lib, _ = sanitized_lib
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True,
                          text=True, check=True).stdout
    assert "__asan_report_load" in syms or "__asan_report_store" in syms
    assert "__ubsan_handle" in syms


def test_abi_validation_under_asan_and_ubsan(sanitized_lib):
    lib, rt = sanitized_lib
    env = dict(os.environ, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = (f"import sys; sys.path.insert(0, {ROOT!r}); "
            "from block_sparse_attention_06_amd import _lib; "
            f"_lib.LIB_PATH = {lib!r}; import pytest; "
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', "
            f"{os.path.join(ROOT, 'tests', 'test_abi_cpu.py')!r}]))")
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                         timeout=900, cwd=ROOT)
    tail = (res.stdout[-4000:] + "\n" + res.stderr[-4000:])
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "ERROR: AddressSanitizer" not in tail
    assert "runtime error" not in tail
