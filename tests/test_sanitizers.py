"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host-side code, CPU only.

* The oracle (plain C) is built with gcc -fsanitize=address,undefined and every oracle pin runs
  against it in a child process with the sanitizer runtimes preloaded.
* libtreeverify's host code (argument validation, plans, launch set-up) is built with the
  sanitizers on the host side only (device code is never sanitized) and the C-ABI argument
  tests run against it the same way; they return before any device call.

Any report aborts the child, which fails the test.  Leak detection is off: the Python
interpreter itself holds allocations until exit.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ENV_SAN = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _child(code: str, preload: str, timeout: int = 900) -> subprocess.CompletedProcess:
    env = dict(os.environ, **ENV_SAN, LD_PRELOAD=preload)
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=timeout)


def _gcc_runtime(name: str) -> str:
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()


def test_oracle_pins_under_asan_ubsan(tmp_path):
    so = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-shared",
                    "-fPIC", "-pthread", os.path.join(ROOT, "oracle", "tree_oracle.c"), "-o", so,
                    "-lm"], check=True)
    code = (
        "import sys; sys.path[:0] = ['tests', '.']\n"
        "import pins\n"
        "from oracle import oracle as O\n"
        f"lib = O.load({so!r})\n"
        "for p in pins.ALL_PINS:\n"
        "    p(lib)\n"
        "print('clean', len(pins.ALL_PINS))\n")
    res = _child(code, f"{_gcc_runtime('libasan.so')} {_gcc_runtime('libubsan.so')}")
    assert res.returncode == 0, res.stderr[-4000:]
    assert "clean" in res.stdout


def test_host_code_under_asan_ubsan(tmp_path):
    from tree_attention_verification_attn_amd import build

    runtime = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not runtime:
        pytest.skip("no clang AddressSanitizer runtime")
    so = str(tmp_path / "libtreeverify_san.so")
    flags = [f for f in build.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    res = subprocess.run([hipcc, *flags, *san, "-I", build.INCLUDE, "-I", build.CSRC,
                          *build.sources(), "-o", so], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    code = (
        "import sys, inspect; sys.path[:0] = ['tests', '.']\n"
        "import tree_attention_verification_attn_amd as tv\n"
        f"lib = tv.load_library({so!r})\n"
        "import test_abi\n"
        "n = 0\n"
        "for name, fn in inspect.getmembers(test_abi, inspect.isfunction):\n"
        "    if name.startswith('test_') and 'lib' in inspect.signature(fn).parameters:\n"
        "        fn(lib)\n"
        "        n += 1\n"
        "print('clean', n)\n")
    res = _child(code, runtime[-1])
    assert res.returncode == 0, res.stderr[-4000:]
    assert "clean" in res.stdout and int(res.stdout.split()[-1]) >= 10
