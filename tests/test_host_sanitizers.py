"""The C-ABI tests (tests/test_abi.py) under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

The library's host code is rebuilt with both sanitizers (device code as
usual) and loaded through MLA_ATTN_LIB in a child Python process that has
the ASan runtime preloaded; any sanitizer report ends that process with an
error.  A canary library built the same way, with a signed overflow in it,
shows that reports from a library loaded like this are seen.
"""

import os
import subprocess
import sys

import pytest

from mla_latent_kv_attn_amd import sanitize


@pytest.fixture(scope="module")
def runtime():
    try:
        return sanitize.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))


def _child(code, env):
    return subprocess.run([sys.executable, "-c", code], env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                          text=True, timeout=300)


def test_canary_overflow_is_reported(runtime, tmp_path):
    src = tmp_path / "canary.cpp"
    src.write_text('extern "C" int add_one(int a) { return a + 1; }\n')
    so = tmp_path / "libcanary.so"
    clang = os.path.join(os.path.dirname(os.path.realpath(sanitize._b.HIPCC)), "..", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang++"
    subprocess.run([clang, "-shared", "-fPIC", "-O1", "-fsanitize=undefined,address", "-fno-sanitize-recover=all",
                    str(src), "-o", str(so)], check=True)
    env = sanitize.sanitized_env(str(so))
    code = f"import ctypes; f = ctypes.CDLL({str(so)!r}).add_one; print(f(41)); print(f({(1 << 31) - 1}))"
    r = _child(code, env)
    assert r.returncode != 0 and "42" in r.stdout and "signed integer overflow" in r.stdout, r.stdout[-2000:]


def test_abi_tests_pass_under_asan_and_ubsan(runtime):
    lib = sanitize.build_host_sanitized()
    env = sanitize.sanitized_env(lib)
    probe = ("from mla_latent_kv_attn_amd import binding; binding.load(); "
             "print(open('/proc/self/maps').read())")
    maps = _child(probe, env)
    assert maps.returncode == 0, maps.stdout[-2000:]
    assert lib in maps.stdout and runtime in maps.stdout
    r = sanitize.run_abi_tests(lib)
    assert r.returncode == 0, r.stdout[-4000:]
    assert " passed" in r.stdout and "failed" not in r.stdout
