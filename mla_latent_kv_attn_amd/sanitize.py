"""Host-only AddressSanitizer + UndefinedBehaviorSanitizer build of the library.

Compiles every source with its host side (argument validation, launch
configuration, launch wrappers) instrumented by ASan and UBSan into a
separate library, for running the C-ABI tests on the CPU under the
sanitizers (device code is built as usual and is not instrumented):

    python -m mla_latent_kv_attn_amd.sanitize          # build, then run tests/test_abi.py

The library is loaded in its place through MLA_ATTN_LIB; Python itself is
not instrumented, so the ASan runtime is preloaded (LD_PRELOAD) into the
test process.  Without a GPU, a call that passes validation reports a HIP
error.
"""

import concurrent.futures
import glob
import os
import subprocess
import sys

from . import build as _b

SAN_DIR = os.path.join(_b.BUILD_DIR, "host_san")
SAN_LIB = os.path.join(SAN_DIR, "libmla_attn_host_san.so")

# Each sanitizer flag applies to the host compilation only.
SAN_FLAGS = [
    *"-Xarch_host -fsanitize=address".split(),
    *"-Xarch_host -fsanitize=undefined".split(),
    *"-Xarch_host -fno-sanitize-recover=all".split(),
    *"-Xarch_host -fno-omit-frame-pointer".split(),
]


def asan_runtime():
    """Path of the compiler's shared ASan runtime (it also holds the UBSan handlers)."""
    llvm = os.path.join(os.path.dirname(os.path.realpath(_b.HIPCC)), "..", "llvm")
    pat = os.path.join(llvm, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")
    hits = sorted(glob.glob(pat)) or sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError(f"no ASan runtime found ({pat})")
    return os.path.realpath(hits[-1])


def build_host_sanitized():
    """Compile every source, its host side with ASan + UBSan; returns the library path."""
    os.makedirs(SAN_DIR, exist_ok=True)
    # Device code as in the regular build; host code at -O1 with debug lines.
    flags = [*_b.COMMON_FLAGS, *"-Xarch_host -O1 -Xarch_host -g".split(), *SAN_FLAGS]
    srcs = _b.sources()
    objs = [os.path.join(SAN_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(lambda so: _b._run([_b.HIPCC, *flags, "-c", so[0], "-o", so[1]]), zip(srcs, objs)))
    # Linked without the runtime: its symbols come from the preloaded ASan library.
    _b._run([_b.HIPCC, "-shared", "-fPIC", *objs, "-o", SAN_LIB])
    return SAN_LIB


def sanitized_env(lib=SAN_LIB):
    env = dict(os.environ)
    env["MLA_ATTN_LIB"] = lib
    env["LD_PRELOAD"] = asan_runtime()
    # Python's own allocations are not tracked: leak reports would be noise.
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


def run_abi_tests(lib=SAN_LIB, timeout=600):
    """Run tests/test_abi.py in a child process under the sanitizers."""
    root = _b.ROOT
    cmd = [sys.executable, "-m", "pytest", os.path.join(root, "tests", "test_abi.py"), "-q", "-p", "no:cacheprovider"]
    return subprocess.run(cmd, cwd=root, env=sanitized_env(lib), stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                          text=True, timeout=timeout)


if __name__ == "__main__":
    print(build_host_sanitized())
    r = run_abi_tests()
    print(r.stdout)
    sys.exit(r.returncode)
