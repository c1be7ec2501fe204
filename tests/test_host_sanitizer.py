"""The host side of the C ABI (argument validation, error reporting, the
static-scratch entry point's checks) under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

The three API sources are compiled with the sanitizers on their host code
only (each -fsanitize flag after -Xarch_host; the device code is unchanged)
and linked with the library's kernel objects into a separate library; the
ABI tests then run against it in a child interpreter with the ASan runtime
preloaded.  Without a GPU every call ends in argument validation or a failed
HIP runtime call, which are exactly the host paths these tests reach.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_decoder_speculative_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
SAN = os.path.join(BUILD, "san")
API = ("api.cpp", "api_draft.cpp", "api_static.cpp")


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _build_sanitized() -> str:
    from moe_decoder_speculative_amd import build as B
    kernel_objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in B.sources()
                   if os.path.basename(s) not in API]
    if not all(os.path.exists(o) for o in kernel_objs):
        B.build(verbose=False)
    os.makedirs(SAN, exist_ok=True)
    host_flags = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
    objs = []
    for name in API:
        out = os.path.join(SAN, name + ".o")
        cmd = [B.HIPCC, *B.COMMON, "-O1", "-g", *host_flags, "-x", "hip", "-c", os.path.join(CSRC, name), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(out)
    lib = os.path.join(SAN, "libmoeverify_san.so")
    clang = os.path.join(os.path.dirname(B.HIPCC), "..", "lib", "llvm", "bin", "clang++")
    # the link is host code only: the sanitizer runtimes come from the preload
    cmd = [clang, "-shared", "-fPIC", *objs, *kernel_objs, "-o", lib, "-L/opt/rocm/lib", "-lamdhip64",
           "-shared-libsan", "-fsanitize=address,undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return lib


@pytest.mark.slow
def test_abi_host_paths_under_asan_and_ubsan():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no ASan runtime in this toolchain")
    lib = _build_sanitized()
    child = (
        "import sys; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
        "from moe_decoder_speculative_amd import binding\n"
        "binding.load_library(%r)\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r]))\n"
    ) % (ROOT, os.path.join(ROOT, "tests"), lib, os.path.join(ROOT, "tests", "test_abi.py"))
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, env=env, timeout=900)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0 and " passed" in out, out[-4000:]
