"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The two host files of the C ABI (dec_api.cpp, attn_api.cpp: configuration checks,
workspace layout, argument validation, staging) are compiled again with the sanitizers
on their host side only (device code is built without them), linked with the regular
kernel objects, and the CPU ABI tests run against that library in a child process that
preloads the sanitizer runtime.  Any report (out-of-bounds access, use after free,
signed overflow, misaligned access, ...) stops the child with a non-zero status.
"""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "memory_bound_transformer_decode_amd")
HOST_FILES = ("dec_api.cpp", "attn_api.cpp")
# host-only instrumentation: every sanitizer flag is scoped to the host compilation
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_abi_checks_under_host_sanitizers(tmp_path):
    from memory_bound_transformer_decode_amd import build
    rt = _runtime()
    if rt is None or not os.path.exists(build.hipcc()):
        pytest.skip("hipcc or the sanitizer runtime is not installed")
    others = [s for s in build.sources() if os.path.basename(s) not in HOST_FILES]
    objs = [os.path.join(build.BUILD, os.path.basename(s) + ".o") for s in others]
    if not all(os.path.exists(o) for o in objs):
        build.build()
    san_objs = []
    for f in HOST_FILES:
        obj = str(tmp_path / (f + ".o"))
        cmd = [build.hipcc(), "-x", "hip", f"--offload-arch={build.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", build.INCLUDE, "-I", build.CSRC, *SAN, "-c", os.path.join(build.CSRC, f), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        san_objs.append(obj)
    lib = str(tmp_path / "libdec_hostsan.so")
    r = subprocess.run([build.hipcc(), f"--offload-arch={build.ARCH}", "-shared", "-fPIC", *san_objs, *objs,
                        *build.LINK_LIBS, "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    # the host code is instrumented: the library calls the sanitizers' report hooks
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms

    child = (
        "import sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "from memory_bound_transformer_decode_amd import dec\n"
        f"l = dec.load_library({lib!r})\n"
        f"assert l._name == {lib!r}\n"
        "import pytest\n"
        f"sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', {os.path.join(ROOT, 'tests', 'test_abi.py')!r}]))\n"
    )
    env = dict(os.environ, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
