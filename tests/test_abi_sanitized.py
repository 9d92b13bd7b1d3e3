"""The C ABI's host-side checks under the host sanitizers (address, undefined behaviour, leaks).

The library's sources are compiled again with ``-Xarch_host`` sanitizer flags (the host code is
instrumented; the device code is built as usual and never launched here) and linked with two plain C
programs: ``c_abi/abi_from_c.c`` and ``c_abi/abi_host_checks.c`` (every entry point at extreme argument
values, each call refused on the host with its documented code).  A signed overflow, an out-of-bounds access
or a leak in the argument checks or the workspace-size functions fails the run.  The checks program also runs
against the product library built by ``build()``.  No GPU is used: every call is answered on the host.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "paged_kv_cache_300_amd")
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")

SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
       "-Xarch_host", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
PROGRAMS = ["abi_from_c.c", "abi_host_checks.c"]


def _sources():
    from paged_kv_cache_300_amd import build as B
    return B.SOURCES


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, " ".join(cmd) + "\n" + res.stdout[-3000:] + res.stderr[-3000:]
    return res


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not available")
    out = tmp_path_factory.mktemp("san")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", f"-I{INCLUDE}", f"-I{CSRC}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN]

    def compile_one(src):
        obj = str(out / (src + ".o"))
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        _run([HIPCC, *lang, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=6) as ex:
        objs = list(ex.map(compile_one, _sources()))
    exes = {}
    for prog in PROGRAMS:
        cobj = str(out / (prog + ".o"))
        _run([CLANG, "-std=c11", "-Wall", "-g", "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}", f"-I{ROCM}/include",
              "-Xarch_host", "-fsanitize=address,undefined", "-c", os.path.join(HERE, "c_abi", prog), "-o", cobj])
        exe = str(out / prog[:-2])
        _run([HIPCC, "--offload-arch=gfx950", *SAN, cobj, *objs, "-o", exe])
        exes[prog] = exe
    return exes


@pytest.mark.parametrize("prog", PROGRAMS)
def test_host_checks_under_sanitizers(sanitized, prog):
    res = subprocess.run([sanitized[prog]], capture_output=True, text=True, timeout=120, env=ENV)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), res.stdout[-3000:] + res.stderr[-3000:]
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-3000:]


def test_host_checks_against_built_library(tmp_path):
    """abi_host_checks.c, plain gcc, against the library as built (libpagedkv.so next to the package)."""
    lib = os.path.join(PKG, "libpagedkv.so")
    gcc = shutil.which("gcc")
    if not os.path.exists(lib) or gcc is None:
        pytest.skip("library not built or gcc missing")
    exe = str(tmp_path / "abi_host_checks")
    _run([gcc, "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}", f"-I{ROCM}/include",
          os.path.join(HERE, "c_abi", "abi_host_checks.c"), f"-L{PKG}", "-lpagedkv", f"-Wl,-rpath,{PKG}", "-lm",
          "-o", exe])
    res = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0 and res.stdout.strip() == "ok", res.stdout + res.stderr
