"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code:
the CPU oracle (oracle/ssd_oracle.c) and the host side of libssd's C ABI
(argument checks, workspace layouts, path choice).  Each is compiled with the
sanitizers into a temporary directory with a driver program of its own
(tests/sanitize/), which is run and must exit cleanly: the sanitizers abort on
an out-of-bounds access, a use after free, a leak, signed overflow or another
undefined operation.  No GPU is used (the ABI driver makes only calls that
return before any HIP call).
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="abort_on_error=1:detect_leaks=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="3")


def _run(cmd, env=None, timeout=300):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "ssd_oracle.c"), os.path.join(SAN, "oracle_driver.c"),
          "-o", exe, "-lm"])
    out = _run([exe], env=ENV)
    assert "oracle sanitizer driver: ok" in out


def test_abi_host_code_under_sanitizers(tmp_path):
    """Every translation unit of libssd rebuilt with the sanitizers on its host
    code only (each flag after -Xarch_host; device code as shipped), linked
    with the driver by the host compiler."""
    from selective_state_space_ssd_amd import _build
    try:
        hipcc = _build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang++"
    if not os.path.exists(clang):
        pytest.skip("ROCm's clang++ not available")
    host_san = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
                 "-fno-omit-frame-pointer", "-g"):
        host_san += ["-Xarch_host", flag]
    flags = [f for f in _build.CFLAGS if f != "-O3"] + ["-O1"] + host_san

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        _run([hipcc, *flags, "-c", os.path.join(_build.CSRC, src), "-o", obj], timeout=600)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, _build.SOURCES))
    # the driver and the link: the same compiler's sanitizer runtimes as the
    # objects (host code only: no .hip file on these lines)
    drv = str(tmp_path / "abi_driver.o")
    _run([clang, "-x", "c", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I",
          os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", "-c",
          os.path.join(SAN, "abi_driver.c"), "-o", drv])
    exe = str(tmp_path / "abi_driver")
    _run([clang, "-fsanitize=address,undefined", drv, *objs, "-L/opt/rocm/lib",
          "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe])
    # the HIP runtime keeps allocations of its own until exit: leaks are not
    # this library's (it allocates nothing), so leak checking is off here
    env = dict(ENV, ASAN_OPTIONS="abort_on_error=1:detect_leaks=0")
    out = _run([exe], env=env)
    assert "abi sanitizer driver: ok" in out
