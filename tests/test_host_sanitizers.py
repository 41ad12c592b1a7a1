"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source is compiled as for the product library (device code for gfx950
unchanged) with the two sanitizers on the host side only, linked with
tests/host_checks.c into an executable, and run.  The checks make no kernel
launch (validation, null arguments, the span bound, context creation with or
without a device, and a random sweep of parameters), so they run on the CPU;
where a device is present the driver also round-trips a small index through
import and export in both tiers.  The build is cached under _build/asan by a
hash of the sources."""
import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_kv_cache_sekv_amd", "csrc")
INC = os.path.join(ROOT, "include")
DRIVER = os.path.join(ROOT, "tests", "host_checks.c")
OUT = os.path.join(ROOT, "_build", "asan")
SOURCES = ["runtime.cpp", "attend.hip", "route.hip", "build.hip", "rsvd.hip", "gather.hip"]
ROCM = "/opt/rocm"


def _tool(*names):
    for n in names:
        if os.path.exists(n):
            return n
    return None


def _digest() -> str:
    h = hashlib.sha256()
    paths = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))] + [DRIVER, os.path.join(INC, "sekv.h")]
    for p in paths:
        with open(p, "rb") as f:
            h.update(p.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def _build(hipcc, clang, clangxx) -> str:
    d = os.path.join(OUT, _digest())
    exe = os.path.join(d, "host_checks")
    if os.path.exists(exe):
        return exe
    os.makedirs(d, exist_ok=True)
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer"]

    def one(src):
        obj = os.path.join(d, os.path.splitext(src)[0] + ".o")
        _run([hipcc, "-O1", "-g", "-std=c++17", "-fPIC", "-x", "hip", "--offload-arch=gfx950",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + host_san +
             ["-I", INC, "-I", CSRC, "-w", "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=6) as ex:
        objs = list(ex.map(one, SOURCES))
    drv = os.path.join(d, "host_checks.o")
    _run([clang, "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
          "-I", INC, "-c", DRIVER, "-o", drv])
    tmp = exe + ".tmp"
    _run([clangxx, "-fsanitize=address,undefined", drv] + objs +
         ["-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", tmp])
    os.replace(tmp, exe)
    return exe


def test_host_code_under_address_and_undefined_behaviour_sanitizers():
    hipcc = _tool(os.path.join(ROCM, "bin", "hipcc"), shutil.which("hipcc") or "")
    clang = _tool(os.path.join(ROCM, "llvm", "bin", "clang"))
    clangxx = _tool(os.path.join(ROCM, "llvm", "bin", "clang++"))
    if not (hipcc and clang and clangxx):
        pytest.skip("ROCm compilers not found")
    exe = _build(hipcc, clang, clangxx)
    env = dict(os.environ)
    # leaks inside the HIP runtime are not this library's; overflow and
    # out-of-bounds reports end the run with a non-zero status
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
