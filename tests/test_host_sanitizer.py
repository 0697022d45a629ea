"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU): every source is compiled with the sanitizers on its host
pass only (device code is compiled as usual and never runs), linked with
sanitizer_driver.cpp and sanitizer_status.c, and the driver is run.  It plans
a grid of shapes (valid, ragged, extreme and invalid), runs the EC scheduler
and its selection step on random inputs, and calls every device entry point
with arguments its checks must reject before anything is enqueued; any
sanitizer finding aborts it.  Objects are cached in _build/sanitizer, keyed by
the sources they depend on."""
import concurrent.futures
import hashlib
import os
import shutil
import subprocess

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(REPO, "w4_gemm_gated_amd", "csrc")
INCLUDE = os.path.join(REPO, "include")
TESTS = os.path.join(REPO, "tests")
OUT = os.path.join(REPO, "_build", "sanitizer")
ROCM = "/opt/rocm"
HIPCC = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
SOURCES = ["api.cpp", "plan.cpp", "sched.cpp", "pack.hip", "ec_project.hip", "gemm.hip", "skinny.hip",
           "util.hip", "noalloc.hip", "ec_init.hip"]

# Sanitizers on the host pass of hipcc only, each after -Xarch_host.
HOST_SAN = ["-Xarch_host", "-fsanitize=address",
            "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all",
            "-Xarch_host", "-g"]
HIP_FLAGS = ["-x", "hip", "--offload-arch=gfx950", "-O1", "-fno-omit-frame-pointer", "-std=c++17", "-fPIC",
             "-I", INCLUDE, "-I", CSRC]
# The driver, the C helper and the link are host-only compiles.
HOST_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer",
              "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)),
                                reason="needs the ROCm toolchain (hipcc, clang++)")


def _digest(paths, flags):
    h = hashlib.sha256(" ".join(flags).encode())
    for p in paths:
        with open(p, "rb") as f:
            h.update(p.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _headers():
    hs = [os.path.join(CSRC, n) for n in sorted(os.listdir(CSRC)) if n.endswith(".h")]
    return hs + [os.path.join(INCLUDE, "spear_w4ec.h")]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
        raise RuntimeError(f"{' '.join(cmd[:3])} ... failed:\n{out[-4000:]}")


def _object(src):
    path = os.path.join(CSRC, src)
    key = _digest([path] + _headers(), HIP_FLAGS + HOST_SAN)
    obj = os.path.join(OUT, f"{src}.{key}.o")
    if not os.path.exists(obj):
        tmp = obj + ".tmp"
        _run([HIPCC, *HIP_FLAGS, *HOST_SAN, "-c", path, "-o", tmp])
        os.replace(tmp, obj)
        for old in os.listdir(OUT):     # objects of earlier versions of this source
            if old.startswith(src + ".") and old.endswith(".o") and os.path.join(OUT, old) != obj:
                os.remove(os.path.join(OUT, old))
    return obj


@pytest.fixture(scope="module")
def driver():
    os.makedirs(OUT, exist_ok=True)
    jobs = max(1, min(len(SOURCES), (os.cpu_count() or 2)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_object, SOURCES))
    drv_o = os.path.join(OUT, "driver.o")
    st_o = os.path.join(OUT, "status.o")
    _run([CLANGXX, *HOST_FLAGS, "-std=c++17", "-I", INCLUDE, "-c",
          os.path.join(TESTS, "sanitizer_driver.cpp"), "-o", drv_o])
    _run([CLANG, *HOST_FLAGS, "-c", os.path.join(TESTS, "sanitizer_status.c"), "-o", st_o])
    exe = os.path.join(OUT, "sanitizer_driver")
    _run([CLANGXX, *HOST_FLAGS, drv_o, st_o, *objs, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe])
    return exe


def test_host_code_is_clean_under_sanitizers(driver):
    env = dict(os.environ)
    # The HIP runtime keeps allocations until exit; leaks are not what is checked.
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    res = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-6000:]
    assert "all checks passed" in out
