"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's sources are compiled as for the library, with the sanitizers on
the host side only, linked with the driver in tests/abi_sanitize/abi_driver.cpp,
and run with no GPU visible, so no kernel can run.  The driver
calls the entry points with valid and invalid arguments, huge sizes, tables of
many descriptors and an injected std::bad_alloc; the sanitizers check the
validation, overlap checks, descriptor tables and error path for memory
errors and undefined behaviour, and the driver checks the statuses.
"""
import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rank_gradient_sketching_logra_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitize")
SOURCES = ["logra_abi.hip", "kernels_sketch.hip", "kernels_merge.hip", "kernels_opt.hip", "kernels_diag.hip",
           "kernels_probe.hip"]
DRIVER = os.path.join(ROOT, "tests", "abi_sanitize", "abi_driver.cpp")
HIPCC = "/opt/rocm/bin/hipcc"
# sanitizers on the host side only (the device side is not compiled at all here)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:  # pragma: no cover
        return False


def _compile(args):
    src, obj, lang = args
    dev = (["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
           if lang == "hip" else [])
    cmd = [HIPCC, "-x", lang, *dev, "-O1", "-g", "-std=c++17", "-fPIC", *SAN,
           "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}{res.stderr}"
    return obj


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.skipif(not glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.a"),
                    reason="no AddressSanitizer runtime for the host compiler")
@pytest.mark.skipif(_gpu_visible(), reason="run where no GPU is visible: the driver uses fake device pointers")
def test_abi_host_code_under_asan_and_ubsan():
    os.makedirs(OUT, exist_ok=True)
    jobs = [(os.path.join(CSRC, s), os.path.join(OUT, s.replace(".hip", ".o")), "hip") for s in SOURCES]
    jobs.append((DRIVER, os.path.join(OUT, "abi_driver.o"), "c++"))
    with ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, jobs))
    exe = os.path.join(OUT, "abi_driver")
    link = [HIPCC, "--offload-arch=gfx950", *SAN, "-o", exe, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    res = subprocess.run(link, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="-1",
               ROCR_VISIBLE_DEVICES="-1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " 0 failed" in run.stdout, out[-4000:]
