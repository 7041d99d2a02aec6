"""The C ABI's host-side validation layer under AddressSanitizer and
UndefinedBehaviorSanitizer (on the CPU, no GPU needed).

``muon_abi.hip`` is compiled with both sanitizers on its host code only
(``-Xarch_host`` before each ``-fsanitize=``; the kernels are built as
usual) and linked into ``abi_validation_driver.cpp``, which calls every
entry point with invalid arguments, overflowing shapes and sizes, overlapping
buffers, more groups than one launch sequence takes and empty batches:
every such call returns before the first HIP call.  Any sanitizer report
(out-of-bounds access, signed overflow, ...) aborts the driver."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "muon_step_03_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]
BASE = ["--offload-arch=gfx950", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
        "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.timeout(600)
def test_validation_layer_under_asan_and_ubsan(tmp_path):
    jobs = [(os.path.join(CSRC, "muon_abi.hip"), ["-O1", "-g"] + SAN),
            (os.path.join(ROOT, "tests", "abi_validation_driver.cpp"), ["-O1", "-g"] + SAN)]
    jobs += [(os.path.join(CSRC, f), ["-O3"]) for f in
             ("k_elementwise.hip", "k_ns_bf16.hip", "k_ns_f32.hip", "k_adamw.hip")]

    def compile_one(job):
        src, flags = job
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, *BASE, *flags, "-c", src, "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, jobs))
    exe = str(tmp_path / "abi_validation_driver")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN[:4], *objs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ALL_VALIDATION_CASES_OK" in r.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
