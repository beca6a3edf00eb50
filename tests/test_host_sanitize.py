"""The library's host code (argument checks, device guard, option parsing, error strings) built with
AddressSanitizer and UndefinedBehaviorSanitizer, driven through every check that needs no GPU by
tests/host/abi_checks.cpp.  The kernels are compiled as usual; only the host side is instrumented
(hipcc's -Xarch_host), so this runs on a machine without a GPU."""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "nvfp4_scale_calibration_lh_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
KERNELS = ["absmax.hip", "accumulate.hip", "sweep.hip", "dequant.hip"]
sys.path.insert(0, ROOT)
from nvfp4_scale_calibration_lh_amd.build import FLAGS  # noqa: E402  (the library's own compile flags)

COMMON = ["-O1", "-g"] + [f for f in FLAGS if f not in ("-O3", "-Wall")]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    p = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{p.stdout[-3000:]}\n{p.stderr[-3000:]}"
    return p


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is not installed")
def test_host_code_under_address_and_undefined_behavior_sanitizers():
    with tempfile.TemporaryDirectory() as d:
        objs = []
        for src in KERNELS:
            o = os.path.join(d, src + ".o")
            _run([HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", o])
            objs.append(o)
        abi = os.path.join(d, "lh_abi.o")
        _run([HIPCC, *COMMON, *SAN, "-x", "hip", "-c", os.path.join(CSRC, "lh_abi.cpp"), "-o", abi])
        drv = os.path.join(d, "abi_checks.o")
        _run([HIPCC, *COMMON, *SAN, "-c", os.path.join(ROOT, "tests", "host", "abi_checks.cpp"), "-o", drv])
        exe = os.path.join(d, "abi_checks")
        _run([HIPCC, "--offload-arch=gfx950", *SAN, drv, abi, *objs, "-o", exe])
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
                   HIP_VISIBLE_DEVICES=os.environ.get("HIP_VISIBLE_DEVICES", ""))
        p = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        assert p.returncode == 0, f"{p.stdout[-3000:]}\n{p.stderr[-5000:]}"
        assert "ok: 0 failures" in p.stdout
        assert "runtime error" not in p.stderr and "AddressSanitizer" not in p.stderr
