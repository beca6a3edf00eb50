"""The accumulation kernels pass partial sums between workgroups through relaxed agent-scope atomic
stores and loads, ordered by the instruction stream: every such store has completed (a
`s_waitcnt vmcnt(0)`) before the arrival counter's atomic add is issued, and the add's returned
count is waited for before the last arriver's loads.  This test compiles accumulate.hip for gfx950
to assembly with the library's own flags and checks that order in every kernel that has a counter;
a listing with the wait removed must fail the same check."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

SCOPED_STORE = re.compile(r"^global_store\S*\s.*\bsc1\b")
SCOPED_LOAD = re.compile(r"^global_load\S*\s.*\bsc1\b")
WAIT_ALL = re.compile(r"^s_waitcnt\b.*\bvmcnt\(0\)")


def kernels(asm: str):
    """(name, instruction list) for every function in an AMDGPU assembly listing."""
    out = []
    for m in re.finditer(r"\n(_ZN2lh\S*?):[^\n]*\n(.*?)\n\.Lfunc_end", asm, re.S):
        ins = []
        for line in m.group(2).splitlines():
            t = line.split(";")[0].strip()
            if t and not t.startswith(".") and not t.endswith(":"):
                ins.append(t)
        out.append((m.group(1), ins))
    return out


def ordering_faults(ins):
    """Faults in straight-line order: an arrival add issued while a scoped store may still be in
    flight, or a scoped load issued after an add before the add's result was waited for."""
    faults = []
    stores_pending = False
    add_pending = False
    for k, t in enumerate(ins):
        if SCOPED_STORE.match(t):
            stores_pending = True
        elif WAIT_ALL.match(t):
            stores_pending = add_pending = False
        elif t.startswith("global_atomic_add"):
            if stores_pending:
                faults.append((k, "counter add issued before the partial stores completed"))
            add_pending = True
        elif SCOPED_LOAD.match(t) and add_pending:
            faults.append((k, "partial load issued before the counter add returned"))
    return faults


@pytest.fixture(scope="module")
def listing():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not installed")
    import sys
    sys.path.insert(0, ROOT)
    from nvfp4_scale_calibration_lh_amd.build import FLAGS
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "accumulate.s")
        src = os.path.join(ROOT, "nvfp4_scale_calibration_lh_amd", "csrc", "accumulate.hip")
        flags = [f for f in FLAGS if f != "-fPIC"]
        p = subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", out], capture_output=True, text=True)
        assert p.returncode == 0, p.stderr[-3000:]
        return open(out).read()


def test_every_counter_add_waits_for_the_partial_stores(listing):
    ks = [(n, ins) for n, ins in kernels(listing) if any(t.startswith("global_atomic_add") for t in ins)]
    assert len(ks) >= 6, "expected the dense, importance-only and grouped kernels to use arrival counters"
    for name, ins in ks:
        assert any(SCOPED_STORE.match(t) for t in ins), f"{name}: partial sums are not stored at agent scope"
        assert any(SCOPED_LOAD.match(t) for t in ins), f"{name}: partial sums are not loaded at agent scope"
        assert not ordering_faults(ins), f"{name}: {ordering_faults(ins)[:3]}"


def test_checker_sees_a_missing_wait(listing):
    name, ins = next((n, i) for n, i in kernels(listing) if any(t.startswith("global_atomic_add") for t in i))
    at = next(k for k, t in enumerate(ins) if t.startswith("global_atomic_add"))
    last_store = max(k for k in range(at) if SCOPED_STORE.match(ins[k]))
    broken = ins[:last_store + 1] + [t for t in ins[last_store + 1:at] if not WAIT_ALL.match(t)] + ins[at:]
    assert ordering_faults(broken), f"{name}: removing the wait before the counter add went unnoticed"
    after = [t for t in ins[at + 1:] if not WAIT_ALL.match(t)]
    if any(SCOPED_LOAD.match(t) for t in after):
        assert ordering_faults(ins[:at + 1] + after)
