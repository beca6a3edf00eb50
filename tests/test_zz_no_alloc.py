"""The allocation-free accumulation (lh_accumulate_noalloc) against lh_accumulate through the C ABI:
two calls in a row on the library's fixed scratch array, the second with a smaller input, each
bit-identical to the pool-backed entry point; dense and grouped rows, H and importance, beta; a
request beyond the array's size is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

lh = pytest.importorskip("nvfp4_scale_calibration_lh_amd")
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def note(msg):
    print(f"[case] {msg}", flush=True)


def dev(a, bf16=True):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(torch.bfloat16) if bf16 else t).to(DEV)


def _pair(X, off, want_h=True, want_imp=True, beta=0.0, prev=None):
    """(noalloc H, imp), (lh_accumulate H, imp) for the same inputs, through the C entry points."""
    rows, cin = X.shape
    G = 1 if off is None else off.numel() - 1
    L = lh.lib()
    outs = []
    for fn in (L.lh_accumulate_noalloc, L.lh_accumulate):
        H = torch.empty((G, cin // 16, 16, 16), dtype=torch.float32, device=DEV) if want_h else None
        imp = torch.empty((G, cin), dtype=torch.float32, device=DEV) if want_imp else None
        if prev is not None:
            if H is not None:
                H.copy_(prev[0])
            if imp is not None:
                imp.copy_(prev[1])
        st = lh._stream(DEV)
        code = fn(ctypes.c_void_p(X.data_ptr()), lh._dtype_code(X), rows, cin,
                  None if off is None else ctypes.c_void_p(off.data_ptr()), G, ctypes.c_float(beta),
                  None if H is None else ctypes.c_void_p(H.data_ptr()),
                  None if imp is None else ctypes.c_void_p(imp.data_ptr()), st)
        assert code == lh.LH_OK, lh.lh_last_error()
        outs.append((H, imp))
    torch.cuda.synchronize()
    return outs


def _same(a, b):
    for x, y in zip(a, b):
        assert (x is None) == (y is None)
        if x is not None:
            assert torch.equal(x.view(torch.int32), y.view(torch.int32))


def test_noalloc_grouped_then_smaller():
    big = synth.make("c5", n_groups=40, cout=1, cin=256, tokens=3000, topk=4)
    small = synth.make("c5", n_groups=9, cout=1, cin=64, tokens=300, topk=2)
    for wl in (big, small):                      # the second call is smaller and reuses the array
        note(f"allocation-free accumulate, grouped X{wl.X.shape} G={wl.n_groups}")
        X, off = dev(wl.X), torch.from_numpy(wl.offsets).to(DEV)
        a, b = _pair(X, off)
        _same(a, b)
        a, b = _pair(X, off, want_h=False)
        _same(a, b)


def test_noalloc_dense_then_smaller_and_beta():
    big = synth.make("c2", cout=1, cin=512, rows=6000)
    small = synth.make("c2", cout=1, cin=48, rows=333)
    for wl in (big, small):
        note(f"allocation-free accumulate, dense X{wl.X.shape}")
        X = dev(wl.X)
        a, b = _pair(X, None)
        _same(a, b)
        a2, b2 = _pair(X, None, beta=0.5, prev=b)
        _same(a2, b2)
    c1 = synth.make("c1")                          # fp32 activations
    note("allocation-free accumulate, dense fp32")
    a, b = _pair(dev(c1.X, bf16=False), None)
    _same(a, b)


def test_noalloc_refuses_oversized_request():
    """A grouped layer whose partial sums would not fit the fixed array is refused with
    INVALID_ARGUMENT before anything is launched (no allocation is attempted)."""
    X = torch.empty((4, 16), dtype=torch.bfloat16, device=DEV)
    H = torch.empty((2, 4096 // 16, 16, 16), dtype=torch.float32, device=DEV)
    off = torch.tensor([0, 2, 4], dtype=torch.int64, device=DEV)
    L = lh.lib()
    # 2^27 rows x 4096 channels (not read: the check happens first)
    code = L.lh_accumulate_noalloc(ctypes.c_void_p(X.data_ptr()), lh.LH_DTYPE_BF16, 1 << 27, 4096,
                                   ctypes.c_void_p(off.data_ptr()), 2, ctypes.c_float(0.0),
                                   ctypes.c_void_p(H.data_ptr()), None, lh._stream(DEV))
    assert code == lh.LH_ERR_INVALID_ARGUMENT and "scratch" in lh.lh_last_error()
