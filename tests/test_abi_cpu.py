"""The C ABI library loads, exports every entry point of include/lh.h, and rejects bad arguments
before touching a device (no compute calls here: this suite runs without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lh.h")

lh = pytest.importorskip("nvfp4_scale_calibration_lh_amd")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lh_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("lh_accumulate", "lh_accumulate_act_aware", "lh_accumulate_act_aware_fq",
              "lh_activation_fake_quant", "lh_scale_sweep", "lh_scale_sweep_ex", "lh_scale_sweep_diag_ex",
              "lh_dequantize_ex", "lh_accumulate_sweep",
              "lh_scale_sweep_diag", "lh_scale_sweep_mse", "lh_dequantize", "lh_absmax", "lh_last_error",
              "lh_version"):
        assert n in names
    assert set(names) == set(lh.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = lh.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    want = int(re.search(r"#define LH_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lh.lh_version() == want


VP = ctypes.c_void_p
FAKE = VP(0x1000)        # a non-null address that is not device memory


def _err(code):
    return code, lh.lh_last_error()


def test_validation_errors_without_device():
    L = lh.lib()
    # unknown dtype
    c, m = _err(L.lh_accumulate(FAKE, 7, 10, 32, None, 1, 0.0, FAKE, None, None))
    assert c == lh.LH_ERR_UNSUPPORTED and "dtype" in m
    # cin not a multiple of 16
    c, m = _err(L.lh_accumulate(FAKE, lh.LH_DTYPE_BF16, 10, 40, None, 1, 0.0, FAKE, None, None))
    assert c == lh.LH_ERR_INVALID_ARGUMENT and "cin" in m
    # negative rows, n_groups < 1, missing offsets for several groups
    assert L.lh_accumulate(FAKE, 1, -1, 32, None, 1, 0.0, FAKE, None, None) == lh.LH_ERR_INVALID_ARGUMENT
    assert L.lh_accumulate(FAKE, 1, 10, 32, None, 0, 0.0, FAKE, None, None) == lh.LH_ERR_INVALID_ARGUMENT
    c, m = _err(L.lh_accumulate(FAKE, 1, 10, 32, None, 3, 0.0, FAKE, None, None))
    assert c == lh.LH_ERR_INVALID_ARGUMENT and "group_offsets" in m
    # activation fake-quant: x_amax required, Xq required, no aliasing, host memory rejected
    c, m = _err(L.lh_activation_fake_quant(FAKE, 1, 10, 32, None, 1, None, VP(0x2000), None))
    assert c == lh.LH_ERR_INVALID_ARGUMENT and "x_amax" in m
    assert L.lh_activation_fake_quant(FAKE, 1, 10, 32, None, 1, FAKE, None, None) == lh.LH_ERR_INVALID_ARGUMENT
    c, m = _err(L.lh_activation_fake_quant(FAKE, 1, 10, 32, None, 1, VP(0x3000), FAKE, None))
    assert c == lh.LH_ERR_INVALID_ARGUMENT and "alias" in m
    assert L.lh_activation_fake_quant(FAKE, 9, 10, 32, None, 1, FAKE, FAKE, None) == lh.LH_ERR_UNSUPPORTED
    # sweep options: scale_norm must be an E4M3 value, at most 128 positive finite multipliers
    def opt(norm, mults):
        arr = (ctypes.c_float * max(1, len(mults)))(*mults)
        return lh.SweepOptions(norm, len(mults), ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))), arr
    for o_, msg in ((opt(300.0, []), "scale_norm"), (opt(0.0, []), "scale_norm"), (opt(448.0, [1.0, -2.0]), "multiplier"),
                    (opt(256.0, [float("nan")]), "multiplier"), (opt(448.0, [1.0] * 129), "n_multipliers")):
        c, m = _err(L.lh_scale_sweep_ex(FAKE, 1, 1, 16, 32, FAKE, FAKE, None, ctypes.byref(o_[0]), FAKE, None, None, None))
        assert c == lh.LH_ERR_INVALID_ARGUMENT and msg in m, (c, m)
        c, m = _err(L.lh_scale_sweep_diag_ex(FAKE, 1, 1, 16, 32, FAKE, None, ctypes.byref(o_[0]), FAKE, None, None, None))
        assert c == lh.LH_ERR_INVALID_ARGUMENT and msg in m, (c, m)
    c, m = _err(L.lh_dequantize_ex(FAKE, FAKE, 1, 1, 16, 32, FAKE, 100.0, FAKE, None, None))
    assert c == lh.LH_ERR_INVALID_ARGUMENT and "scale_norm" in m
    nul = lh.SweepOptions(448.0, 3, None)
    c, m = _err(L.lh_scale_sweep_ex(FAKE, 1, 1, 16, 32, FAKE, FAKE, None, ctypes.byref(nul), FAKE, None, None, None))
    assert c == lh.LH_ERR_INVALID_ARGUMENT and "multipliers" in m
    # fused accumulate-and-sweep: cout limit, offsets for several groups, options checked
    c, m = _err(L.lh_accumulate_sweep(FAKE, FAKE, 1, 10, 32, FAKE, 2, 9000, FAKE, None, FAKE, None, None, None))
    assert c == lh.LH_ERR_INVALID_ARGUMENT and "8192" in m
    c, m = _err(L.lh_accumulate_sweep(FAKE, FAKE, 1, 10, 32, None, 2, 16, FAKE, None, FAKE, None, None, None))
    assert c == lh.LH_ERR_INVALID_ARGUMENT and "group_offsets" in m
    bad = lh.SweepOptions(300.0, 0, None)
    c, m = _err(L.lh_accumulate_sweep(FAKE, FAKE, 1, 10, 32, FAKE, 2, 16, FAKE, ctypes.byref(bad), FAKE, None, None, None))
    assert c == lh.LH_ERR_INVALID_ARGUMENT and "scale_norm" in m
    # no outputs, NULL input
    assert L.lh_accumulate(FAKE, 1, 10, 32, None, 1, 0.0, None, None, None) == lh.LH_ERR_INVALID_ARGUMENT
    assert L.lh_accumulate(None, 1, 10, 32, None, 1, 0.0, FAKE, None, None) == lh.LH_ERR_INVALID_ARGUMENT
    # act-aware needs both outputs
    assert L.lh_accumulate_act_aware(FAKE, FAKE, 1, 10, 32, None, 1, 0.0, FAKE, None, None) == lh.LH_ERR_INVALID_ARGUMENT
    # act-aware with X_q made in the kernel: x_amax, H and P required
    c, m = _err(L.lh_accumulate_act_aware_fq(FAKE, 1, 10, 32, None, 1, None, 0.0, FAKE, FAKE, None))
    assert c == lh.LH_ERR_INVALID_ARGUMENT and "x_amax" in m
    assert L.lh_accumulate_act_aware_fq(FAKE, 1, 10, 32, None, 1, FAKE, 0.0, FAKE, None, None) == lh.LH_ERR_INVALID_ARGUMENT
    assert L.lh_accumulate_act_aware_fq(FAKE, 1, 10, 40, None, 1, FAKE, 0.0, FAKE, FAKE, None) == lh.LH_ERR_INVALID_ARGUMENT
    assert L.lh_accumulate_act_aware_fq(FAKE, 5, 10, 32, None, 1, FAKE, 0.0, FAKE, FAKE, None) == lh.LH_ERR_UNSUPPORTED
    # dequantize: codes and amax required, at least one output, fp4 with Wq
    c, m = _err(L.lh_dequantize(None, FAKE, 1, 1, 4, 32, FAKE, FAKE, None, None))
    assert c == lh.LH_ERR_INVALID_ARGUMENT and "scale_code" in m
    assert L.lh_dequantize(FAKE, FAKE, 1, 1, 4, 32, FAKE, None, None, None) == lh.LH_ERR_INVALID_ARGUMENT
    assert L.lh_dequantize(FAKE, None, 1, 1, 4, 32, FAKE, FAKE, None, None) == lh.LH_ERR_INVALID_ARGUMENT
    assert L.lh_dequantize(FAKE, FAKE, 1, 1, 4, 40, FAKE, FAKE, None, None) == lh.LH_ERR_INVALID_ARGUMENT
    assert L.lh_dequantize(FAKE, FAKE, 7, 1, 4, 32, FAKE, FAKE, None, None) == lh.LH_ERR_UNSUPPORTED
    # sweep
    assert L.lh_scale_sweep(FAKE, 1, 0, 4, 32, FAKE, FAKE, None, FAKE, None, None, None) == lh.LH_ERR_INVALID_ARGUMENT
    assert L.lh_scale_sweep(FAKE, 1, 1, 4, 33, FAKE, FAKE, None, FAKE, None, None, None) == lh.LH_ERR_INVALID_ARGUMENT
    assert L.lh_scale_sweep(FAKE, 1, 65536, 4, 32, FAKE, FAKE, None, FAKE, None, None, None) == lh.LH_ERR_INVALID_ARGUMENT
    assert L.lh_scale_sweep(FAKE, 1, 1, 65535 * 32 + 1, 32, FAKE, FAKE, None, FAKE, None, None, None) == lh.LH_ERR_INVALID_ARGUMENT
    assert L.lh_scale_sweep_diag(FAKE, 1, 1, -1, 32, FAKE, FAKE, FAKE, None, None, None) == lh.LH_ERR_INVALID_ARGUMENT
    assert L.lh_scale_sweep(FAKE, 1, 1, 4, 32, None, FAKE, None, FAKE, None, None, None) == lh.LH_ERR_INVALID_ARGUMENT
    assert L.lh_scale_sweep(FAKE, 9, 1, 4, 32, FAKE, FAKE, None, FAKE, None, None, None) == lh.LH_ERR_UNSUPPORTED
    assert L.lh_scale_sweep_diag(FAKE, 1, 1, 4, 32, FAKE, None, FAKE, None, None, None) == lh.LH_ERR_INVALID_ARGUMENT
    # plain-MSE sweep: no importance argument; amax and codes required, shapes as the others
    c, m = _err(L.lh_scale_sweep_mse(FAKE, 1, 1, 4, 32, None, FAKE, None, None, None))
    assert c == lh.LH_ERR_INVALID_ARGUMENT and "global_amax" in m
    assert L.lh_scale_sweep_mse(FAKE, 1, 1, 4, 32, FAKE, None, None, None, None) == lh.LH_ERR_INVALID_ARGUMENT
    assert L.lh_scale_sweep_mse(FAKE, 1, 1, 4, 40, FAKE, FAKE, None, None, None) == lh.LH_ERR_INVALID_ARGUMENT
    assert L.lh_scale_sweep_mse(FAKE, 1, 0, 4, 32, FAKE, FAKE, None, None, None) == lh.LH_ERR_INVALID_ARGUMENT
    assert L.lh_scale_sweep_mse(FAKE, 9, 1, 4, 32, FAKE, FAKE, None, None, None) == lh.LH_ERR_UNSUPPORTED
    assert L.lh_absmax(FAKE, 1, 0, 10, FAKE, None) == lh.LH_ERR_INVALID_ARGUMENT
    assert L.lh_absmax(FAKE, 1, 1, -1, FAKE, None) == lh.LH_ERR_INVALID_ARGUMENT


def test_host_pointer_is_rejected_not_dereferenced():
    L = lh.lib()
    buf = (ctypes.c_float * 64)()
    out = (ctypes.c_float * 4)()
    c, m = _err(L.lh_absmax(ctypes.cast(buf, VP), lh.LH_DTYPE_F32, 1, 64, ctypes.cast(out, VP), None))
    assert c == lh.LH_ERR_INVALID_ARGUMENT, (c, m)
    assert "W" in m
    c, m = _err(L.lh_accumulate(ctypes.cast(buf, VP), lh.LH_DTYPE_F32, 4, 16, None, 1, 0.0,
                                ctypes.cast(out, VP), None, None))
    assert c == lh.LH_ERR_INVALID_ARGUMENT


def test_binding_checks_shapes_before_calling():
    import torch
    with pytest.raises(ValueError):
        lh.lh_accumulate(torch.zeros((4, 16)))          # CPU tensor
    with pytest.raises(TypeError):
        lh._dtype_code(torch.zeros(2, dtype=torch.float16))
