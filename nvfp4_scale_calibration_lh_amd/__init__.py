"""Python binding of ``liblh.so``, the MI355X local-Hessian NVFP4 weight-scale calibration library.

The functions carry the names of the C entry points in ``include/lh.h`` and only marshal
arguments: they check dtypes, shapes and devices of torch tensors, allocate missing outputs with
torch, and pass raw device pointers plus torch's current HIP stream to the library.  Every step of
the computation runs in the HIP kernels.  Importing this package fails loudly when the library has
not been built (``python -m nvfp4_scale_calibration_lh_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# The library built next to this file; LH_LIBRARY may name another build of the same library.
LIB_PATH = os.environ.get("LH_LIBRARY") or os.path.join(_PKG, "liblh.so")

LH_OK, LH_ERR_INVALID_ARGUMENT, LH_ERR_UNSUPPORTED, LH_ERR_HIP = 0, 1, 2, 3
LH_DTYPE_F32, LH_DTYPE_BF16 = 0, 1

EXPORTED = ("lh_accumulate", "lh_accumulate_noalloc", "lh_accumulate_act_aware", "lh_accumulate_act_aware_fq", "lh_activation_fake_quant",
            "lh_accumulate_sweep", "lh_dequantize", "lh_dequantize_ex", "lh_scale_sweep", "lh_scale_sweep_ex", "lh_scale_sweep_diag",
            "lh_scale_sweep_diag_ex", "lh_scale_sweep_mse", "lh_absmax", "lh_last_error", "lh_version")
MAX_MULTIPLIERS = 128


class SweepOptions(ctypes.Structure):
    """lh_sweep_options: scale_norm (448 or 256 for "4/6"), the amax multipliers (host array)."""
    _fields_ = [("scale_norm", ctypes.c_float), ("n_multipliers", ctypes.c_int32),
                ("multipliers", ctypes.POINTER(ctypes.c_float))]


class LHError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"liblh error {code}: {message}")
        self.code = code
        self.message = message


_lib_handle = None


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it is missing)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m nvfp4_scale_calibration_lh_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
        h.lh_accumulate.argtypes = [vp, i32, i64, i64, vp, i64, f32, vp, vp, vp]
        h.lh_accumulate_noalloc.argtypes = [vp, i32, i64, i64, vp, i64, f32, vp, vp, vp]
        h.lh_accumulate_act_aware.argtypes = [vp, vp, i32, i64, i64, vp, i64, f32, vp, vp, vp]
        h.lh_accumulate_act_aware_fq.argtypes = [vp, i32, i64, i64, vp, i64, vp, f32, vp, vp, vp]
        h.lh_activation_fake_quant.argtypes = [vp, i32, i64, i64, vp, i64, vp, vp, vp]
        h.lh_scale_sweep.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]
        h.lh_scale_sweep_diag.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, vp, vp, vp]
        h.lh_scale_sweep_ex.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp]
        h.lh_scale_sweep_diag_ex.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]
        h.lh_dequantize_ex.argtypes = [vp, vp, i32, i64, i64, i64, vp, f32, vp, vp, vp]
        h.lh_accumulate_sweep.argtypes = [vp, vp, i32, i64, i64, vp, i64, i64, vp, vp, vp, vp, vp, vp]
        h.lh_scale_sweep_mse.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, vp, vp]
        h.lh_absmax.argtypes = [vp, i32, i64, i64, vp, vp]
        h.lh_dequantize.argtypes = [vp, vp, i32, i64, i64, i64, vp, vp, vp, vp]
        for f in ("lh_accumulate", "lh_accumulate_noalloc", "lh_accumulate_act_aware", "lh_accumulate_act_aware_fq",
                  "lh_activation_fake_quant", "lh_scale_sweep", "lh_scale_sweep_ex", "lh_scale_sweep_diag_ex",
                  "lh_dequantize_ex", "lh_accumulate_sweep",
                  "lh_scale_sweep_diag", "lh_scale_sweep_mse", "lh_absmax", "lh_dequantize"):
            getattr(h, f).restype = ctypes.c_int
        h.lh_last_error.argtypes = []
        h.lh_last_error.restype = ctypes.c_char_p
        h.lh_version.argtypes = []
        h.lh_version.restype = ctypes.c_int
        _lib_handle = h
    return _lib_handle


def lh_last_error() -> str:
    return lib().lh_last_error().decode()


def lh_version() -> int:
    return int(lib().lh_version())


def _check(code: int):
    if code != LH_OK:
        raise LHError(code, lh_last_error())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return LH_DTYPE_BF16
    if t.dtype == torch.float32:
        return LH_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, shape=None, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _offsets(offsets: Optional[torch.Tensor], X: torch.Tensor):
    if offsets is None:
        return None, 1
    _need(offsets, "offsets", dtype=torch.int64)
    return offsets, offsets.numel() - 1


def lh_accumulate(X: torch.Tensor, H: Optional[torch.Tensor] = None, imp: Optional[torch.Tensor] = None,
                  offsets: Optional[torch.Tensor] = None, beta: float = 0.0, *, want_h: bool = True,
                  want_imp: bool = False) -> Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]:
    """Per-block Hessian H [G, cin/16, 16, 16] and importance imp [G, cin] of X [rows, cin]."""
    _need(X, "X")
    rows, cin = X.shape
    offsets, G = _offsets(offsets, X)
    if H is None and want_h:
        H = torch.empty((G, cin // 16, 16, 16), dtype=torch.float32, device=X.device)
    if imp is None and want_imp:
        imp = torch.empty((G, cin), dtype=torch.float32, device=X.device)
    if H is not None:
        _need(H, "H", (G, cin // 16, 16, 16), torch.float32)
    if imp is not None:
        _need(imp, "imp", (G, cin), torch.float32)
    _check(lib().lh_accumulate(_ptr(X), _dtype_code(X), rows, cin, _ptr(offsets), G, float(beta),
                               _ptr(H), _ptr(imp), _stream(X.device)))
    return H, imp


def lh_accumulate_noalloc(X: torch.Tensor, H: torch.Tensor = None, imp: Optional[torch.Tensor] = None,
                          offsets: Optional[torch.Tensor] = None, beta: float = 0.0):
    """lh_accumulate that allocates nothing (no output allocation here either: H and/or imp are
    required), its scratch in the library's fixed per-device array; overlapping calls on one
    device race."""
    _need(X, "X")
    rows, cin = X.shape
    offsets, G = _offsets(offsets, X)
    if H is None and imp is None:
        raise ValueError("H and/or imp must be given")
    if H is not None:
        _need(H, "H", (G, cin // 16, 16, 16), torch.float32)
    if imp is not None:
        _need(imp, "imp", (G, cin), torch.float32)
    _check(lib().lh_accumulate_noalloc(_ptr(X), _dtype_code(X), rows, cin, _ptr(offsets), G, float(beta),
                                       _ptr(H), _ptr(imp), _stream(X.device)))
    return H, imp


def lh_accumulate_act_aware(X: torch.Tensor, Xq: torch.Tensor, H: Optional[torch.Tensor] = None,
                            P: Optional[torch.Tensor] = None, offsets: Optional[torch.Tensor] = None,
                            beta: float = 0.0) -> Tuple[torch.Tensor, torch.Tensor]:
    """H = X_q^T X_q / T and P = X_q^T (X_q - X) / T per 16-channel block."""
    _need(X, "X")
    _need(Xq, "Xq", X.shape, X.dtype)
    rows, cin = X.shape
    offsets, G = _offsets(offsets, X)
    shape = (G, cin // 16, 16, 16)
    if H is None:
        H = torch.empty(shape, dtype=torch.float32, device=X.device)
    if P is None:
        P = torch.empty(shape, dtype=torch.float32, device=X.device)
    _need(H, "H", shape, torch.float32)
    _need(P, "P", shape, torch.float32)
    _check(lib().lh_accumulate_act_aware(_ptr(X), _ptr(Xq), _dtype_code(X), rows, cin, _ptr(offsets), G,
                                         float(beta), _ptr(H), _ptr(P), _stream(X.device)))
    return H, P


def lh_accumulate_act_aware_fq(X: torch.Tensor, x_amax: torch.Tensor, H: Optional[torch.Tensor] = None,
                               P: Optional[torch.Tensor] = None, offsets: Optional[torch.Tensor] = None,
                               beta: float = 0.0) -> Tuple[torch.Tensor, torch.Tensor]:
    """As lh_accumulate_act_aware, with X_q the NVFP4 fake-quant of X made in the kernel from the
    input quantizer's amax per group (x_amax [G] fp32)."""
    _need(X, "X")
    rows, cin = X.shape
    offsets, G = _offsets(offsets, X)
    _need(x_amax, "x_amax", (G,), torch.float32)
    shape = (G, cin // 16, 16, 16)
    if H is None:
        H = torch.empty(shape, dtype=torch.float32, device=X.device)
    if P is None:
        P = torch.empty(shape, dtype=torch.float32, device=X.device)
    _need(H, "H", shape, torch.float32)
    _need(P, "P", shape, torch.float32)
    _check(lib().lh_accumulate_act_aware_fq(_ptr(X), _dtype_code(X), rows, cin, _ptr(offsets), G, _ptr(x_amax),
                                            float(beta), _ptr(H), _ptr(P), _stream(X.device)))
    return H, P


def lh_activation_fake_quant(X: torch.Tensor, x_amax: torch.Tensor, Xq: Optional[torch.Tensor] = None,
                             offsets: Optional[torch.Tensor] = None) -> torch.Tensor:
    """X_q [rows, cin]: the NVFP4 fake-quant of X with the input quantizer's amax per group
    (x_amax [G] fp32), as lh_accumulate_act_aware_fq applies it inside its kernel."""
    _need(X, "X")
    rows, cin = X.shape
    offsets, G = _offsets(offsets, X)
    _need(x_amax, "x_amax", (G,), torch.float32)
    if Xq is None:
        Xq = torch.empty_like(X)
    _need(Xq, "Xq", X.shape, X.dtype)
    _check(lib().lh_activation_fake_quant(_ptr(X), _dtype_code(X), rows, cin, _ptr(offsets), G, _ptr(x_amax),
                                          _ptr(Xq), _stream(X.device)))
    return Xq


def _sweep_outputs(W, code, fp4, loss, want_fp4, want_loss):
    G, cout, cin = W.shape
    dev = W.device
    if code is None:
        code = torch.empty((G, cout, cin // 16), dtype=torch.uint8, device=dev)
    if fp4 is None and want_fp4:
        fp4 = torch.empty((G, cout, cin // 2), dtype=torch.uint8, device=dev)
    if loss is None and want_loss:
        loss = torch.empty((G, cout, cin // 16), dtype=torch.float32, device=dev)
    _need(code, "code", (G, cout, cin // 16), torch.uint8)
    if fp4 is not None:
        _need(fp4, "fp4", (G, cout, cin // 2), torch.uint8)
    if loss is not None:
        _need(loss, "loss", (G, cout, cin // 16), torch.float32)
    return code, fp4, loss


def _as3d(W: torch.Tensor) -> torch.Tensor:
    return W.unsqueeze(0) if W.dim() == 2 else W


def lh_scale_sweep(W: torch.Tensor, amax: torch.Tensor, H: torch.Tensor, P: Optional[torch.Tensor] = None,
                   code: Optional[torch.Tensor] = None, fp4: Optional[torch.Tensor] = None,
                   loss: Optional[torch.Tensor] = None, *, want_fp4: bool = True, want_loss: bool = True):
    """126-candidate E4M3 scale sweep scored by e^T H e + 2 e^T (P w): (code, fp4, loss)."""
    W = _as3d(W)
    _need(W, "W")
    G, cout, cin = W.shape
    _need(amax, "amax", (G,), torch.float32)
    _need(H, "H", (G, cin // 16, 16, 16), torch.float32)
    if P is not None:
        _need(P, "P", (G, cin // 16, 16, 16), torch.float32)
    code, fp4, loss = _sweep_outputs(W, code, fp4, loss, want_fp4, want_loss)
    _check(lib().lh_scale_sweep(_ptr(W), _dtype_code(W), G, cout, cin, _ptr(amax), _ptr(H), _ptr(P),
                                _ptr(code), _ptr(fp4), _ptr(loss), _stream(W.device)))
    return code, fp4, loss


def lh_scale_sweep_diag(W: torch.Tensor, amax: torch.Tensor, imp: torch.Tensor,
                        code: Optional[torch.Tensor] = None, fp4: Optional[torch.Tensor] = None,
                        loss: Optional[torch.Tensor] = None, *, want_fp4: bool = True, want_loss: bool = True):
    """126-candidate E4M3 scale sweep scored by sum_i imp_i e_i^2: (code, fp4, loss)."""
    W = _as3d(W)
    _need(W, "W")
    G, cout, cin = W.shape
    _need(amax, "amax", (G,), torch.float32)
    _need(imp, "imp", (G, cin), torch.float32)
    code, fp4, loss = _sweep_outputs(W, code, fp4, loss, want_fp4, want_loss)
    _check(lib().lh_scale_sweep_diag(_ptr(W), _dtype_code(W), G, cout, cin, _ptr(amax), _ptr(imp),
                                     _ptr(code), _ptr(fp4), _ptr(loss), _stream(W.device)))
    return code, fp4, loss


def lh_scale_sweep_mse(W: torch.Tensor, amax: torch.Tensor, code: Optional[torch.Tensor] = None,
                       fp4: Optional[torch.Tensor] = None, loss: Optional[torch.Tensor] = None, *,
                       want_fp4: bool = True, want_loss: bool = True):
    """126-candidate E4M3 scale sweep scored by the plain sum_i e_i^2: (code, fp4, loss)."""
    W = _as3d(W)
    _need(W, "W")
    G, cout, cin = W.shape
    _need(amax, "amax", (G,), torch.float32)
    code, fp4, loss = _sweep_outputs(W, code, fp4, loss, want_fp4, want_loss)
    _check(lib().lh_scale_sweep_mse(_ptr(W), _dtype_code(W), G, cout, cin, _ptr(amax),
                                    _ptr(code), _ptr(fp4), _ptr(loss), _stream(W.device)))
    return code, fp4, loss


def _options(norm: float, multipliers):
    """(ctypes options, keep-alive array) for the *_ex entry points."""
    import array
    m = array.array("f", [] if multipliers is None else [float(x) for x in multipliers])
    buf = (ctypes.c_float * max(1, len(m)))(*m) if len(m) else None
    opt = SweepOptions(float(norm), len(m), ctypes.cast(buf, ctypes.POINTER(ctypes.c_float)) if buf else None)
    return opt, buf


def lh_scale_sweep_ex(W: torch.Tensor, amax: torch.Tensor, H: torch.Tensor, P: Optional[torch.Tensor] = None,
                      code: Optional[torch.Tensor] = None, fp4: Optional[torch.Tensor] = None,
                      loss: Optional[torch.Tensor] = None, *, norm: float = 448.0, multipliers=None,
                      want_fp4: bool = True, want_loss: bool = True):
    """lh_scale_sweep with the global scale normalized to `norm` (448, or 256 for "4/6") and, when
    `multipliers` is given (at most 128 positive values), the amax-multiplier search."""
    W = _as3d(W)
    _need(W, "W")
    G, cout, cin = W.shape
    _need(amax, "amax", (G,), torch.float32)
    _need(H, "H", (G, cin // 16, 16, 16), torch.float32)
    if P is not None:
        _need(P, "P", (G, cin // 16, 16, 16), torch.float32)
    code, fp4, loss = _sweep_outputs(W, code, fp4, loss, want_fp4, want_loss)
    opt, keep = _options(norm, multipliers)
    _check(lib().lh_scale_sweep_ex(_ptr(W), _dtype_code(W), G, cout, cin, _ptr(amax), _ptr(H), _ptr(P),
                                   ctypes.byref(opt), _ptr(code), _ptr(fp4), _ptr(loss), _stream(W.device)))
    del keep
    return code, fp4, loss


def lh_accumulate_sweep(X: torch.Tensor, W: torch.Tensor, amax: torch.Tensor, offsets: Optional[torch.Tensor] = None,
                        code: Optional[torch.Tensor] = None, fp4: Optional[torch.Tensor] = None,
                        loss: Optional[torch.Tensor] = None, *, norm: float = 448.0, multipliers=None,
                        want_fp4: bool = True, want_loss: bool = True):
    """Per-expert Hessians of X's grouped rows and the scale search of W [G, cout, cin] against
    them in one launch, H never written to memory: (code, fp4, loss) as lh_scale_sweep_ex."""
    _need(X, "X")
    W = _as3d(W)
    _need(W, "W")
    rows, cin = X.shape
    offsets, G = _offsets(offsets, X)
    if W.shape[0] != G or W.shape[2] != cin or W.dtype != X.dtype:
        raise ValueError(f"W must be [{G}, cout, {cin}] of X's dtype")
    _need(amax, "amax", (G,), torch.float32)
    code, fp4, loss = _sweep_outputs(W, code, fp4, loss, want_fp4, want_loss)
    opt, keep = _options(norm, multipliers)
    _check(lib().lh_accumulate_sweep(_ptr(X), _ptr(W), _dtype_code(X), rows, cin, _ptr(offsets), G, W.shape[1],
                                     _ptr(amax), ctypes.byref(opt), _ptr(code), _ptr(fp4), _ptr(loss),
                                     _stream(X.device)))
    del keep
    return code, fp4, loss


def lh_scale_sweep_diag_ex(W: torch.Tensor, amax: torch.Tensor, imp: Optional[torch.Tensor],
                           code: Optional[torch.Tensor] = None, fp4: Optional[torch.Tensor] = None,
                           loss: Optional[torch.Tensor] = None, *, norm: float = 448.0, multipliers=None,
                           want_fp4: bool = True, want_loss: bool = True):
    """lh_scale_sweep_diag (imp None: plain MSE) with the options of lh_scale_sweep_ex."""
    W = _as3d(W)
    _need(W, "W")
    G, cout, cin = W.shape
    _need(amax, "amax", (G,), torch.float32)
    if imp is not None:
        _need(imp, "imp", (G, cin), torch.float32)
    code, fp4, loss = _sweep_outputs(W, code, fp4, loss, want_fp4, want_loss)
    opt, keep = _options(norm, multipliers)
    _check(lib().lh_scale_sweep_diag_ex(_ptr(W), _dtype_code(W), G, cout, cin, _ptr(amax), _ptr(imp),
                                        ctypes.byref(opt), _ptr(code), _ptr(fp4), _ptr(loss), _stream(W.device)))
    del keep
    return code, fp4, loss


def lh_dequantize(code: torch.Tensor, fp4: torch.Tensor, amax: torch.Tensor, dtype: torch.dtype = torch.bfloat16,
                  Wq: Optional[torch.Tensor] = None, block_amax: Optional[torch.Tensor] = None,
                  want_wq: bool = True, want_block_amax: bool = True, norm: float = 448.0):
    """Fake-quantized weights Wq [G, cout, cin] (bf16 or fp32) and per-block amax [G, cout, cin/16]
    from the sweep's scale codes and FP4 nibbles (norm: the sweep's scale normalization, through
    lh_dequantize_ex when it is not 448)."""
    if code.dim() != 3:
        raise ValueError("code must be [G, cout, cin/16]")
    G, cout, nb = code.shape
    cin = nb * 16
    _need(code, "code", (G, cout, nb), torch.uint8)
    _need(fp4, "fp4", (G, cout, cin // 2), torch.uint8)
    _need(amax, "amax", (G,), torch.float32)
    if dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("dtype must be torch.bfloat16 or torch.float32")
    if Wq is None and want_wq:
        Wq = torch.empty((G, cout, cin), dtype=dtype, device=code.device)
    if block_amax is None and want_block_amax:
        block_amax = torch.empty((G, cout, nb), dtype=torch.float32, device=code.device)
    if Wq is not None:
        _need(Wq, "Wq", (G, cout, cin), dtype)
    if block_amax is not None:
        _need(block_amax, "block_amax", (G, cout, nb), torch.float32)
    if norm == 448.0:
        _check(lib().lh_dequantize(_ptr(code), _ptr(fp4), 1 if dtype == torch.bfloat16 else 0, G, cout, cin,
                                   _ptr(amax), _ptr(Wq), _ptr(block_amax), _stream(code.device)))
    else:
        _check(lib().lh_dequantize_ex(_ptr(code), _ptr(fp4), 1 if dtype == torch.bfloat16 else 0, G, cout, cin,
                                      _ptr(amax), float(norm), _ptr(Wq), _ptr(block_amax), _stream(code.device)))
    return Wq, block_amax


def lh_absmax(W: torch.Tensor, amax: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-group max |W| for W [G, ...] (a 2-D W is one group)."""
    W = _as3d(W) if W.dim() == 2 else W
    _need(W, "W")
    G = W.shape[0]
    per = W.numel() // G if G else 0
    if amax is None:
        amax = torch.empty((G,), dtype=torch.float32, device=W.device)
    _need(amax, "amax", (G,), torch.float32)
    _check(lib().lh_absmax(_ptr(W), _dtype_code(W), G, per, _ptr(amax), _stream(W.device)))
    return amax
