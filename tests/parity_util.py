"""Shared comparison rules for the GPU-vs-oracle parity tests.

Tolerances (relative 1e-5 for fp32 accumulation, bit-exact codes outside near-ties):
  H:    |dH_ij| <= 1e-5 * sqrt(H_ii H_jj)            (entrywise Cauchy-Schwarz scale)
  P:    |dP_ij| <= 1e-5 * sqrt(H_ii R_jj), R = D^T D / T, D = X_q - X
  imp:  |dImp_i| <= 1e-5 * Imp_i
  loss: |dL| <= 1e-5 * (Q + |C|) of the winning candidate
  codes and FP4 nibbles: identical, except on blocks whose two best float64 losses differ by at
  most 1e-6 * max(Q + |C|) (oracle.exempt_mask).
Plain elementwise relative error is meaningless for near-zero off-diagonal entries, hence the
Cauchy-Schwarz scales.
"""
import numpy as np

import oracle

REL = 1e-5


def assert_h_close(H_gpu, H_ref, rel=REL):
    H_gpu = np.asarray(H_gpu, dtype=np.float64)
    d = np.sqrt(np.maximum(np.einsum("...ii->...i", H_ref), 0.0))
    tol = rel * d[..., :, None] * d[..., None, :] + 1e-30
    bad = np.abs(H_gpu - H_ref) > tol
    assert not bad.any(), f"{bad.sum()} H entries outside tolerance; worst ratio {(np.abs(H_gpu - H_ref) / tol).max():.3g}"


def assert_p_close(P_gpu, P_ref, H_ref, R_ref, rel=REL):
    P_gpu = np.asarray(P_gpu, dtype=np.float64)
    dh = np.sqrt(np.maximum(np.einsum("...ii->...i", H_ref), 0.0))
    dr = np.sqrt(np.maximum(np.einsum("...ii->...i", R_ref), 0.0))
    tol = rel * dh[..., :, None] * dr[..., None, :] + 1e-30
    bad = np.abs(P_gpu - P_ref) > tol
    assert not bad.any(), f"{bad.sum()} P entries outside tolerance; worst ratio {(np.abs(P_gpu - P_ref) / tol).max():.3g}"


def assert_imp_close(imp_gpu, imp_ref, rel=REL):
    imp_gpu = np.asarray(imp_gpu, dtype=np.float64)
    tol = rel * np.abs(imp_ref) + 1e-30
    bad = np.abs(imp_gpu - imp_ref) > tol
    assert not bad.any(), f"{bad.sum()} importance entries outside tolerance"


def cross_gram(X, Xq, offsets):
    """R_g[n] = D^T D / T per block (D = X_q - X), the scale for P's tolerance."""
    D = np.asarray(Xq, dtype=np.float64) - np.asarray(X, dtype=np.float64)
    R, _ = oracle.accumulate(D, offsets)
    return R


def assert_sweep_match(code, fp4, loss, res, allow_exempt=True):
    """code [..., nb], fp4 [..., cin/2], loss [..., nb] from the GPU vs an oracle sweep result."""
    code = np.asarray(code)
    exempt = oracle.exempt_mask(res) if allow_exempt else np.zeros(code.shape, dtype=bool)
    bad = (code != res["code"]) & ~exempt
    assert not bad.any(), (f"{bad.sum()} of {code.size} scale codes differ outside near-ties; first "
                           f"{np.argwhere(bad)[:3].tolist()} gpu {code[bad][:5]} oracle {res['code'][bad][:5]}")
    if fp4 is not None:
        f = np.asarray(fp4).reshape(code.shape + (8,))
        r = res["fp4"].reshape(code.shape + (8,))
        fbad = (f != r).any(-1) & ~exempt
        assert not fbad.any(), f"{fbad.sum()} blocks with FP4 codes differing outside near-ties"
    if loss is not None:
        same = code == res["code"]
        scale = res["Q1"] + np.abs(res["C1"])
        lbad = same & (np.abs(np.asarray(loss, dtype=np.float64) - res["loss"]) > REL * scale + 1e-30)
        assert not lbad.any(), f"{lbad.sum()} losses outside tolerance"
    return int(exempt.sum())


def oracle_xq(X64, offsets, bf16, x_amax=None):
    """X_q of the activation-aware workloads: the oracle's NVFP4 fake-quant of X with the input
    quantizer's amax (default: max |X| of each group), in storage form (bf16 bits or float32)."""
    import synth
    offsets = np.asarray(offsets)
    if x_amax is None:
        x_amax = np.array([np.abs(X64[offsets[g]:offsets[g + 1]]).max(initial=0.0)
                           for g in range(len(offsets) - 1)])
    Xq64 = oracle.activation_fake_quant(X64, np.asarray(x_amax, dtype=np.float64), offsets, bf16=bf16)
    return synth.bf16_bits_from_f32(Xq64.astype(np.float32)) if bf16 else Xq64.astype(np.float32)


def with_oracle_xq(wl):
    """The workload with its X_q input filled in from the oracle (activation-aware mode only)."""
    if wl.mode == "act" and wl.Xq is None:
        wl.Xq = oracle_xq(wl.X_f64(), wl.offsets, wl.dtype == "bf16")
    return wl


def _one_blas_thread():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def pool_map(fn, tasks):
    """fn over tasks in a pool of forked processes (up to 16, the host's CPU share of one GPU), one
    BLAS thread each; results in task order.  The workers run NumPy only."""
    import multiprocessing as mp
    import os
    n = max(1, min(16, len(os.sched_getaffinity(0)), len(tasks)))
    if n == 1:
        return [fn(t) for t in tasks]
    with mp.get_context("fork").Pool(n, initializer=_one_blas_thread) as pool:
        return pool.map(fn, tasks, chunksize=1)
