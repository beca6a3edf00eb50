"""GPU parity of the search options: the 256-normalized ("4/6") global scale and the
amax-multiplier search, through lh_scale_sweep_ex / lh_scale_sweep_diag_ex / lh_dequantize_ex,
against the float64 oracle run with the same options (same fp32 H / P / importance on both sides;
codes and FP4 nibbles identical outside near-ties, losses within 1e-5)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import assert_sweep_match, with_oracle_xq

pytestmark = pytest.mark.gpu

lh = pytest.importorskip("nvfp4_scale_calibration_lh_amd")
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None

# an amax search grid of the usual form: start, stop, step (fp32 values)
GRID = np.float32(np.arange(0.25, 2.0001, 0.05))
SMALL = {
    "c1": dict(),
    "c2": dict(cout=150, cin=80, rows=600),
    "c3": dict(cout=70, cin=96, rows=530),
    "c4": dict(cout=130, cin=112, rows=300),
    "c5": dict(n_groups=12, cout=40, cin=64, tokens=400, topk=3),
}


def note(msg):
    print(f"[case] {msg}", flush=True)


def dev(a, bf16=False):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(torch.bfloat16) if bf16 else t).to(DEV)


def _case(name):
    """Weights (device), float64 weights, amax, and the oracle's fp32 H, P, importance."""
    wl = with_oracle_xq(synth.make(name, **SMALL[name]))
    W64 = wl.W_f64()
    W64[0, 1, :16] = 0.0                                   # a zero block
    Ws = synth.bf16_bits_from_f32(W64.astype(np.float32)) if wl.dtype == "bf16" else W64.astype(np.float32)
    amax = oracle.absmax(W64).astype(np.float32)
    H = P = None
    if wl.mode == "act":
        H, P = oracle.accumulate_act_aware(wl.X_f64(), wl.Xq_f64(), wl.offsets)
        P = P.astype(np.float32)
    else:
        H, _ = oracle.accumulate(wl.X_f64(), wl.offsets)
    _, imp = oracle.accumulate(wl.X_f64(), wl.offsets, want_h=False, want_imp=True)
    return wl, dev(Ws, wl.dtype == "bf16"), W64, amax, H.astype(np.float32), P, imp.astype(np.float32)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c5"])
@pytest.mark.parametrize("norm,grid", [(256.0, None), (448.0, GRID), (256.0, GRID)])
def test_sweep_full_options(name, norm, grid):
    wl, Wd, W64, amax, H, P, _ = _case(name)
    note(f"full sweep {name} norm={norm} multipliers={None if grid is None else len(grid)}")
    code, fp4, loss = lh.lh_scale_sweep_ex(Wd, dev(amax), dev(H), None if P is None else dev(P), norm=norm,
                                           multipliers=grid)
    res = oracle.sweep(W64, amax, H, P, norm=norm, multipliers=grid)
    n_ex = assert_sweep_match(code.cpu().numpy(), fp4.cpu().numpy(), loss.cpu().numpy(), res)
    note(f"  exempt near-ties: {n_ex} of {code.numel()}")
    if norm != 448.0:   # the normalization changes the result (not the default search in disguise)
        assert np.any(res["code"] != oracle.sweep(W64, amax, H, P)["code"])


@pytest.mark.parametrize("name", ["c4", "c2", "c5"])
@pytest.mark.parametrize("norm,grid", [(256.0, None), (448.0, GRID), (256.0, GRID)])
@pytest.mark.parametrize("weighted", [True, False])
def test_sweep_diag_and_mse_options(name, norm, grid, weighted):
    wl, Wd, W64, amax, _, _, imp = _case(name)
    note(f"diag sweep {name} norm={norm} multipliers={None if grid is None else len(grid)} weighted={weighted}")
    imp_d = dev(imp) if weighted else None
    code, fp4, loss = lh.lh_scale_sweep_diag_ex(Wd, dev(amax), imp_d, norm=norm, multipliers=grid)
    res = oracle.sweep_diag(W64, amax, imp if weighted else np.ones_like(imp), norm=norm, multipliers=grid)
    assert_sweep_match(code.cpu().numpy(), fp4.cpu().numpy(), loss.cpu().numpy(), res)


def test_dequantize_256_normalized():
    """Codes from a 256-normalized search decode, bit for bit, to the oracle's weights and block
    amax under the same normalization (and not under 448)."""
    wl, Wd, W64, amax, H, _, _ = _case("c2")
    note("dequantize after a 256-normalized search")
    code, fp4, _ = lh.lh_scale_sweep_ex(Wd, dev(amax), dev(H), norm=256.0)
    for dt, bf16 in ((torch.bfloat16, True), (torch.float32, False)):
        Wq, bam = lh.lh_dequantize(code, fp4, dev(amax), dtype=dt, norm=256.0)
        ref_w, ref_a = oracle.dequantize(code.cpu().numpy(), fp4.cpu().numpy(), amax, bf16=bf16, norm=256.0)
        np.testing.assert_array_equal(Wq.float().cpu().numpy().astype(np.float64), ref_w)
        np.testing.assert_array_equal(bam.cpu().numpy().astype(np.float64), ref_a)
    _, bam448 = lh.lh_dequantize(code, fp4, dev(amax))
    assert not torch.equal(bam, bam448)


def test_multiplier_search_single_multiplier_is_max_scaling():
    """One multiplier 1.0: every block takes the E4M3 code nearest to its amax / (6 g), the plain
    max-calibrated NVFP4 block scale, whatever the objective."""
    wl, Wd, W64, amax, H, _, imp = _case("c2")
    note("multiplier search with the single multiplier 1")
    code, _, _ = lh.lh_scale_sweep_ex(Wd, dev(amax), dev(H), multipliers=[1.0])
    code_d, _, _ = lh.lh_scale_sweep_diag_ex(Wd, dev(amax), dev(imp), multipliers=[1.0])
    G, cout, cin = W64.shape
    ab = np.abs(W64.reshape(G, cout, cin // 16, 16)).max(-1).reshape(-1)
    g = np.repeat(oracle.global_scale(amax.astype(np.float64)), cout * cin // 16)
    want = oracle.multiplier_codes(ab, g, np.array([1.0]))[:, 0].reshape(G, cout, cin // 16)
    np.testing.assert_array_equal(code.cpu().numpy(), want)
    np.testing.assert_array_equal(code_d.cpu().numpy(), want)


@pytest.mark.parametrize("diag", [False, True])
def test_multiplier_search_every_code_and_ranges(diag):
    """Blocks whose best code cycles over all 126 (a 128-value geometric grid proposes a spread of
    codes around each block's amax scale), plus weights and Hessians / importance outside the
    filters' ranges so that the float64 passes apply the grid too."""
    r = np.random.default_rng(37)
    nb, cout = 4, 504
    cin = 16 * nb
    s = oracle.candidate_scales(oracle.global_scale(np.float32(1.0)))
    W = r.standard_normal((1, cout, nb, 16))
    W /= np.abs(W).max(-1, keepdims=True)
    k = (np.arange(cout * nb) % 126).reshape(cout, nb)
    W *= (6.0 * s[k] * r.uniform(0.97, 1.03, (cout, nb)))[None, :, :, None]
    W = W.reshape(1, cout, cin).astype(np.float32)
    W[0, 0, 0] = 1.0
    W = np.concatenate([W, W * np.float32(1e-20)], axis=0)          # group 1: tiny weights
    grid = np.float32(0.3 * 1.012 ** np.arange(128))
    a = oracle.absmax(W.astype(np.float64)).astype(np.float32)
    note(f"multiplier search, every code and ranges, diag={diag}")
    if diag:
        imp = (np.abs(r.standard_normal((2, cin))) + 0.1).astype(np.float32)
        imp[1] *= np.float32(1e36)
        code, fp4, loss = lh.lh_scale_sweep_diag_ex(dev(W), dev(a), dev(imp), multipliers=grid)
        res = oracle.sweep_diag(W.astype(np.float64), a, imp, multipliers=grid)
    else:
        A = r.standard_normal((2, nb, 16, 16))
        H = np.einsum("gnij,gnkj->gnik", A, A) / 16 + 0.5 * np.eye(16)
        H[1] *= 1e34
        H = H.astype(np.float32)
        code, fp4, loss = lh.lh_scale_sweep_ex(dev(W), dev(a), dev(H), multipliers=grid)
        res = oracle.sweep(W.astype(np.float64), a, H, multipliers=grid)
    assert len(np.unique(res["code"][0])) > 100
    assert_sweep_match(code.cpu().numpy(), fp4.cpu().numpy(), loss.cpu().numpy(), res)
