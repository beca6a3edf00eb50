"""GPU parity of the fused accumulate-and-sweep path for grouped rows (lh_accumulate_sweep): codes,
nibbles and losses bit-identical to lh_accumulate followed by lh_scale_sweep_ex, and against the
float64 oracle run on the oracle's own Hessians (near-ties exempt, losses within 1e-5)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import assert_sweep_match

pytestmark = pytest.mark.gpu

lh = pytest.importorskip("nvfp4_scale_calibration_lh_amd")
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
GRID = np.float32(np.arange(0.25, 2.0001, 0.05))


def note(msg):
    print(f"[case] {msg}", flush=True)


def dev(a, bf16=False):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(torch.bfloat16) if bf16 else t).to(DEV)


def _moe(empty_group=True, bf16=True, G=12, cout=40, cin=64, tokens=400, topk=3, seed=0):
    wl = synth.make("c5", seed=seed, n_groups=G, cout=cout, cin=cin, tokens=tokens, topk=topk)
    X, W, off = wl.X, wl.W, wl.offsets.copy()
    if empty_group:                              # group 3 gets no rows (its rows go to group 4)
        off[4] = off[3]
    if not bf16:
        X = synth.f32_from_bf16_bits(X)
        W = synth.f32_from_bf16_bits(W)
    X64 = (synth.f32_from_bf16_bits(X) if bf16 else X).astype(np.float64)
    W64 = (synth.f32_from_bf16_bits(W) if bf16 else W).astype(np.float64)
    return X, W, off, X64, W64


def _two_call(Xd, Wd, ad, offd, norm, grid):
    H, _ = lh.lh_accumulate(Xd, offsets=offd)
    return lh.lh_scale_sweep_ex(Wd, ad, H, norm=norm, multipliers=grid)


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("norm,grid", [(448.0, None), (448.0, GRID), (256.0, None)])
def test_fused_equals_two_calls_and_oracle(bf16, norm, grid):
    X, W, off, X64, W64 = _moe(bf16=bf16)
    G = W.shape[0]
    note(f"fused accumulate+sweep G={G} W{W.shape} X{X.shape} bf16={bf16} norm={norm} "
         f"multipliers={None if grid is None else len(grid)}")
    Xd, Wd, offd = dev(X, bf16), dev(W, bf16), dev(off)
    amax = oracle.absmax(W64).astype(np.float32)
    ad = dev(amax)
    code, fp4, loss = lh.lh_accumulate_sweep(Xd, Wd, ad, offd, norm=norm, multipliers=grid)
    c2, f2, l2 = _two_call(Xd, Wd, ad, offd, norm, grid)
    assert torch.equal(code, c2) and torch.equal(fp4, f2)
    assert torch.equal(loss.view(torch.int32), l2.view(torch.int32))
    H_ref, _ = oracle.accumulate(X64, off)
    res = oracle.sweep(W64, amax, H_ref, norm=norm, multipliers=grid)
    assert_sweep_match(code.cpu().numpy(), fp4.cpu().numpy(), None, res)
    # the empty group searched with the plain weight-MSE objective
    eye = np.broadcast_to(np.eye(16), (1, W.shape[2] // 16, 16, 16))
    plain = oracle.sweep(W64[3:4], amax[3:4], eye, norm=norm, multipliers=grid)
    assert_sweep_match(code.cpu().numpy()[3:4], fp4.cpu().numpy()[3:4], loss.cpu().numpy()[3:4], plain)


def test_fused_float64_path_and_long_groups():
    """Activations scaled by 2^56 put every H beyond the float32 filter's range, so every block of
    the fused kernel is re-scored in float64 after the filter pass; a few long groups split into
    several pieces.  Bit-identical to the two calls."""
    X, W, off, X64, W64 = _moe(empty_group=False, G=5, cout=70, cin=48, tokens=900, topk=2, seed=3)
    note(f"fused accumulate+sweep, float64 path, G=5 W{W.shape} X{X.shape}")
    Xs = synth.bf16_bits_from_f32(synth.f32_from_bf16_bits(X) * np.float32(2.0 ** 56))
    Xd, Wd, offd = dev(Xs, True), dev(W, True), dev(off)
    amax = dev(oracle.absmax(W64).astype(np.float32))
    code, fp4, loss = lh.lh_accumulate_sweep(Xd, Wd, amax, offd)
    c2, f2, l2 = _two_call(Xd, Wd, amax, offd, 448.0, None)
    assert torch.equal(code, c2) and torch.equal(fp4, f2)
    assert torch.equal(loss.view(torch.int32), l2.view(torch.int32))
    # and in the filter's range, rows split into pieces of the grouped accumulation
    big = synth.make("c5", seed=5, n_groups=3, cout=33, cin=64, tokens=6000, topk=2)
    note(f"fused accumulate+sweep, long groups T={np.diff(big.offsets).tolist()}")
    Xd, Wd, offd = dev(big.X, True), dev(big.W, True), dev(big.offsets)
    amax = lh.lh_absmax(Wd)
    code, fp4, loss = lh.lh_accumulate_sweep(Xd, Wd, amax, offd)
    c2, f2, l2 = _two_call(Xd, Wd, amax, offd, 448.0, None)
    assert torch.equal(code, c2) and torch.equal(fp4, f2)
    assert torch.equal(loss.view(torch.int32), l2.view(torch.int32))
