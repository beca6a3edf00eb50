"""The two bounds that let the diagonal sweep score only a window of 32 codes per block, checked
exactly (float64, exact quantization) against every candidate's loss on seeded blocks.

For a block of amax a, kmax is a code with 6 s_kmax >= a and the window is the 32 codes from
start = clamp(kmax - 12, 1, 95).  For every code k below it the loss is at least
LB_lo = sum_i Imp_i (|w_i| - 6 s_{start-1})_+^2 (the block's clipped elements), and for every
code above it at least LB_hi = sum_{|w_i| < s_hi/2} Imp_i min(|w_i|, s_hi/2 - |w_i|)^2 with
s_hi = s_{start+32}.  These are statements about the objective the pages define, so the oracle's
own candidate losses decide them; the kernel relies on them to skip the other codes."""
import numpy as np

import oracle
from oracle.lh_oracle import candidate_scales, e4m3_ladder, fake_quant


def window(amax_b, g):
    """The window's first code (1-based) and kmax, by the rule above: kmax is one above the
    smallest code whose value is at least amax / (6 g)."""
    lad = e4m3_ladder()
    y = amax_b / (6.0 * g)
    k = int(np.searchsorted(lad, y, side="left")) + 1          # smallest code with v >= y
    kmax = min(126, max(1, k) + 1)
    return min(max(kmax - 12, 1), 95), kmax


def blocks(seed, n):
    r = np.random.default_rng(seed)
    W = r.normal(0, 0.01, (n, 16))
    W[: n // 4] *= 10.0 ** r.uniform(-3, 1, (n // 4, 1))           # blocks of other sizes
    W[n // 4: n // 2, 0] *= 40.0                                   # one dominant element
    imp = r.chisquare(64, (n, 16))
    imp[n // 2: 3 * n // 4] *= 10.0 ** r.uniform(-6, 6, (n // 4, 16))   # wide importance spreads
    W = W.astype(np.float32).astype(np.float64)
    return W, imp


def test_window_bounds_hold_for_every_candidate():
    W, imp = blocks(71, 4000)
    amax = np.abs(W).max()
    g = float(oracle.global_scale(np.array([amax]))[0])
    s = candidate_scales(np.full(len(W), g))                      # [n, 126]
    _, _, E = fake_quant(W[:, None, :], s[:, :, None])
    L = np.einsum("bki,bi->bk", E * E, imp)                       # exact candidate losses
    checked_lo = checked_hi = 0
    for b in range(len(W)):
        ab = np.abs(W[b]).max()
        if ab == 0.0:
            continue
        start, kmax = window(ab, g)
        assert 6.0 * s[b, kmax - 1] >= ab                         # kmax as the kernel takes it
        if start > 1:
            lb = (imp[b] * np.maximum(np.abs(W[b]) - 6.0 * s[b, start - 2], 0.0) ** 2).sum()
            assert (L[b, : start - 1] >= lb * (1 - 1e-12)).all()
            checked_lo += 1
        end = start + 31
        if end < 126:
            sh = s[b, end]                                        # code end + 1
            aw = np.abs(W[b])
            lh = (imp[b] * np.where(aw < sh / 2, np.minimum(aw, sh / 2 - aw), 0.0) ** 2).sum()
            assert (L[b, end:] >= lh * (1 - 1e-12)).all()
            # and above kmax + 47 every element rounds to 0
            if kmax + 47 <= 126:
                assert np.allclose(L[b, kmax + 46:], (imp[b] * W[b] ** 2).sum(), rtol=1e-12, atol=0)
            checked_hi += 1
    assert checked_lo > 3000 and checked_hi > 100


def test_window_bounds_decide_most_blocks():
    """On blocks shaped like the WMSE layer's (normal weights, chi-square importance with a few
    outlier channels) the argmin lies in the window and both bounds exceed the window's minimum
    for nearly every block, so few blocks are left to the float64 pass."""
    r = np.random.default_rng(5)
    n = 8000
    W = r.normal(0, 0.01, (n, 16)).astype(np.float32).astype(np.float64)
    imp = r.chisquare(8192, (n, 16))
    imp[r.random((n, 16)) < 0.005] *= 900.0
    amax = np.abs(W).max() * 3
    g = float(oracle.global_scale(np.array([amax]))[0])
    s = candidate_scales(np.full(n, g))
    _, _, E = fake_quant(W[:, None, :], s[:, :, None])
    L = np.einsum("bki,bi->bk", E * E, imp)
    k_opt = np.argmin(L, axis=1) + 1
    decided = 0
    for b in range(n):
        ab = np.abs(W[b]).max()
        start, _ = window(ab, g)
        end = start + 31
        best = L[b, start - 1: end].min()
        lb = (imp[b] * np.maximum(np.abs(W[b]) - 6.0 * s[b, start - 2], 0.0) ** 2).sum() if start > 1 else np.inf
        sh = s[b, end] if end < 126 else np.inf
        aw = np.abs(W[b])
        lh = (imp[b] * np.where(aw < sh / 2, np.minimum(aw, sh / 2 - aw), 0.0) ** 2).sum() if end < 126 else np.inf
        if lb > best * (1 + 1e-4) and lh >= best * (1 + 1e-4):
            assert start <= k_opt[b] <= end
            decided += 1
    assert decided > 0.95 * n
