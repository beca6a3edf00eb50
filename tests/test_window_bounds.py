"""The two bounds that let the diagonal sweep score only a window of 32 codes per block, checked
exactly (float64, exact quantization) against every candidate's loss on seeded blocks.

For a block of amax a, kmax is a code with 6 s_kmax >= a and the window is the 32 codes from
start = clamp(kmax - 12, 1, 95).  For every code k below it the loss is at least
LB_lo = sum_i Imp_i (|w_i| - 6 s_{start-1})_+^2 (the block's clipped elements), and for every
code above it at least LB_hi = sum_{|w_i| < s_hi/2} Imp_i min(|w_i|, s_hi/2 - |w_i|)^2 with
s_hi = s_{start+32}.  These are statements about the objective the pages define, so the oracle's
own candidate losses decide them; the kernel relies on them to skip the other codes."""
import numpy as np
import pytest

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


# --------------------------------------------------------------------------- full Hessian
# The full-Hessian sweep scores codes 97..126 first and skips codes 1..K, K = 96 (else 64 once
# codes 65..96 are scored too), when
#   LB_K = mu * sum_i (|w_i| - 6 s_K)_+^2             (no cross term)
#   LB_K = c (mu c - 2 |b|),  c^2 = that sum,  mu c >= |b|   (b = P w, with the cross term)
# exceeds the lowest loss among the codes scored, mu a lower bound of the smallest eigenvalue of
# the symmetric part of H.  The inequalities L_k >= LB_K for every k <= K are checked here on the
# oracle's own losses with mu = the exact smallest eigenvalue (the kernel's mu is smaller).

def hessians(seed, n):
    """Block Hessians X^T X / T of T in 2..400 rows (singular below 16), some with outlier
    channels or strong correlations, and a few non-symmetric perturbations."""
    r = np.random.default_rng(seed)
    Hs = []
    for j in range(n):
        T = int(r.choice([2, 8, 15, 16, 20, 40, 160, 400]))
        X = r.standard_normal((T, 16))
        if j % 3 == 1:
            X[:, r.integers(16)] *= 20.0
        if j % 3 == 2:
            X = X @ (np.eye(16) + 0.9 * r.standard_normal((16, 16)) / 4)
        H = X.T @ X / T
        if j % 7 == 0:
            H = H + 1e-3 * np.abs(H).max() * r.standard_normal((16, 16))
        Hs.append(H.astype(np.float32).astype(np.float64))
    return np.array(Hs)


@pytest.mark.parametrize("K", [64, 96])
def test_full_window_bound_holds_below_code_K(K):
    r = np.random.default_rng(72)
    n = 600
    W, _ = blocks(73, n)
    H = hessians(74, n)
    P = 0.1 * r.standard_normal((n, 16, 16)) * np.sqrt(np.abs(np.diagonal(H, axis1=1, axis2=2)))[:, :, None]
    amax = np.abs(W).max()
    g = np.full(n, float(oracle.global_scale(np.array([amax]))[0]))
    sK = candidate_scales(g[:1])[0, K - 1]
    L0, Q, C = oracle.candidate_losses(W, g, H, None)
    L1, _, _ = oracle.candidate_losses(W, g, H, P)
    S = 0.5 * (H + np.transpose(H, (0, 2, 1)))
    mu = np.linalg.eigvalsh(S)[:, 0]
    dead = np.trace(H, axis1=1, axis2=2) == 0
    mu[dead] = 1.0
    c2 = (np.maximum(np.abs(W) - 6.0 * sK, 0.0) ** 2).sum(1)
    psd = mu > 0                        # the kernel uses the bound only with a positive mu
    assert 0.3 < psd.mean() < 1.0       # singular and indefinite Hessians are among the cases
    mu = np.where(psd, mu, 0.0)
    lb0 = mu * c2
    low = L0[:, :K]
    assert np.all(low[psd] >= lb0[psd, None] - 1e-12 * np.abs(low[psd])), "mu |e|^2 bound violated"
    b = np.einsum("bij,bj->bi", P, W)
    bn = np.linalg.norm(b, axis=1)
    c = np.sqrt(c2)
    ok = psd & (mu * c >= bn)
    lb1 = c * (mu * c - 2.0 * bn)
    low1 = L1[:, :K]
    assert np.all(low1[ok] >= lb1[ok, None] - 1e-12 * np.abs(low1[ok])), "coupled bound violated"
    # a bound for the larger code set is never above the smaller set's (6 s_K grows with K)
    if K == 96:
        s64 = candidate_scales(g[:1])[0, 63]
        assert np.all(c2 <= (np.maximum(np.abs(W) - 6.0 * s64, 0.0) ** 2).sum(1))
    # not vacuous: for well-conditioned blocks whose argmin is above code K the bound rules out
    # codes <= K for most blocks (many of these blocks sit only a few times above the clipping
    # level of code K)
    U = L0[:, K:].min(1)
    good = np.array([np.linalg.eigvalsh(h)[0] > 1e-3 * np.abs(h).max() for h in S])
    good &= L0.argmin(1) >= K
    assert good.sum() > 40 and np.mean((lb0 > U)[good]) > 0.5
    # ... and on blocks of a layer-like tensor (N(0, 0.02) weights whose tensor amax is that of
    # 3.3M such values, Hessians of 40 to 400 tokens) it rules out codes <= K for nearly all
    rl = np.random.default_rng(76)
    m = 400
    Wl = rl.normal(0, 0.02, (m, 16)).astype(np.float32).astype(np.float64)
    gl = np.full(m, float(oracle.global_scale(np.array([0.02 * 5.1]))[0]))
    Hl = []
    for j in range(m):
        X = rl.standard_normal((int(rl.choice([40, 100, 400])), 16))
        Hl.append((X.T @ X / len(X)).astype(np.float32).astype(np.float64))
    Hl = np.array(Hl)
    Ll, _, _ = oracle.candidate_losses(Wl, gl, Hl, None)
    assert np.all(Ll.argmin(1) >= 96)                 # the argmin sits in the two top tiles
    mul = np.linalg.eigvalsh(Hl)[:, 0]
    lbl = mul * (np.maximum(np.abs(Wl) - 6.0 * candidate_scales(gl[:1])[0, K - 1], 0.0) ** 2).sum(1)
    assert np.all(Ll[:, :K] >= lbl[:, None] - 1e-12 * np.abs(Ll[:, :K]))
    assert np.mean(lbl > Ll[:, K:].min(1)) > 0.9


def _chol32_passes(S, m, rng):
    """The kernel's float32 Cholesky test of S - m I (lane i holds row i): pivots through a
    reciprocal square root carrying up to one unit of error, products and fused updates in
    float32; True when every pivot is positive."""
    f = np.float32
    A = S.astype(np.float32).copy()
    A[np.diag_indices(16)] = (A[np.diag_indices(16)] - f(m)).astype(np.float32)
    for j in range(16):
        piv = A[j, j]
        if not piv > 0:
            return False
        isr = f(1.0 / np.sqrt(np.float64(piv)))
        isr = f(isr * (1.0 + rng.choice([-1.0, 0.0, 1.0]) * 2.0 ** -23))     # one unit either way
        li = (A[j:, j] * isr).astype(np.float32)
        for k in range(j + 1, 16):
            lk = f(A[k, j] * isr)
            A[k:, k] = (A[k:, k].astype(np.float64) - li[k - j:].astype(np.float64) * np.float64(lk)).astype(np.float32)
    return True


def test_cholesky_certificate_margin():
    """A float32 factorization of S - m I that completes with positive pivots certifies
    lambda_min(S) >= m - 2^-12 for S scaled to max |S_ij| < 1: checked on near-singular matrices
    with m just above and below the smallest eigenvalue."""
    r = np.random.default_rng(75)
    tried = passed = 0
    for j in range(300):
        T = int(r.choice([16, 17, 20, 24, 40]))
        X = r.standard_normal((T, 16))
        X[:, 0] *= 10.0 ** r.uniform(-3, 1)
        S = X.T @ X
        S = S / (np.abs(S).max() * 1.0001)
        S = S.astype(np.float32).astype(np.float64)
        lam = np.linalg.eigvalsh(S)[0]
        for m in (lam * (1 + 1e-3), lam + 2.0 ** -16, lam + 2.0 ** -14, lam * 0.999, lam / 2):
            if m <= 0:
                continue
            tried += 1
            if _chol32_passes(S, m, r):
                passed += 1
                assert lam >= m - 2.0 ** -12, (lam, m)
    assert tried > 1000 and passed > 300


def test_cholesky_certificate_negative_shifts():
    """The negative shifts m = -2^-14 .. -2^-8 that the certificate tries when no positive one
    passes: a float32 factorization of S - m I with positive pivots still certifies
    lambda_min(S) >= m - 2^-12, on singular (fewer than 16 rows), near-singular and indefinite S,
    and the shifts pass for singular X^T X (the case they are there for)."""
    r = np.random.default_rng(81)
    tried = passed = passed_singular = singular = 0
    for j in range(300):
        T = int(r.choice([4, 10, 13, 15, 16, 17]))
        X = r.standard_normal((T, 16))
        S = X.T @ X
        if j % 5 == 4:
            S = S - 2.0 ** -9 * np.abs(S).max() * np.eye(16)     # slightly indefinite
        S = S / (np.abs(S).max() * 1.0001)
        S = S.astype(np.float32).astype(np.float64)
        lam = np.linalg.eigvalsh(S)[0]
        singular += T < 16 and j % 5 != 4
        for e in (-14, -12, -10, -8):
            m = -2.0 ** e
            tried += 1
            if _chol32_passes(S, m, r):
                passed += 1
                passed_singular += T < 16 and j % 5 != 4 and e == -12
                assert lam >= m - 2.0 ** -12, (lam, m)
    assert tried == 1200 and passed > 300 and passed_singular > 0.9 * singular


# The full-Hessian sweep also uses, in its uncoupled form, a bound that needs no positive smallest
# eigenvalue.  With mu <= lambda_min(S) (any sign, S the symmetric part of H), S - mu I is positive
# semidefinite; for k <= K the quantized block q (e = q - w) has |q_i| <= tau = 6 s_K, so in the
# seminorm of S - mu I the triangle inequality and |x^T A x| <= max|x_i|^2 sum |A_ij| give
#   L_k = e^T S e >= (sqrt(w^T H w - mu |w|^2) - tau sqrt(sum |H_ij| + 16 |mu|))_+^2 + mu_term,
# mu_term = mu sum_i (|w_i| - tau)_+^2 for mu >= 0 and mu (|w| + 4 tau)^2 for mu < 0.

def _triangle_bound(W, H, mu, tau):
    whw = np.einsum("bi,bij,bj->b", W, H, W)
    ww = (W * W).sum(1)
    A = np.abs(H).sum((1, 2)) + 16.0 * np.abs(mu)
    t = np.maximum(np.sqrt(np.maximum(whw - mu * ww, 0.0)) - tau * np.sqrt(A), 0.0)
    mu_term = np.where(mu >= 0, mu * (np.maximum(np.abs(W) - tau, 0.0) ** 2).sum(1),
                       mu * (np.sqrt(ww) + 4.0 * tau) ** 2)
    return t * t + mu_term


@pytest.mark.parametrize("K", [64, 96])
def test_triangle_bound_holds_below_code_K(K):
    r = np.random.default_rng(77)
    n = 600
    W, _ = blocks(78, n)
    H = hessians(79, n)                             # singular, indefinite and regular
    amax = np.abs(W).max()
    g = np.full(n, float(oracle.global_scale(np.array([amax]))[0]))
    tau = 6.0 * candidate_scales(g[:1])[0, K - 1]
    L, _, _ = oracle.candidate_losses(W, g, H, None)
    S = 0.5 * (H + np.transpose(H, (0, 2, 1)))
    lam = np.linalg.eigvalsh(S)[:, 0]
    live = np.trace(H, axis1=1, axis2=2) != 0
    for shift in (0.0, 1e-3):                       # the exact lambda_min and a smaller mu
        mu = lam - shift * np.abs(S).max((1, 2))
        lb = _triangle_bound(W, H, mu, tau)
        low = L[:, :K]
        assert np.all(low[live] >= lb[live, None] - 1e-12 * np.abs(low[live])), "triangle bound violated"
    # not vacuous where the eigenvalue bound is: Hessians of 10 to 16 tokens (singular or nearly)
    # on layer-like blocks, whose argmin is in the two top tiles
    rl = np.random.default_rng(80)
    m = 400
    Wl = rl.normal(0, 0.02, (m, 16)).astype(np.float32).astype(np.float64)
    gl = np.full(m, float(oracle.global_scale(np.array([0.02 * 5.1]))[0]))
    Hl = np.array([(X.T @ X / len(X)).astype(np.float32).astype(np.float64)
                   for X in (rl.standard_normal((int(rl.choice([10, 13, 16])), 16)) for _ in range(m))])
    Ll, _, _ = oracle.candidate_losses(Wl, gl, Hl, None)
    taul = 6.0 * candidate_scales(gl[:1])[0, K - 1]
    lam_l = np.linalg.eigvalsh(Hl)[:, 0]
    lbl = _triangle_bound(Wl, Hl, lam_l - 2.0 ** -10 * np.abs(Hl).max((1, 2)), taul)
    assert np.all(Ll[:, :K] >= lbl[:, None] - 1e-12 * np.abs(Ll[:, :K]))
    eig_lb = np.maximum(lam_l, 0.0) * (np.maximum(np.abs(Wl) - taul, 0.0) ** 2).sum(1)
    U = Ll[:, K:].min(1)
    assert np.mean(eig_lb > U) < 0.3 and np.mean(lbl > U) > 0.5
