"""Pins of the float64 oracle against facts fixed outside itself (no GPU needed).

Each test checks the oracle against something it does not compute itself: a library decoder,
exact rational arithmetic, a brute-force output-MSE evaluation, a closed-form identity, an
invariance of the method, or hand-derived golden cases.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle import lh_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GRID_F = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
          Fraction(4), Fraction(6)]


def rng(*k):
    return np.random.default_rng(list(k))


# ------------------------------------------------------------------ P1: the E4M3 candidate ladder
def test_e4m3_ladder_matches_library_decoder():
    torch = pytest.importorskip("torch")
    allb = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    pos = [(b, v) for b, v in enumerate(allb) if np.isfinite(v) and v > 0]
    assert len(pos) == 126                                  # "126 candidate scales"
    assert [b for b, _ in pos] == list(range(1, 127))
    lad = oracle.e4m3_ladder()
    np.testing.assert_array_equal(lad, np.array([v for _, v in pos]))
    assert lad[0] == 2.0 ** -9 and lad[-1] == 448.0        # 448-normalized NVFP4 scaling
    assert np.all(np.diff(lad) > 0)


def test_global_and_candidate_scales_are_fp32_roundings():
    amax = np.float32(0.0871234)
    g = oracle.global_scale(amax)
    assert g == np.float64(np.float32(Fraction(float(amax)) / 2688))  # correctly rounded quotient
    s = oracle.candidate_scales(g)
    for k in (0, 7, 63, 125):
        exact = Fraction(float(O.e4m3_ladder()[k])) * Fraction(float(g))
        assert s[k] == float(np.float32(float(exact)))
    # candidate 126 restores the block amax: 6 * s_126 ~= amax (448 * 6 = 2688)
    assert abs(6 * s[-1] - float(amax)) <= 2 * 6 * np.spacing(np.float32(s[-1]))


# ------------------------------------------------------------------ max calibration (absmax)
def _pin_absmax(absmax_fn):
    """max |W_g| per group, checked against an element-by-element walk over exact values that
    never calls abs(): each element's magnitude is decided by a comparison with zero."""
    r = rng(21)
    W = r.normal(0, 0.02, (5, 7, 32)).astype(np.float32).astype(np.float64)
    W[0, 3, 5] = -0.5                       # group 0: its largest magnitude is negative
    W[1] = np.abs(W[1])                     # group 1: all positive
    W[2] = -np.abs(W[2])                    # group 2: all negative
    W[3] = 0.0
    W[3, 0, 0] = -0.0                       # group 3: zeros, one of them -0
    W[4, 6, 31] = 0.25                      # group 4: the max is the last element
    got = absmax_fn(W)
    assert got.shape == (5,)
    for g in range(5):
        best = 0.0
        for x in W[g].reshape(-1).tolist():
            mag = -x if x < 0 else x
            if mag > best:
                best = mag
        assert got[g] == best, (g, got[g], best)
    assert got[0] == 0.5 and got[3] == 0.0 and not np.signbit(got[3]) and got[4] == 0.25
    # groups are independent: changing one group changes only its own amax
    W2 = W.copy()
    W2[1, 0, 0] = 7.0
    got2 = absmax_fn(W2)
    assert got2[1] == 7.0 and np.array_equal(np.delete(got2, 1), np.delete(got, 1))
    # an empty group (no elements) gives 0
    assert np.array_equal(absmax_fn(np.zeros((3, 0))), np.zeros(3))


def test_absmax_against_elementwise_walk():
    _pin_absmax(oracle.absmax)


def _pin_accumulate_beta(accumulate_fn):
    """Streaming form H = beta H_prev + (1/T) sum_t x_t x_t^T and imp = beta imp_prev + sum_t x_t^2,
    each entry checked against a correctly rounded scalar sum (math.fsum) of the definition, with
    H_prev and imp_prev unrelated to the new batch; an empty group keeps only the beta term."""
    import math
    r = rng(22)
    cin = 32
    X = r.normal(0, 1, (11, cin))
    off = np.array([0, 7, 7, 11])            # groups of 7, 0 and 4 rows
    G = 3
    H_prev = r.normal(0, 1, (G, cin // 16, 16, 16))
    imp_prev = r.uniform(0, 5, (G, cin))
    for beta in (0.5, -1.25, 1.0):
        H, imp = accumulate_fn(X, off, beta=beta, H_prev=H_prev, imp_prev=imp_prev, want_h=True, want_imp=True)
        for g in range(G):
            rows = X[off[g]:off[g + 1]]
            T = len(rows)
            for n in range(cin // 16):
                for i in range(16):
                    for j in range(16):
                        s = math.fsum(rows[t, 16 * n + i] * rows[t, 16 * n + j] for t in range(T))
                        want = beta * H_prev[g, n, i, j] + (s / T if T else 0.0)
                        assert abs(H[g, n, i, j] - want) <= 1e-13 * (abs(want) + 1.0), (beta, g, n, i, j)
            for i in range(cin):
                want = beta * imp_prev[g, i] + math.fsum(rows[t, i] ** 2 for t in range(T))
                assert abs(imp[g, i] - want) <= 1e-13 * (abs(want) + 1.0), (beta, g, i)


def test_accumulate_beta_against_closed_form():
    _pin_accumulate_beta(oracle.accumulate)


def test_pins_catch_planted_mistakes():
    """Each pin above fails on a plausible slip planted in a copy of the oracle function."""
    def no_abs(W):                                   # max instead of max |.|
        W = np.asarray(W, dtype=np.float64)
        return W.reshape(W.shape[0], -1).max(axis=1) if W.size else np.zeros(W.shape[0])

    def first_group_only(W):                         # one amax for every group
        a = oracle.absmax(W)
        return np.full_like(a, a[0]) if a.size else a

    for planted in (no_abs, first_group_only):
        with pytest.raises(AssertionError):
            _pin_absmax(planted)

    def beta_ignored(X, off, beta=0.0, H_prev=None, imp_prev=None, **kw):
        return oracle.accumulate(X, off, beta=1.0 if beta != 0 else 0.0, H_prev=H_prev, imp_prev=imp_prev, **kw)

    def beta_on_new_term(X, off, beta=0.0, H_prev=None, imp_prev=None, **kw):
        H, imp = oracle.accumulate(X, off, **kw)
        return H_prev + beta * H, imp_prev + beta * imp

    def imp_divided_by_t(X, off, beta=0.0, H_prev=None, imp_prev=None, **kw):
        H, imp = oracle.accumulate(X, off, beta=beta, H_prev=H_prev, imp_prev=imp_prev, **kw)
        T = np.maximum(np.diff(off), 1)[:, None]
        return H, beta * imp_prev + (imp - beta * imp_prev) / T

    for planted in (beta_ignored, beta_on_new_term, imp_divided_by_t):
        with pytest.raises(AssertionError):
            _pin_accumulate_beta(planted)


# ------------------------------------------------------------------ P2: E2M1 rounding
def _exact_index(w: float, s: float) -> int:
    if s == 0:
        return 0
    r = abs(Fraction(w)) / Fraction(s)
    d = [abs(r - v) for v in GRID_F]
    best = min(d)
    cands = [i for i, x in enumerate(d) if x == best]
    even = [i for i in cands if i % 2 == 0]
    return even[0] if even else cands[0]


def test_e2m1_golden_cases():
    rows = []
    with open(os.path.join(GOLDEN, "e2m1_cases.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                w, s, nib = line.split()[:3]
                rows.append((float(w), float(s), int(nib, 16)))
    assert len(rows) >= 20
    for w, s, nib in rows:
        got, _, _ = oracle.fake_quant(np.array([w]), np.array([s]))
        assert int(got[0]) == nib, (w, s, nib, int(got[0]))


def test_e2m1_rounding_matches_exact_rationals_on_midpoints_and_neighbours():
    r = rng(2)
    cases_w, cases_s = [], []
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    # scales with short mantissas make m*s exactly representable: genuine ties
    for s in [1.0, 0.5, 2.0 ** -7, 0.75, 1.5 * 2.0 ** -9, 0.625]:
        for m in mids:
            w = np.float32(m * s)
            for v in (w, np.nextafter(w, np.float32(np.inf)), np.nextafter(w, np.float32(0))):
                cases_w.append(float(v)); cases_s.append(s)
    # random fp32 scales: nearest fp32 neighbours of the (inexact) midpoints
    for _ in range(300):
        s = float(np.float32(r.uniform(1e-4, 1.0)))
        m = mids[r.integers(len(mids))]
        w = np.float32(m * s)
        for v in (w, np.nextafter(w, np.float32(np.inf)), np.nextafter(w, np.float32(0))):
            cases_w.append(float(v)); cases_s.append(s)
    # bf16 weights against candidate scales from the real ladder
    g = float(oracle.global_scale(0.09))
    sc = oracle.candidate_scales(g)
    wb = synth.f32_from_bf16_bits(synth.bf16_bits_from_f32(r.normal(0, 0.02, 400).astype(np.float32)))
    for w in wb:
        for s in sc[r.integers(0, 126, 4)]:
            cases_w.append(float(w)); cases_s.append(float(s))
    w = np.array(cases_w); s = np.array(cases_s)
    nib, wq, e = oracle.fake_quant(w, s)
    exp = np.array([_exact_index(a, b) for a, b in zip(cases_w, cases_s)])
    np.testing.assert_array_equal(nib & 7, exp)
    np.testing.assert_array_equal(nib >> 3, (w < 0).astype(np.uint8))
    # e is exact: compare with rationals
    for i in range(0, len(w), 97):
        q = GRID_F[exp[i]] * Fraction(s[i]) * (-1 if w[i] < 0 else 1)
        assert Fraction(e[i]) == q - Fraction(w[i])


def test_pack_nibbles_low_first():
    nib = np.array([[1, 2, 3, 4, 0xf, 0]], dtype=np.uint8)
    np.testing.assert_array_equal(oracle.pack_nibbles(nib), [[0x21, 0x43, 0x0f]])


# ------------------------------------------------------------------ accumulation identities
def test_hessian_quadratic_form_and_importance_identities():
    r = rng(3)
    T, cin = 53, 48
    X = r.standard_normal((T, cin))
    off = np.array([0, T])
    H, imp = oracle.accumulate(X, off, want_imp=True)
    for n in range(cin // 16):
        v = r.standard_normal(16)
        q = X[:, 16 * n:16 * n + 16] @ v
        assert np.isclose(v @ H[0, n] @ v, q @ q / T, rtol=1e-12)
        np.testing.assert_allclose(np.diag(H[0, n]) * T, imp[0, 16 * n:16 * n + 16], rtol=1e-12)
        assert np.allclose(H[0, n], H[0, n].T)
    assert np.isclose(imp.sum(), (X * X).sum(), rtol=1e-12)


def test_cross_matrix_bilinear_identity_and_beta():
    r = rng(4)
    T, cin = 41, 32
    X = r.standard_normal((T, cin))
    Xq = X + 0.1 * r.standard_normal((T, cin))
    off = np.array([0, T])
    H, P = oracle.accumulate_act_aware(X, Xq, off)
    u, v = r.standard_normal(16), r.standard_normal(16)
    for n in range(2):
        sl = slice(16 * n, 16 * n + 16)
        assert np.isclose(u @ P[0, n] @ v, (Xq[:, sl] @ u) @ ((Xq - X)[:, sl] @ v) / T, rtol=1e-12)
        assert np.isclose(u @ H[0, n] @ u, np.sum((Xq[:, sl] @ u) ** 2) / T, rtol=1e-12)
    H2, P2 = oracle.accumulate_act_aware(X, Xq, off, beta=0.5, H_prev=H, P_prev=P)
    np.testing.assert_allclose(H2, 1.5 * H, rtol=1e-14)
    np.testing.assert_allclose(P2, 1.5 * P, rtol=1e-14)
    Hx, Px = oracle.accumulate_act_aware(X, X, off)
    assert np.all(Px == 0)                                   # X_q = X => P = 0


def test_empty_group_gives_zero_sums():
    X = rng(5).standard_normal((10, 16))
    H, imp = oracle.accumulate(X, np.array([0, 0, 10, 10]), want_imp=True)
    assert np.all(H[0] == 0) and np.all(H[2] == 0) and np.all(imp[0] == 0)
    assert np.any(H[1] != 0)


# ------------------------------------------------------------------ P3: expanded output-MSE identity
@pytest.mark.parametrize("cin,act", [(16, False), (16, True), (48, False), (48, True)])
def test_objective_equals_output_mse_minus_constant(cin, act):
    r = rng(6, cin, int(act))
    T, cout = 37, 5
    X = r.standard_normal((T, cin))
    Xq = (X + 0.15 * r.standard_normal((T, cin))) if act else X.copy()
    W = r.normal(0, 0.02, (1, cout, cin))
    amax = oracle.absmax(W)
    g = oracle.global_scale(amax)[0]
    if act:
        H, P = oracle.accumulate_act_aware(X, Xq, np.array([0, T]))
    else:
        H, _ = oracle.accumulate(X, np.array([0, T]))
        P = None
    s = oracle.candidate_scales(g)
    saw_negative = False
    for c in range(cout):
        for n in range(cin // 16):
            sl = slice(16 * n, 16 * n + 16)
            w0 = W[0, c, sl]
            L, Q, C = oracle.candidate_losses(w0[None], [g], H[0, n][None],
                                              None if P is None else P[0, n][None])
            direct = np.empty(126)
            for k in range(126):
                _, wq, _ = oracle.fake_quant(w0, s[k])
                y = Xq[:, sl] @ wq - X[:, sl] @ w0
                direct[k] = y @ y / T
            const = np.sum(((Xq - X)[:, sl] @ w0) ** 2) / T
            np.testing.assert_allclose(L[0] + const, direct, rtol=1e-10, atol=1e-14)
            saw_negative |= bool(np.any(L[0] < 0))
            res = oracle.sweep_blocks(w0[None], [g], H[0, n][None], None if P is None else P[0, n][None])
            kd = int(np.argmin(direct))
            if abs(np.sort(direct)[1] - direct[kd]) > 1e-9 * abs(direct[kd]):
                assert res["code"][0] == kd + 1
    if act:
        assert saw_negative, "the activation-aware objective should go negative on some candidate"


# ------------------------------------------------------------------ P4: diagonal equivalence
def test_diagonal_hessian_equals_wmse_form():
    r = rng(7)
    G, cout, cin = 2, 12, 64
    W = r.normal(0, 0.02, (G, cout, cin))
    imp = r.uniform(0.1, 50.0, (G, cin))
    imp[1, :16] = 0.0                                       # a dead block: both sides use 1
    H = np.zeros((G, cin // 16, 16, 16))
    for gi in range(G):
        for n in range(cin // 16):
            H[gi, n] = np.diag(imp[gi, 16 * n:16 * n + 16])
    amax = oracle.absmax(W)
    a = oracle.sweep(W, amax, H)
    b = oracle.sweep_diag(W, amax, imp)
    np.testing.assert_array_equal(a["code"], b["code"])
    np.testing.assert_array_equal(a["fp4"], b["fp4"])
    np.testing.assert_allclose(a["loss"], b["loss"], rtol=1e-12)


def test_diag_of_hessian_scales_by_token_count():
    r = rng(8)
    T, cin, cout = 29, 32, 6
    X = r.standard_normal((T, cin))
    W = r.normal(0, 0.02, (1, cout, cin))
    H, imp = oracle.accumulate(X, np.array([0, T]), want_imp=True)
    Hd = np.zeros_like(H)
    for n in range(cin // 16):
        Hd[0, n] = np.diag(np.diag(H[0, n]))
    amax = oracle.absmax(W)
    a = oracle.sweep(W, amax, Hd)
    b = oracle.sweep_diag(W, amax, imp)
    np.testing.assert_array_equal(a["code"], b["code"])
    np.testing.assert_allclose(b["loss"], T * a["loss"], rtol=1e-12)


# ------------------------------------------------------------------ P5: H = I is the plain MSE search
def _scalar_quant(w, s):
    """Independent scalar E2M1 rounding through the midpoint thresholds."""
    if s == 0:
        return 0.0
    a = abs(w)
    mids_down = [(0.25, 0), (1.25, 2), (2.5, 4), (5.0, 6)]      # ties go to the lower (even) index
    mids_up = [(0.75, 2), (1.75, 4), (3.5, 6)]                  # ties go to the upper (even) index
    c = 0
    for m, _ in mids_down:
        c += Fraction(a) > Fraction(m) * Fraction(s)
    for m, _ in mids_up:
        c += Fraction(a) >= Fraction(m) * Fraction(s)
    v = [0, 0.5, 1, 1.5, 2, 3, 4, 6][c] * s
    return -v if w < 0 else v


def test_identity_hessian_is_plain_weight_mse():
    r = rng(9)
    cout, cin = 6, 32
    W = r.normal(0, 0.02, (1, cout, cin))
    H = np.broadcast_to(np.eye(16), (1, cin // 16, 16, 16)).copy()
    res = oracle.sweep(W, oracle.absmax(W), H)
    g = float(oracle.global_scale(oracle.absmax(W))[0])
    s = oracle.candidate_scales(g)
    for c in range(cout):
        for n in range(cin // 16):
            w = W[0, c, 16 * n:16 * n + 16]
            best, bk = np.inf, -1
            for k in range(126):
                err = sum((_scalar_quant(x, s[k]) - x) ** 2 for x in w)
                if err < best:
                    best, bk = err, k
            assert res["code"][0, c, n] == bk + 1
            assert np.isclose(res["loss"][0, c, n], best, rtol=1e-12)
    # the diagonal form with unit importance is the same plain MSE (the lh_scale_sweep_mse mode)
    d = oracle.sweep_diag(W, oracle.absmax(W), np.ones((1, cin)))
    np.testing.assert_array_equal(d["code"], res["code"])
    np.testing.assert_array_equal(d["fp4"], res["fp4"])
    np.testing.assert_allclose(d["loss"], res["loss"], rtol=1e-12)


# ------------------------------------------------------------------ P6: invariances
def test_invariances():
    r = rng(10)
    T, cout, cin = 64, 10, 48
    X = r.standard_normal((T, cin))
    Xq = X + 0.1 * r.standard_normal((T, cin))
    W = r.normal(0, 0.02, (1, cout, cin))
    off = np.array([0, T])
    H, P = oracle.accumulate_act_aware(X, Xq, off)
    amax = oracle.absmax(W)
    base = oracle.sweep(W, amax, H, P)
    # common positive scale of H and P
    a = oracle.sweep(W, amax, 3.7 * H, 3.7 * P)
    np.testing.assert_array_equal(a["code"], base["code"])
    # X scaled by 2^j
    H2, P2 = oracle.accumulate_act_aware(4 * X, 4 * Xq, off)
    np.testing.assert_array_equal(oracle.sweep(W, amax, H2, P2)["code"], base["code"])
    # W scaled by 2^j: the global scale, candidates and quotients scale exactly
    b = oracle.sweep(8 * W, oracle.absmax(8 * W), H, P)
    np.testing.assert_array_equal(b["code"], base["code"])
    np.testing.assert_array_equal(b["fp4"], base["fp4"])
    np.testing.assert_allclose(b["loss"], 64 * base["loss"], rtol=1e-12)
    # output-row permutation
    perm = r.permutation(cout)
    c = oracle.sweep(W[:, perm], amax, H, P)
    np.testing.assert_array_equal(c["code"], base["code"][:, perm])
    # X_q = X makes the act-aware search the plain one
    Hx, Px = oracle.accumulate_act_aware(X, X, off)
    Hp, _ = oracle.accumulate(X, off)
    np.testing.assert_array_equal(oracle.sweep(W, amax, Hx, Px)["code"], oracle.sweep(W, amax, Hp)["code"])


# ------------------------------------------------------------------ P7: grouped == per-group
def test_grouped_equals_per_group():
    wl = synth.make("c5", n_groups=6, cout=8, cin=32, tokens=60, topk=2)
    X, off = wl.X_f64(), wl.offsets
    W = wl.W_f64()
    H, imp = oracle.accumulate(X, off, want_imp=True)
    res = oracle.sweep(W, oracle.absmax(W), H)
    for g in range(wl.n_groups):
        Xg = X[off[g]:off[g + 1]]
        Hg, ig = oracle.accumulate(Xg, np.array([0, len(Xg)]), want_imp=True)
        np.testing.assert_array_equal(Hg[0], H[g])
        np.testing.assert_array_equal(ig[0], imp[g])
        rg = oracle.sweep(W[g:g + 1], oracle.absmax(W[g:g + 1]), Hg)
        np.testing.assert_array_equal(rg["code"][0], res["code"][g])
        np.testing.assert_array_equal(rg["fp4"][0], res["fp4"][g])


# ------------------------------------------------------------------ P8: non-vacuity
def test_hessian_changes_codes_against_plain_mse():
    wl = synth.make("c2", cout=64, cin=256, rows=512)
    X, W = wl.X_f64(), wl.W_f64()
    H, _ = oracle.accumulate(X, wl.offsets)
    amax = oracle.absmax(W)
    a = oracle.sweep(W, amax, H)["code"]
    eye = np.broadcast_to(np.eye(16), H.shape).copy()
    b = oracle.sweep(W, amax, eye)["code"]
    frac = np.mean(a != b)
    assert frac > 0.05, frac


# ------------------------------------------------------------------ P9: optimality re-check
def test_winner_is_optimal_on_independent_reevaluation():
    r = rng(11)
    B = 40
    w = r.normal(0, 0.02, (B, 16))
    g = oracle.global_scale(np.full(B, 0.1))
    A = r.standard_normal((B, 16, 16))
    H = np.einsum("bij,bkj->bik", A, A) / 16
    P = 0.1 * r.standard_normal((B, 16, 16))
    res = oracle.sweep_blocks(w, g, H, P)
    for b in range(B):
        s = oracle.candidate_scales(g[b])
        bias = P[b] @ w[b]
        Ls = []
        for k in range(126):
            e = np.array([_scalar_quant(x, s[k]) for x in w[b]]) - w[b]
            Ls.append(float(e @ H[b] @ e + 2 * e @ bias))
        kbest = int(np.argmin(Ls))
        assert res["code"][b] == kbest + 1
        assert np.isclose(res["loss"][b], Ls[kbest], rtol=1e-10, atol=1e-18)


# ------------------------------------------------------------------ degenerate blocks
def test_degenerate_blocks():
    w = np.zeros((3, 16))
    w[1] = np.linspace(-0.05, 0.05, 16)
    g = oracle.global_scale(np.array([0.1, 0.1, 0.0]))
    H = np.zeros((3, 16, 16))                                 # zero trace: plain MSE
    res = oracle.sweep_blocks(w, g, H)
    # all-zero block: every candidate scores 0, first (lowest) code wins, nibbles 0
    assert res["code"][0] == 1 and np.all(res["nib"][0] == 0) and res["loss"][0] == 0
    eye = np.broadcast_to(np.eye(16), (1, 16, 16))
    ref = oracle.sweep_blocks(w[1:2], g[1:2], eye)
    assert res["code"][1] == ref["code"][0]
    # zero global scale (all-zero matrix): all scales 0 -> everything quantizes to 0, code 1
    assert res["code"][2] == 1 and np.all(res["nib"][2] == 0)


def test_exemption_rule_flags_true_ties_only():
    res = dict(L1=np.array([1.0, 1.0, -1e-3]), L2=np.array([1.0 + 5e-7, 1.1, -1e-3 + 1e-10]),
               Q1=np.array([1.0, 1.0, 0.5]), C1=np.array([0.0, 0.0, -0.501]),
               Q2=np.array([1.0, 1.1, 0.5]), C2=np.array([0.0, 0.0, -0.501]))
    np.testing.assert_array_equal(oracle.exempt_mask(res), [True, False, True])


# ------------------------------------------------------------------ input generator determinism
def test_generator_is_deterministic_and_shaped():
    a = synth.make("c1")
    b = synth.make("c1")
    assert a.sha256() == b.sha256()
    assert a.W.shape == (1, 64, 128) and a.X.shape == (256, 128) and a.W.dtype == np.float32
    with open(os.path.join(GOLDEN, "synth_sha256.txt")) as f:
        want = dict(line.split() for line in f if line.strip() and not line.startswith("#"))
    assert a.sha256()["W"] == want["c1.W"] and a.sha256()["X"] == want["c1.X"]
    c = synth.make("c5", n_groups=8, cout=4, cin=32, tokens=100, topk=3)
    assert c.offsets[-1] == 300 and np.all(np.diff(c.offsets) >= 0)


# ------------------------------------------------------------------ activation fake-quant (X_q)
def test_e4m3_nearest_matches_library_encoder_and_saturates():
    """Block scales round like torch's float8_e4m3fn encoder (nearest, ties to even) on fp32
    inputs covering every binade, every midpoint and its float neighbours; above 448 they stay
    at 448 and below 2^-10 they flush to 0."""
    import torch
    values = np.concatenate([[0.0], oracle.e4m3_ladder()])
    mids = (values[:-1] + values[1:]) / 2
    r = np.random.default_rng(5)
    y = np.concatenate([np.exp2(r.uniform(-12, np.log2(448.0), 4000)), mids,
                        np.nextafter(mids.astype(np.float32), np.float32(0)),
                        np.nextafter(mids.astype(np.float32), np.float32(1e9)), values])
    y = y.astype(np.float32).astype(np.float64)
    y = y[y <= 448.0]
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.e4m3_nearest(y), ref)
    assert np.all(oracle.e4m3_nearest(np.array([448.0, 450.0, 464.0, 1e6])) == 448.0)
    assert oracle.e4m3_nearest(np.array([2.0 ** -10]))[0] == 0.0          # tie to even code 0
    assert oracle.e4m3_nearest(np.array([2.0 ** -10 * 1.0001]))[0] == 2.0 ** -9


def _exact_act_fq(x, amax, bf16):
    """One row's X_q by exact rational arithmetic (brute force over every E4M3 and E2M1 value)."""
    import math
    import torch
    gx = Fraction(float(np.float32(Fraction(amax) / 2688)))
    vals = [Fraction(0)] + [Fraction(v) for v in oracle.e4m3_ladder()]
    grid = [Fraction(v) for v in oracle.E2M1_GRID]
    out = []
    for blk in np.asarray(x).reshape(-1, 16):
        am = max(abs(Fraction(float(t))) for t in blk)
        y = am / (6 * gx) if gx else Fraction(0)
        d = [abs(y - v) for v in vals]
        best = min(d)
        code = [k for k in range(127) if d[k] == best]
        code = [k for k in code if k % 2 == 0] or code
        s = Fraction(float(np.float32(vals[code[0]] * gx)))
        for t in blk:
            if s == 0:
                out.append(math.copysign(0.0, float(t)))
                continue
            rr = abs(Fraction(float(t))) / s
            dg = [abs(rr - gv) for gv in grid]
            m = min(dg)
            c = [k for k in range(8) if dg[k] == m]
            c = [k for k in c if k % 2 == 0] or c
            q = float(np.float32(float(grid[c[0]] * s)))
            out.append(math.copysign(q, float(t)))           # the sign bit of x, -0 included
    out = np.array(out, dtype=np.float32)
    if bf16:
        out = torch.from_numpy(out).to(torch.bfloat16).to(torch.float32).numpy()
    return out.astype(np.float64)


@pytest.mark.parametrize("bf16", [True, False])
def test_activation_fake_quant_matches_exact_rationals(bf16):
    r = np.random.default_rng(9 + bf16)
    x = (r.standard_t(4, size=(6, 64)) * 0.7).astype(np.float32)
    x[1, :16] = 0.0                                  # zero block
    x[2, 16:32] *= 1e-4                              # block far below the global scale
    x[3, 32:48] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5] * 2, dtype=np.float32)
    x[4] = -x[4]
    x[5, 48:52] = -0.0                               # negative zeros keep their sign
    x[5, 52:56] = -1e-9                              # tiny negatives quantize to -0
    if bf16:
        x = synth.f32_from_bf16_bits(synth.bf16_bits_from_f32(x))
    amax = float(np.abs(x).max())
    for a in (amax, amax / 3.0, 0.0):                 # the second saturates some blocks at 448
        got = oracle.activation_fake_quant(x.astype(np.float64), [a], np.array([0, 6]), bf16=bf16)
        for row in range(6):
            want = _exact_act_fq(x[row], a, bf16)
            np.testing.assert_array_equal(got[row], want)
            np.testing.assert_array_equal(np.signbit(got[row]), np.signbit(want))
    zero = oracle.activation_fake_quant(x.astype(np.float64), [0.0], np.array([0, 6]), bf16)
    assert np.all(zero == 0.0) and np.array_equal(np.signbit(zero), np.signbit(x))


def test_activation_fake_quant_is_on_the_grid_and_per_group():
    r = np.random.default_rng(4)
    X = r.normal(0, 1, (40, 32)).astype(np.float32).astype(np.float64)
    off = np.array([0, 10, 10, 40])
    amax = np.array([np.abs(X[:10]).max(), 1.0, 0.5 * np.abs(X[10:]).max()])
    Q = oracle.activation_fake_quant(X, amax, off, bf16=False)
    for g in range(3):
        sub = oracle.activation_fake_quant(X[off[g]:off[g + 1]], amax[g:g + 1], np.array([0, off[g + 1] - off[g]]), False)
        np.testing.assert_array_equal(Q[off[g]:off[g + 1]], sub)
    assert np.all(np.sign(Q) * np.sign(X) >= 0)      # never flips a sign


# ------------------------------------------------------------------ dequantized weights
@pytest.mark.parametrize("bf16", [True, False])
def test_dequantize_reproduces_fake_quant_of_the_chosen_scale(bf16):
    """Decoding codes and packed nibbles gives back, element for element, the fake-quantized
    block that the search scored (fake_quant at the chosen scale, rounded to the storage type);
    block amax is 6 s and bounds every |Wq| of the block."""
    import torch
    r = np.random.default_rng(13)
    G, cout, cin = 2, 5, 48
    W = r.normal(0, 0.02, (G, cout, cin))
    W[0, 1, :16] = 0.0
    W[1, 2, 3] = -1e-12                            # quantizes to -0
    amax = oracle.absmax(W).astype(np.float32)
    code = r.integers(1, 127, size=(G, cout, cin // 16)).astype(np.uint8)
    s = oracle.candidate_scales(oracle.global_scale(amax.astype(np.float64)))       # [G, 126]
    sb = np.take_along_axis(s, code.reshape(G, -1).astype(np.int64) - 1, axis=1).reshape(G, cout, -1)
    nib, wq, _ = oracle.fake_quant(W.reshape(G, cout, -1, 16), sb[..., None])
    fp4 = oracle.pack_nibbles(nib.reshape(G, cout, cin))
    Wq, bam = oracle.dequantize(code, fp4, amax, bf16=bf16)
    ref = wq.reshape(G, cout, cin).astype(np.float32)
    if bf16:
        ref = torch.from_numpy(ref).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(Wq, ref.astype(np.float64))
    assert np.signbit(Wq[1, 2, 3]) and Wq[1, 2, 3] == 0.0
    np.testing.assert_array_equal(bam, (6.0 * sb).astype(np.float32).astype(np.float64))
    assert np.all(np.abs(Wq).reshape(G, cout, -1, 16).max(axis=-1) <= bam * (1 + 2 ** -7))


# ------------------------------------------------------------------ 256-normalized ("4/6") scaling
def test_global_scale_256_normalized_is_fp32_rounding():
    """norm 256: g = fp32(amax / (6 * 256)) correctly rounded, for many amax."""
    r = rng(31)
    for amax in np.float32(r.uniform(1e-3, 10.0, 200)):
        want = np.float32(Fraction(float(amax)) / 1536)
        assert oracle.global_scale(amax, 256.0) == np.float64(want)
    assert oracle.global_scale(np.float32(3.0), 256.0) == 3.0 / 1536


def test_256_normalization_equals_448_with_scaled_amax():
    """The global scale is all the normalization changes: amax / (6*256) = (7/4 amax) / (6*448), so
    with 7/4 amax exact in fp32 the 256-normalized search equals the 448 one on 7/4 amax (codes,
    nibbles, losses), for the full and the diagonal form; and it differs from the 448 search on
    the same amax for some blocks."""
    wl = synth.make("c2", cout=24, cin=64, rows=200)
    W, X = wl.W_f64(), wl.X_f64()
    H, imp = oracle.accumulate(X, wl.offsets, want_imp=True)
    amax = oracle.absmax(W).astype(np.float32)                # bf16 values: 7/4 amax is exact
    amax7 = (amax * np.float32(1.75)).astype(np.float64)
    assert Fraction(float(amax7[0])) == Fraction(7, 4) * Fraction(float(amax[0]))
    a = oracle.sweep(W, amax, H, norm=256.0)
    b = oracle.sweep(W, amax7, H, norm=448.0)
    for k in ("code", "fp4", "loss"):
        np.testing.assert_array_equal(a[k], b[k])
    c = oracle.sweep(W, amax, H)
    assert np.any(a["code"] != c["code"])
    ad = oracle.sweep_diag(W, amax, imp, norm=256.0)
    bd = oracle.sweep_diag(W, amax7, imp, norm=448.0)
    np.testing.assert_array_equal(ad["code"], bd["code"])
    np.testing.assert_array_equal(ad["fp4"], bd["fp4"])
    # dequantize follows the same scale
    Wq, bam = oracle.dequantize(a["code"], a["fp4"], amax, bf16=True, norm=256.0)
    Wq7, bam7 = oracle.dequantize(b["code"], b["fp4"], amax7, bf16=True)
    np.testing.assert_array_equal(Wq, Wq7)
    np.testing.assert_array_equal(bam, bam7)


# ------------------------------------------------------------------ amax-multiplier search
def _exact_code(a, m, g):
    """Nearest of the 126 positive E4M3 values to a*m/(6g), ties to the even code, by rationals."""
    y = Fraction(float(a)) * Fraction(float(m)) / (6 * Fraction(float(g)))
    vals = [Fraction(float(v)) for v in oracle.e4m3_ladder()]
    d = [abs(y - v) for v in vals]
    best = min(d)
    ks = [k + 1 for k in range(126) if d[k] == best]
    even = [k for k in ks if k % 2 == 0]
    return even[0] if even else ks[0]


def test_multiplier_codes_match_exact_rationals():
    """Random blocks and multipliers, exact midpoints (ties go to the even code) and their float
    neighbours, saturation at 448 and at 2^-9, and an all-zero block."""
    r = rng(32)
    a = np.float32(r.uniform(1e-3, 0.2, 60)).astype(np.float64)
    g = np.float32(r.uniform(1e-5, 1e-4, 60)).astype(np.float64)
    m = np.float32(r.uniform(0.2, 3.0, 12)).astype(np.float64)
    got = oracle.multiplier_codes(a, g, m)
    for b in range(0, 60, 3):
        for j in range(12):
            assert got[b, j] == _exact_code(a[b], m[j], g[b])
    # exact midpoints y = (v_k + v_k+1)/2 with a = 6 g y exactly, m = 1, and their neighbours
    lad = oracle.e4m3_ladder()
    gg = 2.0 ** -10
    ys = (lad[:-1] + lad[1:]) / 2
    aa = []
    for y in ys:
        t = np.float32(6 * gg * y)
        aa += [float(t), float(np.nextafter(t, np.float32(1))), float(np.nextafter(t, np.float32(0)))]
    aa += [0.0, 1e-30, 1e6]                                  # zero block, underflow, saturation
    aa = np.array(aa)
    got = oracle.multiplier_codes(aa, np.full(len(aa), gg), np.array([1.0]))[:, 0]
    want = [_exact_code(x, 1.0, gg) for x in aa]
    np.testing.assert_array_equal(got, want)
    assert got[-3] == 1 and got[-2] == 1 and got[-1] == 126
    ties = got[0:3 * len(ys):3]
    assert np.all(ties % 2 == 0)                             # every exact midpoint went to the even code


def _dense_grid(lo=1e-7, hi=1e3, ratio=1.01):
    return np.float32(lo * ratio ** np.arange(int(np.log(hi / lo) / np.log(ratio)) + 1)).astype(np.float64)


def test_multiplier_search_with_a_covering_grid_is_the_full_sweep():
    """A grid dense enough to propose every code for every block turns the multiplier search into
    the 126-candidate sweep (full, coupled and diagonal forms)."""
    wl = synth.make("c2", cout=16, cin=48, rows=120)
    W, X = wl.W_f64(), wl.X_f64()
    W[0, 0, :16] = 0.0                                       # all-zero block: every code proposes 1
    Xq = X + 0.1 * rng(33).standard_normal(X.shape)
    H, P = oracle.accumulate_act_aware(X, Xq, wl.offsets)
    _, imp = oracle.accumulate(X, wl.offsets, want_h=False, want_imp=True)
    amax = oracle.absmax(W)
    grid = _dense_grid()
    g = oracle.global_scale(amax)
    blk_amax = np.abs(W.reshape(-1, 16)).max(axis=1)
    allowed = oracle.multiplier_allowed(blk_amax, np.repeat(g, len(blk_amax)), grid)
    assert allowed[blk_amax > 0].all()
    for a, b in ((oracle.sweep(W, amax, H, P, multipliers=grid), oracle.sweep(W, amax, H, P)),
                 (oracle.sweep_diag(W, amax, imp, multipliers=grid), oracle.sweep_diag(W, amax, imp))):
        np.testing.assert_array_equal(a["code"], b["code"])
        np.testing.assert_array_equal(a["fp4"], b["fp4"])
        np.testing.assert_array_equal(a["loss"], b["loss"])


def test_multiplier_search_against_scalar_reevaluation():
    """Each block's winner is the lowest-loss candidate over its multipliers' codes, re-evaluated
    by an independent scalar loop (quantizer and objective written out per element)."""
    r = rng(34)
    B = 30
    w = r.normal(0, 0.02, (B, 16))
    w[3] = 0.0
    g = oracle.global_scale(np.full(B, 0.1))
    A = r.standard_normal((B, 16, 16))
    H = np.einsum("bij,bkj->bik", A, A) / 16
    P = 0.1 * r.standard_normal((B, 16, 16))
    mult = np.float32(np.arange(0.5, 1.6, 0.1)).astype(np.float64)
    allowed = oracle.multiplier_allowed(np.abs(w).max(axis=1), g, mult)
    res = oracle.sweep_blocks(w, g, H, P, allowed=allowed)
    for b in range(B):
        s = oracle.candidate_scales(g[b])
        bias = P[b] @ w[b]
        best, kbest = np.inf, None
        for m in mult:
            k = _exact_code(np.abs(w[b]).max(), m, g[b])
            e = np.array([_scalar_quant(x, s[k - 1]) for x in w[b]]) - w[b]
            L = float(e @ H[b] @ e + 2 * e @ bias)
            if L < best or (L == best and k < kbest):
                best, kbest = L, k
        assert res["code"][b] == kbest, (b, res["code"][b], kbest)
        assert np.isclose(res["loss"][b], best, rtol=1e-10, atol=1e-18)
    assert res["code"][3] == 1
