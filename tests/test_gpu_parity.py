"""GPU parity: the HIP library (called through its C ABI) against the float64 oracle.

Sizes are small enough for the oracle to finish in seconds but span several accumulation tiles
(256 rows), several sweep workgroups (64 rows x 4 block columns), partial tiles and ragged tails.
Every case prints its name, seed and shapes before it touches the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import (assert_h_close, assert_imp_close, assert_p_close, assert_sweep_match,
                         cross_gram, with_oracle_xq)

pytestmark = pytest.mark.gpu

lh = pytest.importorskip("nvfp4_scale_calibration_lh_amd")
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def note(msg):
    print(f"[case] {msg}", flush=True)


def to_dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(DEV)


def upload(wl):
    W = to_dev(wl.W, wl.dtype)
    X = to_dev(wl.X, wl.dtype)
    Xq = to_dev(wl.Xq, wl.dtype) if wl.Xq is not None else None
    off = torch.from_numpy(wl.offsets).to(DEV) if wl.n_groups > 1 else None
    return W, X, Xq, off


SMALL = {
    "c1": dict(),
    "c2": dict(cout=150, cin=80, rows=600),
    "c3": dict(cout=70, cin=96, rows=530),
    "c4": dict(cout=130, cin=112, rows=300),
    "c5": dict(n_groups=12, cout=40, cin=64, tokens=400, topk=3),
}


# ------------------------------------------------------------------------------------ absmax
@pytest.mark.parametrize("name", list(SMALL))
def test_absmax_bit_exact(name):
    wl = synth.make(name, **SMALL[name])
    note(f"absmax {name} W{wl.W.shape}")
    W, _, _, _ = upload(wl)
    got = lh.lh_absmax(W).cpu().numpy()
    ref = oracle.absmax(wl.W_f64()).astype(np.float32)
    np.testing.assert_array_equal(got, ref)


def test_absmax_ragged_and_unaligned():
    r = np.random.default_rng(1)
    a = r.normal(0, 1, 3 * 1001).astype(np.float32)
    a[1500] = -77.0
    note("absmax ragged fp32 3x1001")
    t = torch.from_numpy(a).to(DEV).view(3, 1, 1001)          # 3 groups of 1001 elements
    np.testing.assert_array_equal(lh.lh_absmax(t).cpu().numpy(), np.abs(a.reshape(3, 1001)).max(1))
    b = synth.bf16_bits_from_f32(r.normal(0, 1, 2 * 37).astype(np.float32))
    tb = torch.from_numpy(b).view(torch.bfloat16).to(DEV).view(2, 1, 37)
    ref = np.abs(synth.f32_from_bf16_bits(b).reshape(2, 37)).max(1)
    np.testing.assert_array_equal(lh.lh_absmax(tb).cpu().numpy(), ref)


# ------------------------------------------------------------------------------------ accumulation
@pytest.mark.parametrize("name", ["c1", "c2", "c4", "c5"])
def test_accumulate_h_and_imp(name):
    wl = synth.make(name, **SMALL[name])
    note(f"accumulate {name} X{wl.X.shape} groups={wl.n_groups}")
    _, X, _, off = upload(wl)
    H, imp = lh.lh_accumulate(X, offsets=off, want_imp=True)
    H_ref, imp_ref = oracle.accumulate(wl.X_f64(), wl.offsets, want_imp=True)
    assert_h_close(H.cpu().numpy(), H_ref)
    assert_imp_close(imp.cpu().numpy(), imp_ref)


def test_accumulate_deterministic_and_only_imp():
    wl = synth.make("c2", cout=16, cin=128, rows=1000)
    note("accumulate determinism c2 rows=1000")
    _, X, _, _ = upload(wl)
    H1, i1 = lh.lh_accumulate(X, want_imp=True)
    H2, i2 = lh.lh_accumulate(X, want_imp=True)
    _, i3 = lh.lh_accumulate(X, want_h=False, want_imp=True)
    _, i4 = lh.lh_accumulate(X, want_h=False, want_imp=True)
    # bit-identical run to run for one call configuration
    assert torch.equal(H1, H2) and torch.equal(i1, i2) and torch.equal(i3, i4)
    # the importance-only path tiles the rows differently: same values up to fp32 summation order
    _, imp_ref = oracle.accumulate(wl.X_f64(), wl.offsets, want_h=False, want_imp=True)
    assert_imp_close(i3.cpu().numpy(), imp_ref)
    assert_imp_close(i1.cpu().numpy(), imp_ref)


def test_accumulate_empty_groups_and_beta():
    r = np.random.default_rng(5)
    rows, cin = 700, 48
    X = synth.bf16_bits_from_f32(r.normal(0, 1, (rows, cin)).astype(np.float32))
    off = np.array([0, 0, 5, 5, 300, 301, 700, 700], dtype=np.int64)   # empty, tiny, spans tiles
    note("accumulate groups with empty/one-row/tile-spanning members, beta streaming")
    Xd = torch.from_numpy(X).view(torch.bfloat16).to(DEV)
    offd = torch.from_numpy(off).to(DEV)
    Xf = synth.f32_from_bf16_bits(X).astype(np.float64)
    H_ref, imp_ref = oracle.accumulate(Xf, off, want_imp=True)
    H, imp = lh.lh_accumulate(Xd, offsets=offd, want_imp=True)
    assert_h_close(H.cpu().numpy(), H_ref)
    assert_imp_close(imp.cpu().numpy(), imp_ref)
    # streaming: second call with beta = 0.5 on the same data
    lh.lh_accumulate(Xd, H=H, imp=imp, offsets=offd, beta=0.5)
    H2_ref, imp2_ref = oracle.accumulate(Xf, off, beta=0.5, H_prev=H_ref, imp_prev=imp_ref, want_imp=True)
    assert_h_close(H.cpu().numpy(), H2_ref)
    assert_imp_close(imp.cpu().numpy(), imp2_ref)


def test_accumulate_two_streams_share_scratch():
    # the library's accumulation scratch is handed from call to call in stream order; calls that
    # alternate between two streams without any host synchronization must each give the result
    # of the same call made alone (multi-tile dense and grouped layers both use the scratch)
    r = np.random.default_rng(11)
    rows, cin = 3000, 320
    off = np.array([0, 40, 1500, 1510, 3000], dtype=np.int64)
    note(f"accumulate on two streams: X[{rows},{cin}] dense and 4 groups, 6 calls each")
    Xs = [torch.from_numpy(synth.bf16_bits_from_f32(r.normal(0, 1 + k, (rows, cin)).astype(np.float32)))
          .view(torch.bfloat16).to(DEV) for k in range(4)]
    offd = torch.from_numpy(off).to(DEV)
    alone = []
    for k, X in enumerate(Xs):
        o = offd if k % 2 else None
        H, imp = lh.lh_accumulate(X, offsets=o, want_imp=True)
        torch.cuda.synchronize()
        alone.append((H.clone(), imp.clone()))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]     # default priority
    torch.cuda.synchronize()
    outs = []
    for rep in range(3):
        for k, X in enumerate(Xs):
            with torch.cuda.stream(streams[(k + rep) % 2]):
                outs.append((k, lh.lh_accumulate(X, offsets=offd if k % 2 else None, want_imp=True)))
    torch.cuda.synchronize()
    for k, (H, imp) in outs:
        assert torch.equal(H, alone[k][0]) and torch.equal(imp, alone[k][1]), f"input {k} differs"


def test_accumulate_zero_rows():
    note("accumulate rows=0")
    X = torch.empty((0, 32), dtype=torch.bfloat16, device=DEV)
    H, imp = lh.lh_accumulate(X, want_imp=True)
    assert torch.count_nonzero(H) == 0 and torch.count_nonzero(imp) == 0


@pytest.mark.parametrize("name", ["c3", "c1"])
def test_accumulate_act_aware(name):
    if name == "c1":      # fp32 act-aware: X_q from a perturbation of X
        wl = synth.make("c1")
        r = np.random.default_rng(7)
        Xq = (wl.X + 0.05 * r.standard_normal(wl.X.shape)).astype(np.float32)
        wl.Xq = Xq
    else:
        wl = with_oracle_xq(synth.make(name, **SMALL[name]))
    note(f"act-aware accumulate {name} X{wl.X.shape}")
    _, X, Xq, off = upload(wl)
    H, P = lh.lh_accumulate_act_aware(X, Xq, offsets=off)
    H_ref, P_ref = oracle.accumulate_act_aware(wl.X_f64(), wl.Xq_f64(), wl.offsets)
    R_ref = cross_gram(wl.X_f64(), wl.Xq_f64(), wl.offsets)
    assert_h_close(H.cpu().numpy(), H_ref)
    assert_p_close(P.cpu().numpy(), P_ref, H_ref, R_ref)



@pytest.mark.parametrize("name", ["c1", "c3", "c5"])
def test_accumulate_act_aware_fused_fake_quant(name):
    """X_q made in the kernel from X and the input quantizer's amax: H and P against the oracle
    (its own activation fake-quant), and identical to the two-input kernel fed the oracle's X_q
    (same summation order), which holds only if every X_q element matches bit for bit."""
    wl = synth.make(name, **SMALL[name])
    G, bf16 = wl.n_groups, wl.dtype == "bf16"
    X64 = wl.X_f64()
    amax = np.array([np.abs(X64[wl.offsets[g]:wl.offsets[g + 1]]).max(initial=0.0) for g in range(G)])
    if G > 2:
        amax[1] *= 0.25                     # blocks of this group saturate at 448
        amax[2] = 0.0                       # X_q = 0 for this group
    amax = amax.astype(np.float32)
    note(f"fused fake-quant accumulate {name} X{wl.X.shape} G={G} dtype={wl.dtype}")
    _, X, _, off = upload(wl)
    H, P = lh.lh_accumulate_act_aware_fq(X, torch.from_numpy(amax).to(DEV), offsets=off)
    Xq64 = oracle.activation_fake_quant(X64, amax.astype(np.float64), wl.offsets, bf16=bf16)
    H_ref, P_ref = oracle.accumulate_act_aware(X64, Xq64, wl.offsets)
    R_ref = cross_gram(X64, Xq64, wl.offsets)
    assert_h_close(H.cpu().numpy(), H_ref)
    assert_p_close(P.cpu().numpy(), P_ref, H_ref, R_ref)
    Xq_store = synth.bf16_bits_from_f32(Xq64.astype(np.float32)) if bf16 else Xq64.astype(np.float32)
    H2, P2 = lh.lh_accumulate_act_aware(X, to_dev(Xq_store, wl.dtype), offsets=off)
    assert torch.equal(H, H2) and torch.equal(P, P2)


def test_accumulate_fused_fake_quant_beta_and_zero_rows():
    wl = synth.make("c3", **SMALL["c3"])
    _, X, _, _ = upload(wl)
    amax = torch.tensor([float(np.abs(wl.X_f64()).max())], dtype=torch.float32, device=DEV)
    note("fused fake-quant accumulate: beta and zero rows")
    H, P = lh.lh_accumulate_act_aware_fq(X, amax)
    H0, P0 = H.clone(), P.clone()
    H, P = lh.lh_accumulate_act_aware_fq(X, amax, H=H, P=P, beta=1.0)
    torch.testing.assert_close(H, 2 * H0, rtol=1e-6, atol=0)
    torch.testing.assert_close(P, 2 * P0, rtol=1e-6, atol=0)
    lh.lh_accumulate_act_aware_fq(X[:0], amax, H=H, P=P, beta=0.5)
    torch.testing.assert_close(H, H0, rtol=1e-6, atol=0)

@pytest.mark.parametrize("name", ["c3", "c1", "c5"])
def test_activation_fake_quant_entry_point(name):
    """lh_activation_fake_quant writes, bit for bit, the oracle's X_q (per-group amax, one group
    saturating at 448 and one at amax 0), and the two-input accumulation fed that X_q equals the
    fused one value for value."""
    wl = synth.make(name, **SMALL[name])
    G, bf16 = wl.n_groups, wl.dtype == "bf16"
    plant = np.float32([-0.0, -1e-9, 1e-9, 0.0])          # signed zeros and values that quantize to 0
    xs = synth.f32_from_bf16_bits(wl.X) if bf16 else wl.X.copy()
    xs[::7, 5] = plant[np.arange(xs[::7].shape[0]) % 4]
    wl.X = synth.bf16_bits_from_f32(xs) if bf16 else xs
    X64 = wl.X_f64()
    amax = np.array([np.abs(X64[wl.offsets[g]:wl.offsets[g + 1]]).max(initial=0.0) for g in range(G)])
    if G > 2:
        amax[1] *= 0.25
        amax[2] = 0.0
    amax = amax.astype(np.float32)
    note(f"activation fake-quant {name} X{wl.X.shape} G={G} dtype={wl.dtype}")
    _, X, _, off = upload(wl)
    am = torch.from_numpy(amax).to(DEV)
    Xq = lh.lh_activation_fake_quant(X, am, offsets=off)
    ref = oracle.activation_fake_quant(X64, amax.astype(np.float64), wl.offsets, bf16=bf16)
    got = Xq.float().cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(got, ref)
    # zeros carry the sign bit of x (-0 for -0 and for a negative x that quantizes to 0)
    np.testing.assert_array_equal(np.signbit(got), np.signbit(ref))
    H1, P1 = lh.lh_accumulate_act_aware(X, Xq, offsets=off)
    H2, P2 = lh.lh_accumulate_act_aware_fq(X, am, offsets=off)
    assert torch.equal(H1, H2) and torch.equal(P1, P2)


@pytest.mark.parametrize("bf16", [True, False])
def test_activation_fake_quant_block_scale_ties(bf16):
    """Block maxima placed exactly on every E4M3 midpoint of max|x| / (6 gX) (gX = 2^-8, so each
    one is a short binary fraction, exact in bf16) and one bf16 step either side: the block scale
    is the tie's even code or the nearer neighbour, as the oracle decides it, in the standalone
    fake-quant and in the fused accumulation (equal to the two-input kernel fed the oracle's X_q)."""
    gx = 2.0 ** -8
    amax = np.float32(2688.0 * gx)                     # fp32(amax / 2688) = gX exactly
    lad = oracle.e4m3_ladder()
    mids = np.concatenate([[lad[0] / 2], (lad[:-1] + lad[1:]) / 2])   # 126 midpoints from 2^-10
    peak = mids * 6.0 * gx
    step = 2.0 ** (np.floor(np.log2(peak)) - 7)        # one bf16 unit at each peak
    peaks = np.concatenate([peak, peak + step, peak - step])
    rng = np.random.default_rng(58)
    nblk = 4
    rows = (len(peaks) + nblk - 1) // nblk
    X = rng.uniform(-0.9, 0.9, size=(rows, nblk * 16))
    pk = np.resize(peaks, rows * nblk).reshape(rows, nblk)
    X *= np.repeat(pk, 16, axis=1)
    X[:, ::16] = pk * np.where(rng.random((rows, nblk)) < 0.5, -1.0, 1.0)   # the block maximum
    if bf16:
        bits = synth.bf16_bits_from_f32(X.astype(np.float32))
        X64 = synth.f32_from_bf16_bits(bits).astype(np.float64)
        assert np.array_equal(np.abs(X64[:, ::16]), pk), "planted maxima are not exact bf16 values"
        Xd = to_dev(bits, "bf16")
    else:
        X64 = X.astype(np.float32).astype(np.float64)
        Xd = to_dev(X64.astype(np.float32), "f32")
    note(f"activation fake-quant block-scale ties bf16={bf16} X[{rows},{nblk * 16}]")
    off = np.array([0, rows], dtype=np.int64)
    am = torch.tensor([amax], device=DEV)
    Xq = lh.lh_activation_fake_quant(Xd, am)
    ref = oracle.activation_fake_quant(X64, np.array([float(amax)]), off, bf16=bf16)
    np.testing.assert_array_equal(Xq.float().cpu().numpy().astype(np.float64), ref)
    H1, P1 = lh.lh_accumulate_act_aware_fq(Xd, am)
    Xq_store = synth.bf16_bits_from_f32(ref.astype(np.float32)) if bf16 else ref.astype(np.float32)
    H2, P2 = lh.lh_accumulate_act_aware(Xd, to_dev(Xq_store, "bf16" if bf16 else "f32"))
    assert torch.equal(H1, H2) and torch.equal(P1, P2)


@pytest.mark.parametrize("bf16", [True, False])
def test_accumulate_act_aware_unrelated_xq(bf16):
    """X_q far from X: a 9-12 binade gap (D with more than 16 significant bits), blocks where
    X_q or X is zero, and X_q larger than X.  H and P within the 1e-5 Cauchy-Schwarz tolerance."""
    r = np.random.default_rng(17)
    rows, cin = 700, 96
    X = r.normal(0, 1, (rows, cin)).astype(np.float32)
    Xq = X * np.float32(2.0 ** -12) * (1 + r.integers(0, 7, (rows, cin))).astype(np.float32)
    X[:, 1] = 1.0078125                          # the case 1 + 2^-7 against X * 2^-12
    Xq[:, 1] = np.float32(1.0078125 * 2 ** -12)
    Xq[:, 16:32] = 0.0                           # X_q zero block
    X[:, 32:48] = 0.0                            # X zero block (D = X_q)
    Xq[:, 48:64] = X[:, 48:64] * np.float32(512.0)   # X_q 9 binades above X
    Xq[100:200, 64:80] = X[100:200, 64:80]       # rows where D = 0
    if bf16:
        Xs, Xqs = synth.bf16_bits_from_f32(X), synth.bf16_bits_from_f32(Xq)
        X64, Xq64 = synth.f32_from_bf16_bits(Xs).astype(np.float64), synth.f32_from_bf16_bits(Xqs).astype(np.float64)
        dt = "bf16"
    else:
        Xs, Xqs, X64, Xq64, dt = X, Xq, X.astype(np.float64), Xq.astype(np.float64), "f32"
    off = np.array([0, rows])
    note(f"act-aware accumulate, X_q unrelated to X, bf16={bf16}")
    H, P = lh.lh_accumulate_act_aware(to_dev(Xs, dt), to_dev(Xqs, dt))
    H_ref, P_ref = oracle.accumulate_act_aware(X64, Xq64, off)
    R_ref = cross_gram(X64, Xq64, off)
    assert_h_close(H.cpu().numpy(), H_ref)
    assert_p_close(P.cpu().numpy(), P_ref, H_ref, R_ref)
    # the same through the grouped kernel (rows split into three experts)
    offg = np.array([0, 250, 250, rows])
    Hg, Pg = lh.lh_accumulate_act_aware(to_dev(Xs, dt), to_dev(Xqs, dt), offsets=torch.from_numpy(offg).to(DEV))
    H_ref, P_ref = oracle.accumulate_act_aware(X64, Xq64, offg)
    R_ref = cross_gram(X64, Xq64, offg)
    assert_h_close(Hg.cpu().numpy(), H_ref)
    assert_p_close(Pg.cpu().numpy(), P_ref, H_ref, R_ref)


# ------------------------------------------------------------------------------------ sweep
def _oracle_h32(wl):
    """fp32 Hessians computed by the oracle: the identical input both sweeps receive."""
    if wl.mode == "act":
        H, P = oracle.accumulate_act_aware(wl.X_f64(), wl.Xq_f64(), wl.offsets)
        return H.astype(np.float32), P.astype(np.float32)
    H, _ = oracle.accumulate(wl.X_f64(), wl.offsets)
    return H.astype(np.float32), None


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c5"])
def test_sweep_full_parity(name):
    wl = with_oracle_xq(synth.make(name, **SMALL[name]))
    note(f"sweep {name} W{wl.W.shape} mode={wl.mode}")
    W, _, _, _ = upload(wl)
    H32, P32 = _oracle_h32(wl)
    amax = oracle.absmax(wl.W_f64()).astype(np.float32)
    code, fp4, loss = lh.lh_scale_sweep(W, torch.from_numpy(amax).to(DEV), torch.from_numpy(H32).to(DEV),
                                        None if P32 is None else torch.from_numpy(P32).to(DEV))
    res = oracle.sweep(wl.W_f64(), amax, H32, P32)
    n_ex = assert_sweep_match(code.cpu().numpy(), fp4.cpu().numpy(), loss.cpu().numpy(), res)
    note(f"  exempt near-ties: {n_ex} of {code.numel()}")


def test_sweep_diag_parity():
    wl = synth.make("c4", **SMALL["c4"])
    note(f"diag sweep c4 W{wl.W.shape}")
    W, _, _, _ = upload(wl)
    _, imp = oracle.accumulate(wl.X_f64(), wl.offsets, want_h=False, want_imp=True)
    imp32 = imp.astype(np.float32)
    amax = oracle.absmax(wl.W_f64()).astype(np.float32)
    code, fp4, loss = lh.lh_scale_sweep_diag(W, torch.from_numpy(amax).to(DEV), torch.from_numpy(imp32).to(DEV))
    res = oracle.sweep_diag(wl.W_f64(), amax, imp32)
    assert_sweep_match(code.cpu().numpy(), fp4.cpu().numpy(), loss.cpu().numpy(), res)


@pytest.mark.parametrize("bf16", [True, False])
def test_sweep_mse_parity(bf16):
    """Plain-MSE mode (no importance): the oracle's diagonal form with Imp = 1, and bit for bit the
    diagonal entry point given an all-ones importance; zero blocks and a ragged row count included."""
    r = np.random.default_rng(41)
    G, cout, cin = 2, 77, 96
    W = r.normal(0, 0.02, (G, cout, cin)).astype(np.float32)
    W[0, 3, 16:32] = 0.0
    W[1, :, :] *= 10.0
    if bf16:
        Wb = synth.bf16_bits_from_f32(W)
        W64 = synth.f32_from_bf16_bits(Wb).astype(np.float64)
        Wd = to_dev(Wb, "bf16")
    else:
        W64 = W.astype(np.float64)
        Wd = torch.from_numpy(W).to(DEV)
    amax = oracle.absmax(W64).astype(np.float32)
    ad = torch.from_numpy(amax).to(DEV)
    note(f"plain-MSE sweep bf16={bf16} G={G} cout={cout} cin={cin}")
    code, fp4, loss = lh.lh_scale_sweep_mse(Wd, ad)
    res = oracle.sweep_diag(W64, amax, np.ones((G, cin)))
    assert_sweep_match(code.cpu().numpy(), fp4.cpu().numpy(), loss.cpu().numpy(), res)
    c2, f2, l2 = lh.lh_scale_sweep_diag(Wd, ad, torch.ones((G, cin), device=DEV))
    assert torch.equal(code, c2) and torch.equal(fp4, f2) and torch.equal(loss, l2)


def test_sweep_degenerate_blocks():
    """All-zero blocks, zero-trace Hessians, an all-zero matrix (amax 0), ragged shapes."""
    r = np.random.default_rng(3)
    G, cout, cin = 3, 21, 48
    W = r.normal(0, 0.02, (G, cout, cin)).astype(np.float32)
    W[0, 3, 16:32] = 0.0                      # zero block
    W[1, :, :] *= 1e3                         # large weights
    W[2] = 0.0                                # amax 0 group
    W[0, 5, 0] = -0.0
    A = r.standard_normal((G, cin // 16, 16, 16)).astype(np.float32)
    H = np.einsum("gnij,gnkj->gnik", A, A).astype(np.float32) / 16
    H[0, 1] = 0.0                             # zero trace: plain MSE
    P = (0.1 * r.standard_normal(H.shape)).astype(np.float32)
    amax = oracle.absmax(W).astype(np.float32)
    note("sweep degenerate cases fp32 G=3 cout=21 cin=48")
    args = [torch.from_numpy(x).to(DEV) for x in (W, amax, H)]
    for with_p in (False, True):
        code, fp4, loss = lh.lh_scale_sweep(*args, torch.from_numpy(P).to(DEV) if with_p else None)
        res = oracle.sweep(W.astype(np.float64), amax, H, P if with_p else None)
        assert_sweep_match(code.cpu().numpy(), fp4.cpu().numpy(), loss.cpu().numpy(), res)
        assert np.all(code.cpu().numpy()[2] == 1) and np.all(fp4.cpu().numpy()[2] == 0)
    imp = np.abs(r.standard_normal((G, cin))).astype(np.float32)
    imp[1, 16:32] = 0.0
    code, fp4, loss = lh.lh_scale_sweep_diag(args[0], args[1], torch.from_numpy(imp).to(DEV))
    res = oracle.sweep_diag(W.astype(np.float64), amax, imp)
    assert_sweep_match(code.cpu().numpy(), fp4.cpu().numpy(), loss.cpu().numpy(), res)



def test_sweep_signed_zeros_bf16():
    """bf16 weights holding -0 and tiny values that quantize to zero at every candidate: the
    nibble is (w < 0) << 3 | index, so -0 encodes as 0x0 and a tiny negative as 0x8."""
    r = np.random.default_rng(21)
    G, cout, cin = 2, 70, 64
    W = r.normal(0, 0.02, (G, cout, cin)).astype(np.float32)
    cls = r.integers(0, 8, size=W.shape)      # disjoint classes of planted values
    W[cls == 0] = -0.0
    W[cls == 1] = -1e-9
    W[cls == 2] = 1e-9
    W[1, 9, 16:32] = -0.0                     # a block of -0 only
    cls[1, 9, 16:32] = 0
    Wb = synth.bf16_bits_from_f32(W)
    W64 = synth.f32_from_bf16_bits(Wb).astype(np.float64)
    amax = oracle.absmax(W64).astype(np.float32)
    A = r.standard_normal((G, cin // 16, 16, 16)).astype(np.float32)
    H = np.einsum("gnij,gnkj->gnik", A, A).astype(np.float32) / 16
    P = (0.1 * r.standard_normal(H.shape)).astype(np.float32)
    imp = np.abs(r.standard_normal((G, cin))).astype(np.float32)
    note(f"sweep signed zeros bf16 G={G} cout={cout} cin={cin}")
    Wd, ad = to_dev(Wb, "bf16"), torch.from_numpy(amax).to(DEV)
    for with_p in (False, True):
        code, fp4, loss = lh.lh_scale_sweep(Wd, ad, torch.from_numpy(H).to(DEV),
                                            torch.from_numpy(P).to(DEV) if with_p else None)
        res = oracle.sweep(W64, amax, H, P if with_p else None)
        nib = res["nib"].reshape(G, cout, cin)
        assert (nib[cls == 1] == 8).all() and (nib[cls == 0] == 0).all()
        assert_sweep_match(code.cpu().numpy(), fp4.cpu().numpy(), loss.cpu().numpy(), res)
    code, fp4, loss = lh.lh_scale_sweep_diag(Wd, ad, torch.from_numpy(imp).to(DEV))
    res = oracle.sweep_diag(W64, amax, imp)
    assert_sweep_match(code.cpu().numpy(), fp4.cpu().numpy(), loss.cpu().numpy(), res)


@pytest.mark.parametrize("name", ["c2", "c5"])
def test_dequantize_matches_oracle(name):
    """Fake-quantized weights and block amax from the GPU sweep's own codes and nibbles, bit for
    bit against the oracle's decoding, in bf16 and fp32."""
    wl = synth.make(name, **SMALL[name])
    note(f"dequantize {name} W{wl.W.shape}")
    W, _, _, _ = upload(wl)
    H32, P32 = _oracle_h32(wl)
    amax = torch.from_numpy(oracle.absmax(wl.W_f64()).astype(np.float32)).to(DEV)
    code, fp4, _ = lh.lh_scale_sweep(W, amax, torch.from_numpy(H32).to(DEV), None)
    for dt, bf16 in ((torch.bfloat16, True), (torch.float32, False)):
        Wq, bam = lh.lh_dequantize(code, fp4, amax, dtype=dt)
        ref_w, ref_a = oracle.dequantize(code.cpu().numpy(), fp4.cpu().numpy(), amax.cpu().numpy(), bf16=bf16)
        got = Wq.float().cpu().numpy().astype(np.float64)
        np.testing.assert_array_equal(got, ref_w)
        assert np.array_equal(np.signbit(got), np.signbit(ref_w))
        np.testing.assert_array_equal(bam.cpu().numpy().astype(np.float64), ref_a)
    Wq2, none = lh.lh_dequantize(code, fp4, amax, want_block_amax=False)
    assert none is None and torch.equal(Wq2, lh.lh_dequantize(code, fp4, amax)[0])

def test_sweep_exact_midpoint_ties():
    """Weights placed exactly on E2M1 midpoints of some candidate scale must round like the oracle."""
    r = np.random.default_rng(4)
    cout, cin = 64, 32
    amax = np.float32(0.0875)
    g = oracle.global_scale(amax)
    s = oracle.candidate_scales(g)
    W = r.normal(0, 0.02, (1, cout, cin)).astype(np.float32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for c in range(cout):
        for j in range(0, cin, 3):
            k = r.integers(90, 126)
            v = np.float32(mids[r.integers(7)] * s[k])      # nearest fp32 to the midpoint
            W[0, c, j] = v if r.random() < 0.5 else np.nextafter(v, np.float32(1))
    W[0, 0, 0] = amax
    H = np.broadcast_to(np.eye(16, dtype=np.float32) * 2.0, (1, cin // 16, 16, 16)).copy()
    note("sweep exact midpoint ties")
    code, fp4, loss = lh.lh_scale_sweep(torch.from_numpy(W).to(DEV), torch.from_numpy(np.array([amax])).to(DEV),
                                        torch.from_numpy(H).to(DEV))
    res = oracle.sweep(W.astype(np.float64), np.array([amax]), H)
    assert_sweep_match(code.cpu().numpy(), fp4.cpu().numpy(), loss.cpu().numpy(), res)


@pytest.mark.parametrize("diag", [False, True])
def test_sweep_power_of_two_fractions_of_amax(diag):
    """bf16 weights equal to amax * 2^-j (times 1, 1.5, 1.25, 1.75) put |w|/s_k within a few ulps of
    an E2M1 midpoint for several candidates: the filter must decide those quotients exactly."""
    r = np.random.default_rng(8)
    cout, cin = 200, 64
    w32 = r.normal(0, 0.02, (1, cout, cin)).astype(np.float32)
    amax = np.float32(0.10498046875)                      # a bf16 value (mantissa 215)
    fr = np.array([1.0, 1.5, 1.25, 1.75])
    mask = r.random(w32.shape) < 0.15
    picks = amax * fr[r.integers(0, 4, w32.shape)] * 2.0 ** -r.integers(1, 9, w32.shape)
    w32 = np.where(mask, np.sign(r.standard_normal(w32.shape)) * picks, w32).astype(np.float32)
    w32[0, 0, 0] = amax
    Wb = synth.bf16_bits_from_f32(w32)
    Wf = synth.f32_from_bf16_bits(Wb).astype(np.float64)
    a = oracle.absmax(Wf).astype(np.float32)
    note(f"sweep power-of-two fractions of amax, diag={diag}")
    Wd = torch.from_numpy(Wb).view(torch.bfloat16).to(DEV)
    if diag:
        imp = np.abs(r.standard_normal((1, cin))).astype(np.float32) + 0.1
        code, fp4, loss = lh.lh_scale_sweep_diag(Wd, torch.from_numpy(a).to(DEV), torch.from_numpy(imp).to(DEV))
        res = oracle.sweep_diag(Wf, a, imp)
    else:
        A = r.standard_normal((1, cin // 16, 16, 16)).astype(np.float32)
        H = (np.einsum("gnij,gnkj->gnik", A, A) / 16 + 0.5 * np.eye(16)).astype(np.float32)
        code, fp4, loss = lh.lh_scale_sweep(Wd, torch.from_numpy(a).to(DEV), torch.from_numpy(H).to(DEV))
        res = oracle.sweep(Wf, a, H)
    assert_sweep_match(code.cpu().numpy(), fp4.cpu().numpy(), loss.cpu().numpy(), res)


def _every_code_weights(r, cout, cin):
    """Blocks whose max |w| is 6 s_k (within 3%) for k cycling over all 126 codes, global amax 1:
    the argmin lands on every code, the subnormal ones included."""
    nb = cin // 16
    s = oracle.candidate_scales(oracle.global_scale(np.float32(1.0)))
    W = r.standard_normal((1, cout, nb, 16))
    W /= np.abs(W).max(-1, keepdims=True)
    k = (np.arange(cout * nb) % 126).reshape(cout, nb)
    W *= (6.0 * s[k] * r.uniform(0.97, 1.03, (cout, nb)))[None, :, :, None]
    W = W.reshape(1, cout, cin).astype(np.float32)
    W[0, 0, 0] = 1.0
    return W


@pytest.mark.parametrize("diag", [False, True])
def test_sweep_every_code_wins(diag):
    """Each of the 126 E4M3 codes is the winner of some block (the oracle's choice), so every
    lane and slot of the filter's candidate layout decides a winner at least once."""
    r = np.random.default_rng(31)
    cout, cin = 504, 64
    W = _every_code_weights(r, cout, cin)
    a = oracle.absmax(W.astype(np.float64)).astype(np.float32)
    note(f"sweep every code wins, diag={diag}")
    Wd, ad = torch.from_numpy(W).to(DEV), torch.from_numpy(a).to(DEV)
    if diag:
        imp = (np.abs(r.standard_normal((1, cin))) + 0.1).astype(np.float32)
        code, fp4, loss = lh.lh_scale_sweep_diag(Wd, ad, torch.from_numpy(imp).to(DEV))
        res = oracle.sweep_diag(W.astype(np.float64), a, imp)
    else:
        A = r.standard_normal((1, cin // 16, 16, 16)).astype(np.float32)
        H = (np.einsum("gnij,gnkj->gnik", A, A) / 16 + 0.5 * np.eye(16)).astype(np.float32)
        code, fp4, loss = lh.lh_scale_sweep(Wd, ad, torch.from_numpy(H).to(DEV))
        res = oracle.sweep(W.astype(np.float64), a, H)
    assert set(np.unique(res["code"]).tolist()) == set(range(1, 127))
    assert_sweep_match(code.cpu().numpy(), fp4.cpu().numpy(), loss.cpu().numpy(), res)


def test_sweep_diag_importance_and_weight_ranges():
    """Rows outside the diagonal filter's range and wide importance spreads: tiny weights (the
    row's sum Imp w^2 under 2^-100), huge importance (over 2^100), importance spanning 1e-30..1e30
    inside a block, and importance with exact zeros.  All must give the oracle's argmin."""
    r = np.random.default_rng(33)
    G, cout, cin = 4, 40, 64
    W = r.normal(0, 0.02, (G, cout, cin)).astype(np.float32)
    W[0] *= np.float32(1e-25)
    imp = (np.abs(r.standard_normal((G, cin))) + 0.1).astype(np.float32)
    imp[1] *= np.float32(1e36)
    imp[2] = (10.0 ** r.uniform(-30, 30, cin)).astype(np.float32)
    imp[3, r.random(cin) < 0.25] = 0.0
    a = oracle.absmax(W.astype(np.float64)).astype(np.float32)
    note(f"diag sweep importance and weight ranges G={G} cout={cout} cin={cin}")
    code, fp4, loss = lh.lh_scale_sweep_diag(torch.from_numpy(W).to(DEV), torch.from_numpy(a).to(DEV),
                                             torch.from_numpy(imp).to(DEV))
    res = oracle.sweep_diag(W.astype(np.float64), a, imp)
    assert_sweep_match(code.cpu().numpy(), fp4.cpu().numpy(), loss.cpu().numpy(), res)


def test_sweep_diag_outside_the_window():
    """Blocks the diagonal sweep's 32-code window cannot settle by its bounds: a dominant element
    with almost no importance (the argmin lies far below the window, which starts 12 codes below
    the block's amax code), blocks whose elements all lie within a factor 2 of each other (no
    element is small enough for the bound on the codes above the window), and, for contrast,
    ordinary blocks.  The first two kinds go to the float64 pass; every block must get the
    oracle's argmin, nibbles and loss."""
    r = np.random.default_rng(41)
    G, cout, cin = 3, 48, 64
    W = r.normal(0, 0.02, (G, cout, cin)).astype(np.float32)
    imp = (np.abs(r.standard_normal((G, cin))) + 0.5).astype(np.float32)
    W[0, :, ::16] = np.float32(0.5)                      # element 0 of every block dominates ...
    imp[0, ::16] = np.float32(1e-9)                      # ... and hardly counts
    W[0, 0, 1] = np.float32(8.0)                         # (the group's amax, well above 0.5)
    W[1] = (np.sign(r.standard_normal((cout, cin))) * r.uniform(0.6, 1.0, (cout, cin)) * 0.02).astype(np.float32)
    a = oracle.absmax(W.astype(np.float64)).astype(np.float32)
    res = oracle.sweep_diag(W.astype(np.float64), a, imp)
    # the first kind's argmin is below its window (from 12 codes under the amax code) by construction
    g = oracle.global_scale(a)[0]
    kmax = np.searchsorted(oracle.e4m3_ladder(), 0.5 / (6 * g)) + 2
    assert (res["code"][0, 1:] < kmax - 12).mean() > 0.9
    note(f"diag sweep outside the window G={G} cout={cout} cin={cin}")
    code, fp4, loss = lh.lh_scale_sweep_diag(torch.from_numpy(W).to(DEV), torch.from_numpy(a).to(DEV),
                                             torch.from_numpy(imp).to(DEV))
    assert_sweep_match(code.cpu().numpy(), fp4.cpu().numpy(), loss.cpu().numpy(), res)


@pytest.mark.parametrize("coupled", [False, True])
def test_sweep_full_hessian_and_weight_ranges(coupled):
    """Hessians far from unit scale, where the fp32 filter's intermediate values would overflow or
    sink to the subnormal range (H and P near 1e34 and 1e-34, g^2 |H| above 2^76, entries
    spanning 1e-24..1e24 in one block, tiny weights): every block must still get the oracle's
    argmin, through the filter where its range allows and the float64 pass elsewhere."""
    r = np.random.default_rng(35)
    G, cout, cin = 6, 40, 64
    nb = cin // 16
    W = r.normal(0, 0.02, (G, cout, cin)).astype(np.float32)
    W[3] *= np.float32(1e-20)
    W[4] *= np.float32(1e12)
    A = r.standard_normal((G, nb, 16, 16))
    H = np.einsum("gnij,gnkj->gnik", A, A) / 16 + 0.5 * np.eye(16)
    H[0] *= 1e34
    H[1] *= 1e-34
    d = 10.0 ** r.uniform(-12, 12, (nb, 16))
    H[2] *= d[:, :, None] * d[:, None, :]
    H[5] *= 1e20
    H = H.astype(np.float32)
    P = None
    if coupled:
        B = r.standard_normal((G, nb, 16, 16)) * 0.05
        P = (B * np.sqrt(np.abs(np.einsum("gnii->gni", H.astype(np.float64))))[:, :, :, None]).astype(np.float32)
    a = oracle.absmax(W.astype(np.float64)).astype(np.float32)
    note(f"full sweep Hessian and weight ranges coupled={coupled} G={G} cout={cout} cin={cin}")
    code, fp4, loss = lh.lh_scale_sweep(torch.from_numpy(W).to(DEV), torch.from_numpy(a).to(DEV),
                                        torch.from_numpy(H).to(DEV),
                                        torch.from_numpy(P).to(DEV) if coupled else None)
    res = oracle.sweep(W.astype(np.float64), a, H, P)
    assert_sweep_match(code.cpu().numpy(), fp4.cpu().numpy(), loss.cpu().numpy(), res)


def test_sweep_full_near_singular_and_indefinite_hessians():
    """Hessians of 2 to 20 tokens (singular below 16), slightly and strongly indefinite ones,
    non-symmetric ones and outlier channels, on layer-like weights: the eigenvalue certificate
    takes negative shifts here and the sweep skips low codes by the triangle-inequality bound where
    that certificate allows; every block must still get the oracle's argmin, FP4 codes and loss."""
    r = np.random.default_rng(36)
    G, cout, cin = 8, 96, 128
    nb = cin // 16
    W = r.normal(0, 0.02, (G, cout, cin)).astype(np.float32)
    H = np.empty((G, nb, 16, 16))
    for g in range(G):
        for n in range(nb):
            T = int(r.choice([2, 8, 13, 15, 16, 20]))
            X = r.standard_normal((T, 16))
            if (g + n) % 5 == 1:
                X[:, r.integers(16)] *= 20.0
            h = X.T @ X / T
            if g == 5:
                h -= 2.0 ** -11 * np.abs(h).max() * np.eye(16)      # slightly indefinite
            if g == 6:
                h -= 0.05 * np.abs(h).max() * np.eye(16)            # indefinite beyond any shift
            if g == 7:
                h += 1e-3 * np.abs(h).max() * r.standard_normal((16, 16))   # not symmetric
            H[g, n] = h
    H = H.astype(np.float32)
    a = oracle.absmax(W.astype(np.float64)).astype(np.float32)
    note(f"full sweep near-singular and indefinite Hessians G={G} cout={cout} cin={cin}")
    code, fp4, loss = lh.lh_scale_sweep(torch.from_numpy(W).to(DEV), torch.from_numpy(a).to(DEV),
                                        torch.from_numpy(H).to(DEV), None)
    res = oracle.sweep(W.astype(np.float64), a, H, None)
    # codes and FP4 codes exactly; the loss, an fp32 evaluation of e^T H e, within 1e-5 of the
    # scale its roundings follow, sum_ij |e_i||H_ij||e_j|, which for singular and indefinite H can
    # be far above e^T H e itself (the Q + |C| scale of reading 16 presumes a positive definite H)
    assert_sweep_match(code.cpu().numpy(), fp4.cpu().numpy(), None, res)
    W64 = W.astype(np.float64).reshape(G, cout, nb, 16)
    cs = oracle.candidate_scales(oracle.global_scale(a.astype(np.float64)))          # [G, 126]
    sk = cs[np.arange(G)[:, None], res["code"].reshape(G, -1).astype(np.int64) - 1]        # [G, cout*nb]
    _, _, e = oracle.fake_quant(W64, sk.reshape(G, cout, nb, 1))
    scale = np.einsum("gcni,gnij,gcnj->gcn", np.abs(e), np.abs(H.astype(np.float64)), np.abs(e))
    dl = np.abs(loss.cpu().numpy().astype(np.float64) - res["loss"])
    assert np.all(dl <= 1e-5 * scale + 1e-30), f"max |dL|/scale {np.max(dl / (scale + 1e-300)):.3g}"


def test_sweep_deterministic():
    wl = synth.make("c2", cout=100, cin=64, rows=300)
    note("sweep determinism")
    W, X, _, _ = upload(wl)
    amax = lh.lh_absmax(W)
    H, _ = lh.lh_accumulate(X)
    a = lh.lh_scale_sweep(W, amax, H)
    b = lh.lh_scale_sweep(W, amax, H)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.uint8 else x,
                           y.view(torch.uint8) if y.dtype != torch.uint8 else y)


# ------------------------------------------------------------------------------------ end to end
@pytest.mark.parametrize("name", list(SMALL))
def test_end_to_end(name):
    """absmax -> accumulate -> sweep entirely on the GPU, against the oracle's own float64 path."""
    wl = with_oracle_xq(synth.make(name, **SMALL[name]))
    note(f"end-to-end {name}")
    W, X, Xq, off = upload(wl)
    amax = lh.lh_absmax(W)
    Wo = wl.W_f64()
    a_ref = oracle.absmax(Wo)
    if wl.mode == "diag":
        _, imp = lh.lh_accumulate(X, offsets=off, want_h=False, want_imp=True)
        code, fp4, loss = lh.lh_scale_sweep_diag(W, amax, imp)
        _, imp_ref = oracle.accumulate(wl.X_f64(), wl.offsets, want_h=False, want_imp=True)
        res = oracle.sweep_diag(Wo, a_ref, imp_ref)
    elif wl.mode == "act":
        H, P = lh.lh_accumulate_act_aware(X, Xq, offsets=off)
        code, fp4, loss = lh.lh_scale_sweep(W, amax, H, P)
        H_ref, P_ref = oracle.accumulate_act_aware(wl.X_f64(), wl.Xq_f64(), wl.offsets)
        res = oracle.sweep(Wo, a_ref, H_ref, P_ref)
    else:
        H, _ = lh.lh_accumulate(X, offsets=off)
        code, fp4, loss = lh.lh_scale_sweep(W, amax, H)
        H_ref, _ = oracle.accumulate(wl.X_f64(), wl.offsets)
        res = oracle.sweep(Wo, a_ref, H_ref)
    # each side used its own Hessian; near-ties within 1e-6 are exempt as everywhere
    assert_sweep_match(code.cpu().numpy(), fp4.cpu().numpy(), None, res)
