"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

Each workload (dense 2048x2048, activation-aware up_proj 12288x4096, WMSE down_proj 4096x12288,
512-expert MoE gate_up 1280x2560) runs absmax -> accumulation -> sweep once on the GPU through the
C ABI, exactly as one benchmark step does.  The oracle then checks:

* the per-group absmax of every group, bit for bit;
* H / P / importance of every block column of every group, in float64;
* the full 126-candidate float64 search of every weight block of the dense layers and of every
  block of eight whole experts of the MoE layer (seeded, with the experts of the largest and the
  smallest routed-token counts), against the GPU's own fp32 H / P / importance: codes and FP4
  nibbles identical outside near-ties, losses within 1e-5.  The oracle runs in a pool of up to 16
  processes (one BLAS thread each); the count of near-tie blocks is printed;
* the activation-aware layer's X_q made by lh_activation_fake_quant is the oracle's bit for bit,
  and H, P made with X_q formed inside the accumulation kernel equal the two-input kernel's.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import (assert_h_close, assert_imp_close, assert_p_close, cross_gram, oracle_xq,
                         pool_map)

pytestmark = pytest.mark.gpu

lh = pytest.importorskip("nvfp4_scale_calibration_lh_amd")
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
FULL = ["c2", "c3", "c4", "c5"]
MOE_EXPERTS = 8


def note(msg):
    print(f"[case] {msg}", flush=True)


def to_dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(DEV)


def _xq_rows(task):
    X64, amax, bf16 = task
    return oracle_xq(X64, np.array([0, len(X64)]), bf16, x_amax=[amax])


def full_xq(wl):
    """The oracle's X_q of a single-group activation-aware layer (per-tensor amax max|X|), made in
    row chunks over the process pool."""
    X64 = wl.X_f64()
    amax = float(np.abs(X64).max())
    step = 512
    parts = pool_map(_xq_rows, [(X64[a:a + step], amax, wl.dtype == "bf16") for a in range(0, len(X64), step)])
    return np.concatenate(parts)


@pytest.fixture(scope="module", params=FULL)
def run(request):
    name = request.param
    note(f"full-size {name}: generating inputs")
    wl = synth.make(name)
    if wl.mode == "act":
        wl.Xq = full_xq(wl)
    G, cout, cin = wl.n_groups, wl.cout, wl.cin
    note(f"full-size {name}: W{wl.W.shape} X{wl.X.shape} mode={wl.mode} on the GPU")
    W = to_dev(wl.W, wl.dtype)
    X = to_dev(wl.X, wl.dtype)
    off = torch.from_numpy(wl.offsets).to(DEV) if G > 1 else None
    amax = lh.lh_absmax(W)
    H = P = imp = None
    if wl.mode == "act":
        H, P = lh.lh_accumulate_act_aware(X, to_dev(wl.Xq, wl.dtype), offsets=off)
    elif wl.mode == "diag":
        _, imp = lh.lh_accumulate(X, offsets=off, want_h=False, want_imp=True)
    else:
        H, _ = lh.lh_accumulate(X, offsets=off)
    if wl.mode == "diag":
        code, fp4, loss = lh.lh_scale_sweep_diag(W, amax, imp)
    else:
        code, fp4, loss = lh.lh_scale_sweep(W, amax, H, P)
    torch.cuda.synchronize()
    host = lambda t: None if t is None else t.cpu().numpy()
    out = dict(amax=host(amax), H=host(H), P=host(P), imp=host(imp), code=host(code), fp4=host(fp4),
               loss=host(loss))
    del W, X, H, P, imp, code, fp4, loss
    torch.cuda.empty_cache()
    note(f"full-size {name}: GPU done")
    return name, wl, out


def _sweep_groups(wl):
    """Groups whose every block is checked: all of a dense layer; for the MoE layer a seeded set of
    whole experts holding the largest and the smallest routed-token counts."""
    G = wl.n_groups
    if G == 1:
        return np.array([0])
    T = np.diff(wl.offsets)
    pick = {int(np.argmax(T)), int(np.argmin(T))}
    rng = np.random.default_rng(7)
    for g in rng.permutation(G):
        if len(pick) >= MOE_EXPERTS:
            break
        pick.add(int(g))
    return np.array(sorted(pick))


def test_fullsize_absmax(run):
    name, wl, out = run
    note(f"full-size {name}: absmax of {wl.n_groups} groups")
    ref = np.array([oracle.absmax(wl.W_f64(g)[None])[0] for g in range(wl.n_groups)], dtype=np.float32)
    np.testing.assert_array_equal(out["amax"], ref)


def test_fullsize_accumulation_all_columns(run):
    """Every block column of every group against the float64 accumulation (64 columns at a time)."""
    name, wl, out = run
    nb = wl.n_blocks
    note(f"full-size {name}: accumulation of all {nb} block columns of {wl.n_groups} group(s)")
    for n0 in range(0, nb, 4):
        cols = slice(16 * n0, 16 * min(nb, n0 + 4))
        blk = slice(n0, min(nb, n0 + 4))
        Xn = wl._f64(wl.X[:, cols])
        if wl.mode == "diag":
            _, imp_ref = oracle.accumulate(Xn, wl.offsets, want_h=False, want_imp=True)
            assert_imp_close(out["imp"][:, cols], imp_ref)
        elif wl.mode == "act":
            Xqn = wl._f64(wl.Xq[:, cols])
            H_ref, P_ref = oracle.accumulate_act_aware(Xn, Xqn, wl.offsets)
            R_ref = cross_gram(Xn, Xqn, wl.offsets)
            assert_h_close(out["H"][:, blk], H_ref)
            assert_p_close(out["P"][:, blk], P_ref, H_ref, R_ref)
        else:
            H_ref, _ = oracle.accumulate(Xn, wl.offsets)
            assert_h_close(out["H"][:, blk], H_ref)


def _oracle_rows(task):
    """Pool worker: the oracle's search of every block of rows [r0, r1) of one group; returns the
    codes, packed nibbles, losses, the loss scale Q + |C| and the near-tie flags."""
    mode, r0, w, g, H, P, imp = task
    rows, cin = w.shape
    nb = cin // 16
    wb = w.reshape(-1, 16)
    n = np.tile(np.arange(nb), rows)
    gs = np.full(len(wb), g)
    if mode == "diag":
        res = oracle.sweep_blocks_diag(wb, gs, imp.reshape(nb, 16)[n])
    else:
        res = oracle.sweep_blocks(wb, gs, H, P, hidx=n)
    fp4 = oracle.pack_nibbles(res["nib"]).reshape(rows, nb, 8)
    return (r0, res["code"].reshape(rows, nb), fp4, res["loss"].reshape(rows, nb),
            (res["Q1"] + np.abs(res["C1"])).reshape(rows, nb), oracle.exempt_mask(res).reshape(rows, nb))


def test_fullsize_sweep_every_block(run):
    """The whole layer (the dense workloads) or eight whole experts (MoE) against the oracle's
    search on the GPU's own fp32 H / P / importance."""
    name, wl, out = run
    cout, nb = wl.cout, wl.n_blocks
    groups = _sweep_groups(wl)
    step = max(1, 16384 // nb)
    total = exempt_total = 0
    note(f"full-size {name}: oracle search of every block of group(s) {groups.tolist()} "
         f"({len(groups) * cout * nb} blocks)")
    for g in groups:
        g = int(g)
        Wg = wl.W_f64(g)
        gsc = float(oracle.global_scale(out["amax"][g:g + 1].astype(np.float64))[0])
        H = None if out["H"] is None else out["H"][g].astype(np.float64)
        P = None if out["P"] is None else out["P"][g].astype(np.float64)
        imp = None if out["imp"] is None else out["imp"][g].astype(np.float64)
        mode = "diag" if wl.mode == "diag" else "full"
        tasks = [(mode, r0, Wg[r0:r0 + step], gsc, H, P, imp) for r0 in range(0, cout, step)]
        code = out["code"][g]
        fp4 = out["fp4"][g].reshape(cout, nb, 8)
        loss = out["loss"][g].astype(np.float64)
        for r0, rc, rf, rl, rs, rx in pool_map(_oracle_rows, tasks):
            sl = slice(r0, r0 + len(rc))
            bad = (code[sl] != rc) & ~rx
            assert not bad.any(), (f"group {g}: {bad.sum()} scale codes differ outside near-ties, first at "
                                   f"rows/blocks {(np.argwhere(bad)[:3] + [r0, 0]).tolist()}")
            fbad = (fp4[sl] != rf).any(-1) & ~rx
            assert not fbad.any(), f"group {g}: {fbad.sum()} blocks with FP4 codes differing outside near-ties"
            same = code[sl] == rc
            lbad = same & (np.abs(loss[sl] - rl) > 1e-5 * rs + 1e-30)
            assert not lbad.any(), f"group {g}: {lbad.sum()} losses outside 1e-5"
            total += rc.size
            exempt_total += int(rx.sum())
    note(f"full-size {name}: {total} blocks checked, {exempt_total} near-tie blocks exempt")
    assert total == len(groups) * cout * nb


def test_fullsize_codes_and_nibbles_consistent(run):
    name, wl, out = run
    G, cout, nb = wl.n_groups, wl.cout, wl.n_blocks
    code = out["code"]
    assert code.min() >= 1 and code.max() <= 126, "every block must carry a candidate byte 0x01..0x7E"
    assert np.isfinite(out["loss"]).all()
    groups = range(G) if G == 1 else np.random.default_rng(5).choice(G, size=8, replace=False)
    note(f"full-size {name}: nibbles of every block in {len(list(groups))} group(s)")
    for g in groups:
        s_all = oracle.candidate_scales(oracle.global_scale(out["amax"][g:g + 1].astype(np.float64)))[0]
        fp4 = out["fp4"][g].reshape(cout, nb, 8)
        step = max(1, (1 << 20) // (nb * 16))
        for r0 in range(0, cout, step):
            r1 = min(cout, r0 + step)
            w = wl._f64(wl.W[int(g), r0:r1]).reshape(r1 - r0, nb, 16)
            s = s_all[code[g, r0:r1].astype(np.int64) - 1]
            nib, _, _ = oracle.fake_quant(w, s[..., None])
            ref = oracle.pack_nibbles(nib)
            bad = (fp4[r0:r1] != ref).any(-1)
            assert not bad.any(), f"group {g}: {bad.sum()} blocks whose FP4 bytes are not the encoding at their scale"


def test_fullsize_dequantize(run):
    """Fake-quantized bf16 weights and block amax of every block (8 sampled experts for the MoE
    layer) from the full-size sweep's codes, bit for bit against the oracle's decoding."""
    name, wl, out = run
    G = wl.n_groups
    groups = np.arange(G) if G == 1 else np.sort(np.random.default_rng(6).choice(G, size=8, replace=False))
    note(f"full-size {name}: dequantize {len(groups)} group(s)")
    code = np.ascontiguousarray(out["code"][groups])
    fp4 = np.ascontiguousarray(out["fp4"][groups])
    amax = np.ascontiguousarray(out["amax"][groups])
    Wq, bam = lh.lh_dequantize(torch.from_numpy(code).to(DEV), torch.from_numpy(fp4).to(DEV),
                               torch.from_numpy(amax).to(DEV), dtype=torch.bfloat16)
    got_w = Wq.view(torch.int16).cpu().numpy()
    got_a = bam.cpu().numpy()
    del Wq, bam
    torch.cuda.empty_cache()
    step = max(1, (1 << 22) // wl.cin)
    for k in range(len(groups)):
        for r0 in range(0, wl.cout, step):
            r1 = min(wl.cout, r0 + step)
            ref_w, ref_a = oracle.dequantize(code[k:k + 1, r0:r1], fp4[k:k + 1, r0:r1], amax[k:k + 1], bf16=True)
            ref_bits = synth.bf16_bits_from_f32(ref_w.astype(np.float32)).view(np.int16)
            np.testing.assert_array_equal(got_w[k, r0:r1], ref_bits[0])
            np.testing.assert_array_equal(got_a[k, r0:r1].astype(np.float64), ref_a[0])


def test_fullsize_activation_fake_quant_and_fused_accumulation():
    """Activation-aware up_proj 12288x4096 (X [8192,4096] bf16 Student-t(4)): the library's X_q
    (lh_activation_fake_quant) is the oracle's bit for bit; H and P made with X_q formed inside the
    accumulation kernel are within tolerance of the oracle's on every block column and equal,
    value for value, those of the two-input kernel fed the oracle's X_q."""
    wl = synth.make("c3")
    note("full-size c3: oracle X_q")
    Xq_ref = full_xq(wl)
    note("full-size c3: X_q and fused fake-quant accumulation on the GPU")
    X = to_dev(wl.X, "bf16")
    amax = torch.tensor([float(np.abs(wl.X_f64()).max())], dtype=torch.float32, device=DEV)
    Xq_gpu = lh.lh_activation_fake_quant(X, amax)
    H1, P1 = lh.lh_accumulate_act_aware(X, to_dev(Xq_ref, "bf16"))
    H2, P2 = lh.lh_accumulate_act_aware_fq(X, amax)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(Xq_gpu.view(torch.int16).cpu().numpy(), Xq_ref.view(np.int16))
    assert torch.equal(H1, H2) and torch.equal(P1, P2)
    H2, P2 = H2.cpu().numpy(), P2.cpu().numpy()
    note("full-size c3: fused H and P against the oracle on every block column")
    for n0 in range(0, wl.n_blocks, 4):
        cols = slice(16 * n0, 16 * (n0 + 4))
        Xn = wl._f64(wl.X[:, cols])
        Xqn = wl._f64(Xq_ref[:, cols])
        H_ref, P_ref = oracle.accumulate_act_aware(Xn, Xqn, wl.offsets)
        assert_h_close(H2[:, n0:n0 + 4], H_ref)
        assert_p_close(P2[:, n0:n0 + 4], P_ref, H_ref, cross_gram(Xn, Xqn, wl.offsets))


def test_fullsize_fused_moe_equals_two_calls(run):
    """The whole 512-expert layer through lh_accumulate_sweep (Hessians kept on chip): every code,
    nibble and loss bit-identical to the two-call path the other tests checked against the oracle."""
    name, wl, out = run
    if wl.n_groups == 1:
        pytest.skip("the fused path is for grouped rows")
    note(f"full-size {name}: fused accumulate-and-sweep of all {wl.n_groups} experts")
    W = to_dev(wl.W, wl.dtype)
    X = to_dev(wl.X, wl.dtype)
    off = torch.from_numpy(wl.offsets).to(DEV)
    code, fp4, loss = lh.lh_accumulate_sweep(X, W, torch.from_numpy(out["amax"]).to(DEV), off)
    torch.cuda.synchronize()
    got = (code.cpu().numpy(), fp4.cpu().numpy(), loss.cpu().numpy())
    del W, X, code, fp4, loss
    torch.cuda.empty_cache()
    np.testing.assert_array_equal(got[0], out["code"])
    np.testing.assert_array_equal(got[1], out["fp4"])
    np.testing.assert_array_equal(got[2].view(np.int32), out["loss"].view(np.int32))


def test_fullsize_grouped_equals_per_expert(run):
    """Grouped rows against one call per expert (the expert's rows alone, as a dense layer) on eight
    whole experts of the 512-expert layer, with the largest and the smallest routed-token counts:
    the sweep of one expert's weights and Hessian is bit-identical to that expert's part of the
    grouped sweep; the expert's own accumulation and the grouped one are both within tolerance of
    the float64 sums of exactly its rows (the summation orders differ, so not bit for bit); and the
    tolerance is not vacuous: the same check against the rows of the next expert fails."""
    name, wl, out = run
    if wl.n_groups == 1:
        pytest.skip("grouped rows only")
    groups = _sweep_groups(wl)
    off = wl.offsets
    note(f"full-size {name}: per-expert calls for experts {groups.tolist()}")
    for g in groups:
        g = int(g)
        a, b = int(off[g]), int(off[g + 1])
        Wg = to_dev(wl.W[g], wl.dtype)
        am = torch.from_numpy(out["amax"][g:g + 1]).to(DEV)
        Hg = torch.from_numpy(np.ascontiguousarray(out["H"][g:g + 1])).to(DEV)
        code, fp4, loss = lh.lh_scale_sweep(Wg, am, Hg)
        Hd = lh.lh_accumulate(to_dev(wl.X[a:b], wl.dtype))[0] if b > a else None
        torch.cuda.synchronize()
        np.testing.assert_array_equal(code.cpu().numpy()[0], out["code"][g])
        np.testing.assert_array_equal(fp4.cpu().numpy()[0], out["fp4"][g])
        np.testing.assert_array_equal(loss.cpu().numpy()[0].view(np.int32), out["loss"][g].view(np.int32))
        H_ref, _ = oracle.accumulate(wl._f64(wl.X[a:b]), np.array([0, b - a]))
        assert_h_close(out["H"][g:g + 1], H_ref)
        if Hd is None:
            assert not out["H"][g].any(), f"expert {g} has no rows and must have H = 0"
            continue
        assert_h_close(Hd.cpu().numpy(), H_ref)
        nxt = int(np.nonzero(np.diff(off)[g + 1:])[0][0]) + g + 1 if np.diff(off)[g + 1:].any() else None
        if nxt is not None:
            c, d = int(off[nxt]), int(off[nxt + 1])
            H_other, _ = oracle.accumulate(wl._f64(wl.X[c:d]), np.array([0, d - c]))
            with pytest.raises(AssertionError):
                assert_h_close(out["H"][g:g + 1], H_other)
        del Wg, Hg, Hd, code, fp4, loss
    torch.cuda.empty_cache()


def test_fullsize_non_vacuity(run):
    """The local-Hessian (or importance-weighted) codes differ from the plain weight-MSE search's on
    a clearly non-zero share of the blocks of the whole layer: the objective decides."""
    name, wl, out = run
    note(f"full-size {name}: plain MSE search of the whole layer")
    W = to_dev(wl.W, wl.dtype)
    code, _, _ = lh.lh_scale_sweep_mse(W, torch.from_numpy(out["amax"]).to(DEV), want_fp4=False, want_loss=False)
    torch.cuda.synchronize()
    frac = float(np.mean(code.cpu().numpy() != out["code"]))
    del W, code
    torch.cuda.empty_cache()
    note(f"full-size {name}: {frac:.3f} of the blocks take a different scale than under plain MSE")
    assert frac > 0.05, frac


def test_fullsize_full_sweep_on_diagonal_hessian(run):
    """The full-Hessian sweep given H_n = diag(importance of block n) chooses, block for block, what
    the diagonal sweep chose on the whole WMSE layer: identical codes and FP4 nibbles outside
    near-ties (each differing block is confirmed a near-tie by the oracle), losses within 1e-5."""
    name, wl, out = run
    if wl.mode != "diag":
        pytest.skip("the diagonal (importance) workload")
    imp = out["imp"]
    G, nb = imp.shape[0], wl.n_blocks
    Hd = np.zeros((G, nb, 16, 16), dtype=np.float32)
    idx = np.arange(16)
    Hd[:, :, idx, idx] = imp.reshape(G, nb, 16)
    note(f"full-size {name}: full sweep on H = diag(importance)")
    W = to_dev(wl.W, wl.dtype)
    code, fp4, loss = lh.lh_scale_sweep(W, torch.from_numpy(out["amax"]).to(DEV), torch.from_numpy(Hd).to(DEV))
    torch.cuda.synchronize()
    code, fp4, loss = code.cpu().numpy(), fp4.cpu().numpy(), loss.cpu().numpy()
    del W
    torch.cuda.empty_cache()
    cout = wl.cout
    diff = (code != out["code"]) | (fp4.reshape(G, cout, nb, 8) != out["fp4"].reshape(G, cout, nb, 8)).any(-1)
    note(f"full-size {name}: {int(diff.sum())} of {diff.size} blocks differ; checking them with the oracle")
    if diff.any():
        g_, r_, n_ = np.nonzero(diff)
        w = np.stack([wl._f64(wl.W[g, r, 16 * n:16 * n + 16]) for g, r, n in zip(g_, r_, n_)])
        gs = oracle.global_scale(out["amax"][g_].astype(np.float64))
        res = oracle.sweep_blocks_diag(w, gs, imp[g_].reshape(len(g_), nb, 16)[np.arange(len(g_)), n_].astype(np.float64))
        assert oracle.exempt_mask(res).all(), f"{int((~oracle.exempt_mask(res)).sum())} differing blocks are not near-ties"
    same = ~diff
    scale = np.abs(out["loss"].astype(np.float64))
    lbad = same & (np.abs(loss.astype(np.float64) - out["loss"]) > 1e-5 * scale + 1e-30)
    assert not lbad.any(), f"{int(lbad.sum())} losses differ by more than 1e-5"
