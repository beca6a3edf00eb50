"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

Each workload (dense 2048x2048, activation-aware up_proj 12288x4096, WMSE down_proj 4096x12288,
512-expert MoE gate_up 1280x2560) runs absmax -> accumulation -> sweep once on the GPU through the
C ABI, exactly as one benchmark step does.  The oracle then checks, one by one:

* the per-group absmax of every group, bit for bit;
* the Hessian / cross matrix / importance of sampled blocks (every group for the MoE layer);
* the full 126-candidate float64 search of several thousand sampled weight blocks (seeded random
  blocks plus the block holding each sampled group's absmax), against the GPU's own fp32 H / P /
  importance: codes and FP4 nibbles identical outside near-ties, losses within 1e-5;
* over all blocks (all experts' blocks in 8 sampled experts for the MoE layer): every code is a
  valid candidate byte and the FP4 nibbles are the E2M1 encoding of the block at the chosen scale.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import assert_h_close, assert_imp_close, assert_p_close, assert_sweep_match

pytestmark = pytest.mark.gpu

lh = pytest.importorskip("nvfp4_scale_calibration_lh_amd")
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
FULL = ["c2", "c3", "c4", "c5"]
N_SAMPLE = 6144


def note(msg):
    print(f"[case] {msg}", flush=True)


def to_dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(DEV)


@pytest.fixture(scope="module", params=FULL)
def run(request):
    name = request.param
    note(f"full-size {name}: generating inputs")
    wl = synth.make(name)
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


def _sample_groups(wl, k=16):
    G = wl.n_groups
    if G == 1:
        return np.array([0])
    T = np.diff(wl.offsets)
    rng = np.random.default_rng(7)
    pick = set(rng.choice(G, size=min(k, G), replace=False).tolist())
    pick |= {int(np.argmax(T)), int(np.argmin(T)), 0, G - 1}
    return np.array(sorted(pick))


def test_fullsize_absmax(run):
    name, wl, out = run
    note(f"full-size {name}: absmax of {wl.n_groups} groups")
    ref = np.array([oracle.absmax(wl.W_f64(g)[None])[0] for g in range(wl.n_groups)], dtype=np.float32)
    np.testing.assert_array_equal(out["amax"], ref)


def test_fullsize_accumulation_sampled(run):
    name, wl, out = run
    nb = wl.n_blocks
    blocks = sorted({0, nb - 1, *np.random.default_rng(3).choice(nb, size=min(6, nb), replace=False).tolist()})
    note(f"full-size {name}: accumulation of blocks {blocks}")
    for n in blocks:
        cols = slice(16 * n, 16 * n + 16)
        Xn = wl._f64(wl.X[:, cols])
        if wl.mode == "diag":
            _, imp_ref = oracle.accumulate(Xn, wl.offsets, want_h=False, want_imp=True)
            assert_imp_close(out["imp"][:, cols], imp_ref)
        elif wl.mode == "act":
            Xqn = wl._f64(wl.Xq[:, cols])
            H_ref, P_ref = oracle.accumulate_act_aware(Xn, Xqn, wl.offsets)
            R_ref, _ = oracle.accumulate(Xqn - Xn, wl.offsets)
            assert_h_close(out["H"][:, n], H_ref[:, 0])
            assert_p_close(out["P"][:, n], P_ref[:, 0], H_ref[:, 0], R_ref[:, 0])
        else:
            H_ref, _ = oracle.accumulate(Xn, wl.offsets)
            assert_h_close(out["H"][:, n], H_ref[:, 0])


def test_fullsize_sweep_sampled(run):
    name, wl, out = run
    G, cout, nb = wl.n_groups, wl.cout, wl.n_blocks
    rng = np.random.default_rng(11)
    groups = _sample_groups(wl)
    per = max(1, N_SAMPLE // len(groups))
    total_exempt = 0
    note(f"full-size {name}: oracle search of {per * len(groups)}+ sampled blocks in {len(groups)} groups")
    for g in groups:
        Wg = wl.W_f64(int(g)).reshape(cout, nb, 16)
        flat = rng.choice(cout * nb, size=min(per, cout * nb), replace=False)
        am = int(np.argmax(np.abs(Wg).reshape(-1)))          # block holding the group's absmax
        flat = np.unique(np.concatenate([flat, [am // 16, 0, cout * nb - 1]]))
        c, n = flat // nb, flat % nb
        w = Wg[c, n]
        gs = np.repeat(oracle.global_scale(out["amax"][g:g + 1].astype(np.float64))[0], len(flat))
        if wl.mode == "diag":
            res = oracle.sweep_blocks_diag(w, gs, out["imp"][g].reshape(nb, 16)[n].astype(np.float64))
        else:
            P = None if out["P"] is None else out["P"][g].astype(np.float64)
            res = oracle.sweep_blocks(w, gs, out["H"][g].astype(np.float64), P, hidx=n)
        res["fp4"] = oracle.pack_nibbles(res["nib"])
        total_exempt += assert_sweep_match(out["code"][g][c, n], out["fp4"][g].reshape(cout, nb, 8)[c, n],
                                           out["loss"][g][c, n], res)
    note(f"full-size {name}: {total_exempt} near-tie blocks exempt")


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

def test_fullsize_fused_fake_quant_matches_two_input_path():
    """Activation-aware up_proj 12288x4096 (X [8192,4096] bf16): H and P with X_q made in the
    kernel equal, value for value, those of the two-input kernel fed the generator's X_q (the
    same quantizer recipe, pinned against the oracle's), so every X_q element is bit-exact."""
    wl = synth.make("c3")
    note("full-size c3: fused fake-quant accumulation against the two-input path")
    X = to_dev(wl.X, "bf16")
    Xq = to_dev(wl.Xq, "bf16")
    amax = torch.tensor([float(np.abs(wl.X_f64()).max())], dtype=torch.float32, device=DEV)
    H1, P1 = lh.lh_accumulate_act_aware(X, Xq)
    H2, P2 = lh.lh_accumulate_act_aware_fq(X, amax)
    torch.cuda.synchronize()
    assert torch.equal(H1, H2) and torch.equal(P1, P2)
