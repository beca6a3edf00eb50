"""Float64 CPU oracle of the local-Hessian NVFP4 weight-scale calibration (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may use
this module.  It shares no code with the HIP library and imports nothing from it.

What it computes, in the order and notation of the pages:

* ``accumulate``: per group g (an MoE expert, or the whole layer) and per 16-wide input-channel
  block n, ``H_g[n] = (1/T_g) sum_t x_t[n] x_t[n]^T`` and ``Imp_g[i] = sum_t X[t,i]^2``.
  Pages: "add local hessian calibration" (PR #788), Overview / Changes ("compute per-block
  Hessians"); "Add WMSE weight scale search calibration" (PR #2283), What / How (Imp_i = ||X[:,i]||^2,
  accumulated as x.square().sum(-1) into an [n_blocks, block_size] buffer).
* ``accumulate_act_aware``: ``H = X_q^T X_q / B`` and ``P = X_q^T (X_q - X) / B`` per block.
  Page: "Add activation-aware local Hessian scale calibration" (PR #1976), What does this PR do?
* ``activation_fake_quant``: the X_q those use when the layer's NVFP4 input quantizer is applied
  to X (per-token 16-channel E4M3 block scales under the 448-normalized global scale).
* ``dequantize``: the fake-quantized weights and per-block amax that the chosen codes define.
* ``sweep``: for every 16-element weight block try each of the 126 positive finite E4M3 block
  scales, fake-quantize to E2M1, score ``dw^T H_n dw + 2 dw^T (P_n w0)`` with ``dw = quant(w) - w``
  and keep the argmin, starting from best = +inf.  Pages: PR #1976 review assessment (sign of dw,
  the 2 dw^T(P W0) coupling term, the nbd,cnd->cnb einsum for P.W0, best_loss=inf / argmin with
  negative losses); PR #788 review (the cnb,nbd,cnd->cn block loss); PR #2283 How ("126
  candidate scales"); "Add composable scale calibration to GPTQ" (PR #2004), What does this PR
  do? (NVFP4 scaling is 448-normalized).
* ``sweep_diag``: same search scored by ``sum_i Imp_i dw_i^2`` (PR #2283 How: cnb,nb->cn, the
  DIAGONAL specialization that never materializes diag_embed(Imp)).

Readings where the pages are silent (each is listed in the design doc):

* NVFP4 element grid {0, 0.5, 1, 1.5, 2, 3, 4, 6} (E2M1), round to nearest with ties to the even
  grid index, saturating at 6; the quotient |w|/s is rounded as an exact real number.
* Candidate block scales s_k = fp32(v_k * g) for the E4M3 values v_k of bytes 0x01..0x7E, with the
  per-matrix global scale g = fp32(amax / (6 * 448)); amax = max |W_g|.
* Sign nibble bit = (w < 0); nibble = sign << 3 | grid index; low nibble = even element.
* A block whose Hessian has zero trace (no activation energy, e.g. an expert no token reached)
  is scored with H = I and no cross term -- the plain weight-MSE search that "[2/3] Speed up
  layerwise GPTQ on MoE models" (embedded #2840 text) gives an expert no token reaches.  The
  diagonal form uses Imp = 1 when the block's importance sums to zero.
* Ties between equal losses go to the lowest code (ascending scan with strict <).

Exactness notes.  w is bf16 or fp32 and s is fp32, so |w| and m*s (m a grid midpoint, at most 3
significant bits) are dyadic numbers with at most 27 significant bits; if they differ, they differ
by more than 2^-29 of their size, far above float64's 2^-53 division error.  Hence the float64
quotient r = |w|/s lies on the same side of every midpoint as the exact quotient and equals a
midpoint only when the exact quotient does.  The distances r - lo and hi - r between r and its two
neighbouring grid values are exact (Sterbenz), so the nearest/tie decision is exact.  The error
e = quant(w) - w is exact in float64 (the operands span fewer than 53 bits).

Pins (tests/test_oracle_pins.py): the E4M3 ladder against torch's float8_e4m3fn decoder; the
E2M1 rounding against exact rational arithmetic on every midpoint and its float neighbours;
the expanded output-MSE identity by brute force; diagonal-H equivalence; H = I against a scalar
weight-MSE search; scale/permutation invariances; grouped == per-group; optimality re-check;
H and Imp against quadratic-form and Frobenius identities; golden cases in tests/golden/.
"""
from __future__ import annotations

import numpy as np

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E4M3_MAX = 448.0
FP4_MAX = 6.0
BLOCK = 16
N_CANDIDATES = 126


# ----------------------------------------------------------------------------- scales
def e4m3_ladder() -> np.ndarray:
    """Values of the E4M3 bytes 0x01..0x7E (the 126 positive finite block scales), ascending.

    E4M3: 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is subnormal
    (m * 2^-9); 0x7F is NaN in the finite-only variant, so 0x7E = 448 is the largest value."""
    codes = np.arange(1, 127)
    e = codes >> 3
    m = codes & 7
    return np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))


def global_scale(amax, norm: float = E4M3_MAX) -> np.ndarray:
    """fp32(amax / (6 * norm)): the per-matrix scale that maps the global amax to the E4M3 value
    norm -- 448 for NVFP4 ("Add composable scale calibration to GPTQ", What does this PR do?:
    448-normalized scaling), 256 for its "4/6" variant (same passage).  norm is an E4M3 value, so
    6 * norm is an fp32 number and one float64 divide rounded once to fp32 is the correctly rounded
    fp32 quotient (double rounding is harmless for a single binary32 division)."""
    return np.asarray(np.asarray(amax, dtype=np.float64) / (FP4_MAX * float(norm)), dtype=np.float32).astype(np.float64)


def candidate_scales(g) -> np.ndarray:
    """s_k = fp32(v_k * g) for the 126 ladder values; shape g.shape + (126,).  v_k * g is exact
    in float64 (4 + 24 significant bits), so the cast is the single fp32 rounding."""
    g = np.asarray(g, dtype=np.float64)
    return (g[..., None] * e4m3_ladder()).astype(np.float32).astype(np.float64)


def absmax(W) -> np.ndarray:
    """Per-group max |W_g| (max calibration of the weight, the step that runs first)."""
    W = np.asarray(W, dtype=np.float64)
    return np.abs(W.reshape(W.shape[0], -1)).max(axis=1) if W.size else np.zeros(W.shape[0])


def multiplier_codes(block_amax, g, multipliers) -> np.ndarray:
    """Candidate codes of the amax-multiplier search ("add local hessian calibration", Changes: the
    local-Hessian calibration config has a configurable step size and multipliers for its amax
    search, next to the FP8 scale sweep).  A block with amax a and multiplier m proposes the block
    amax a*m, i.e. the block scale (a*m)/6 under the global scale g: its code is the positive
    finite E4M3 value (bytes 1..126) nearest to the exact real y = a*m / (6 g), ties to the even
    code, saturating at 448 above and at 2^-9 below.

    block_amax [B], g [B], multipliers [M] -> codes [B, M] (int).  a*m is exact in float64 (at most
    48 significant bits) and so is v*6g for every ladder value v (at most 30 bits); two ladder values
    nearest to y lie within a factor 2 of a*m, where the float64 difference |a*m - v*6g| is exact
    (Sterbenz), so the nearest value and every tie are decided exactly."""
    a = np.asarray(block_amax, dtype=np.float64)[:, None, None]
    gg = np.asarray(g, dtype=np.float64)[:, None, None]
    m = np.asarray(multipliers, dtype=np.float64)[None, :, None]
    ladder = e4m3_ladder()[None, None, :]
    d = np.abs(a * m - ladder * (6.0 * gg))                    # [B, M, 126], exact where it matters
    is_min = d == d.min(axis=-1, keepdims=True)
    codes = np.arange(1, 127)
    even_min = is_min & (codes % 2 == 0)
    idx = np.where(even_min.any(axis=-1), np.argmax(even_min, axis=-1), np.argmax(is_min, axis=-1))
    return idx + 1


def multiplier_allowed(block_amax, g, multipliers) -> np.ndarray:
    """[B, 126] mask of the codes the multiplier grid proposes for each block."""
    codes = multiplier_codes(block_amax, g, multipliers)
    allowed = np.zeros((codes.shape[0], N_CANDIDATES), dtype=bool)
    np.put_along_axis(allowed, codes - 1, True, axis=1)
    return allowed


# ----------------------------------------------------------------------------- fake quant
def e2m1_index(r) -> np.ndarray:
    """Grid index (0..7) of the E2M1 value nearest to r >= 0, ties to the even index.

    Values above 6 are nearest to 6, which gives the saturation."""
    r = np.asarray(r, dtype=np.float64)
    d = np.abs(r[..., None] - E2M1_GRID)
    best = d.min(axis=-1, keepdims=True)
    is_min = d == best
    idx = np.arange(8)
    # among the (at most two, adjacent) nearest grid points prefer the even index
    even_min = is_min & (idx % 2 == 0)
    has_even = even_min.any(axis=-1)
    first_even = np.argmax(even_min, axis=-1)
    first_any = np.argmax(is_min, axis=-1)
    return np.where(has_even, first_even, first_any)


def fake_quant(w, s):
    """Fake-quantize weights w with block scale s (broadcasting).

    Returns (nibble uint8, wq float64, e float64) with e = wq - w.  s == 0 quantizes everything
    to 0."""
    w = np.asarray(w, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    s_b = np.broadcast_to(s, np.broadcast_shapes(w.shape, s.shape))
    safe = np.where(s_b > 0, s_b, 1.0)
    c = e2m1_index(np.abs(w) / safe)
    c = np.where(s_b > 0, c, 0)
    neg = w < 0
    mag = E2M1_GRID[c] * s_b
    wq = np.where(neg, -mag, mag)
    nib = (c | (neg.astype(np.int64) << 3)).astype(np.uint8)
    return nib, wq, wq - w


def pack_nibbles(nib) -> np.ndarray:
    """[..., 2k] nibbles -> [..., k] bytes, low nibble = even element."""
    nib = np.asarray(nib, dtype=np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


# ----------------------------------------------------------------------------- accumulation
def _group_rows(offsets, g):
    return int(offsets[g]), int(offsets[g + 1])


def accumulate(X, offsets, beta: float = 0.0, H_prev=None, imp_prev=None, want_h=True, want_imp=False):
    """H_g[n] = beta*H_prev + (1/T_g) X_g[:,n]^T X_g[:,n];  imp_g = beta*imp_prev + sum_t X_g[t]^2.

    X: [rows, cin] (float64-convertible), offsets: int [G+1].  T_g = 0 leaves the sum term 0."""
    X = np.asarray(X, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    G = len(offsets) - 1
    cin = X.shape[1]
    nb = cin // BLOCK
    H = np.zeros((G, nb, BLOCK, BLOCK)) if want_h else None
    imp = np.zeros((G, cin)) if want_imp else None
    for g in range(G):
        r0, r1 = _group_rows(offsets, g)
        T = r1 - r0
        Xg = X[r0:r1]
        if want_h and T > 0:
            Xb = Xg.reshape(T, nb, BLOCK).transpose(1, 2, 0)        # [nb, 16, T]
            H[g] = np.matmul(Xb, Xb.transpose(0, 2, 1)) / T
        if want_imp and T > 0:
            imp[g] = np.sum(Xg * Xg, axis=0)
    if want_h and beta != 0.0:
        H = beta * np.asarray(H_prev, dtype=np.float64) + H
    if want_imp and beta != 0.0:
        imp = beta * np.asarray(imp_prev, dtype=np.float64) + imp
    return H, imp


def accumulate_act_aware(X, Xq, offsets, beta: float = 0.0, H_prev=None, P_prev=None):
    """H_g[n] = X_q^T X_q / T_g and P_g[n] = X_q^T (X_q - X) / T_g per 16-channel block."""
    X = np.asarray(X, dtype=np.float64)
    Xq = np.asarray(Xq, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    G = len(offsets) - 1
    nb = X.shape[1] // BLOCK
    H = np.zeros((G, nb, BLOCK, BLOCK))
    P = np.zeros((G, nb, BLOCK, BLOCK))
    for g in range(G):
        r0, r1 = _group_rows(offsets, g)
        T = r1 - r0
        if T == 0:
            continue
        Q = Xq[r0:r1].reshape(T, nb, BLOCK).transpose(1, 2, 0)          # [nb, 16, T]
        D = (Xq[r0:r1] - X[r0:r1]).reshape(T, nb, BLOCK).transpose(1, 0, 2)  # [nb, T, 16]
        H[g] = np.matmul(Q, Q.transpose(0, 2, 1)) / T
        P[g] = np.matmul(Q, D) / T
    if beta != 0.0:
        H = beta * np.asarray(H_prev, dtype=np.float64) + H
        P = beta * np.asarray(P_prev, dtype=np.float64) + P
    return H, P


def e4m3_nearest(y) -> np.ndarray:
    """The E4M3 value (0 or one of the 126 positive finite values) nearest to y >= 0, ties to the
    even code; values above 448 are nearest to 448 (saturation).  Brute force over all 127.

    y is a float64 quotient of a bf16/fp32 amax by 6 gX (at most 26 significant bits): it lies on
    the exact quotient's side of every E4M3 midpoint (at most 5 bits) and equals one only when the
    exact quotient does, and its distances to the two nearest values are exact (Sterbenz)."""
    y = np.asarray(y, dtype=np.float64)
    values = np.concatenate([[0.0], e4m3_ladder()])                 # index = E4M3 code 0..126
    d = np.abs(y[..., None] - values)
    is_min = d == d.min(axis=-1, keepdims=True)
    even_min = is_min & (np.arange(127) % 2 == 0)
    code = np.where(even_min.any(axis=-1), np.argmax(even_min, axis=-1), np.argmax(is_min, axis=-1))
    return values[code]


def _bf16_round(x32) -> np.ndarray:
    """Nearest-even bf16 of float32 values, returned as float64 (torch's conversion)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)


def activation_fake_quant(X, x_amax, offsets, bf16: bool, rows_per_chunk: int = 256) -> np.ndarray:
    """X_q: the NVFP4 fake-quant the layer's input quantizer applies to its activations, which the
    activation-aware Hessian is built from ("Add activation-aware local Hessian scale
    calibration", What does this PR do?), with the 448-normalized NVFP4 scaling ("Add composable
    scale calibration to GPTQ", What does this PR do?) applied per token.

    Group g has the global scale gX = fp32(x_amax[g] / (6*448)).  Each row's 16-channel block gets
    the block scale v = the E4M3 value nearest to max|x| / (6 gX) (ties to the even code, so 448 at
    most and 0 for a block whose max rounds to 0), s = fp32(v gX); each element becomes
    sign(x) * E2M1(|x|/s) * s, the product rounded to fp32 and then, for bf16 activations, to bf16.
    sign(x) is the sign bit of x, as in an IEEE product: an element that quantizes to 0 keeps it
    (-0 for a negative or -0 input).  x_amax = 0 gives X_q = sign(x) * 0."""
    X = np.asarray(X, dtype=np.float64)
    x_amax = np.asarray(x_amax, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    rows, cin = X.shape
    nb = cin // BLOCK
    out = np.zeros_like(X)
    for g in range(len(offsets) - 1):
        gx = float(global_scale(x_amax[g]))
        r0, r1 = _group_rows(offsets, g)
        if gx == 0.0:
            out[r0:r1] = np.copysign(0.0, X[r0:r1])
            continue
        for a in range(r0, r1, rows_per_chunk):
            b = min(r1, a + rows_per_chunk)
            xb = X[a:b].reshape(b - a, nb, BLOCK)
            v = e4m3_nearest(np.abs(xb).max(axis=-1) / (6.0 * gx))
            s = (v * gx).astype(np.float32).astype(np.float64)       # v gX is exact in float64
            _, wq, _ = fake_quant(xb, s[..., None])                  # E2M1(|x|/s) s, exact
            q32 = np.copysign(np.abs(wq), xb).astype(np.float32)     # sign bit of x; the product in fp32
            out[a:b] = (_bf16_round(q32) if bf16 else q32.astype(np.float64)).reshape(b - a, cin)
    return out


def dequantize(code, fp4, amax, bf16: bool, norm: float = E4M3_MAX):
    """Fake-quantized weights and per-block amax from scale codes [G, cout, nb] (bytes 1..126)
    and packed nibbles [G, cout, cin/2] -- the calibrated quantizer state whose amax, scales and
    final fake-quantized weights "Add WMSE weight scale search calibration" fingerprints.

    s = fp32(v_code * g) with g = fp32(amax / (6*448)); Wq = sign * E2M1 value * s rounded to fp32
    (then to bf16 for bf16 weights), a set sign bit giving -0 for a zero value; block amax =
    fp32(6 s).  Returns (Wq float64 values [G, cout, cin], block_amax float64 [G, cout, nb])."""
    code = np.asarray(code, dtype=np.int64)
    fp4 = np.asarray(fp4, dtype=np.uint8)
    G, cout, nb = code.shape
    g = global_scale(np.asarray(amax, dtype=np.float64), norm)
    v = e4m3_ladder()[code - 1]
    s = (v * g[:, None, None]).astype(np.float32).astype(np.float64)
    nib = np.empty((G, cout, nb * BLOCK), dtype=np.uint8)
    nib[..., 0::2] = fp4 & 15
    nib[..., 1::2] = fp4 >> 4
    mag = E2M1_GRID[nib & 7] * np.repeat(s, BLOCK, axis=-1)
    wq = np.where(nib >= 8, -mag, mag).astype(np.float32)
    Wq = _bf16_round(wq) if bf16 else wq.astype(np.float64)
    return Wq, (6.0 * s).astype(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------- sweep
def _select(L, Q, C):
    """Argmin over the candidate axis with the first minimum winning; also the runner-up."""
    k1 = np.argmin(L, axis=-1)                              # first occurrence = lowest code
    rows = np.arange(L.shape[0])
    L1 = L[rows, k1]
    L_other = L.copy()
    L_other[rows, k1] = np.inf
    k2 = np.argmin(L_other, axis=-1)
    return k1, dict(L1=L1, Q1=Q[rows, k1], C1=C[rows, k1],
                    L2=L[rows, k2], Q2=Q[rows, k2], C2=C[rows, k2], k2=k2)


def _candidate_losses(wb, s, Hb, Pb):
    """L, Q, C for every (block, candidate): Q = e^T H e, C = 2 e^T (P w0), L = Q + C."""
    _, _, E = fake_quant(wb[:, None, :], s[:, :, None])     # [b, 126, 16]
    Q = np.einsum("bki,bij,bkj->bk", E, Hb, E)
    if Pb is None:
        C = np.zeros_like(Q)
    else:
        bias = np.einsum("bij,bj->bi", Pb, wb)               # P_n w0 (nbd,cnd->cnb)
        C = 2.0 * np.einsum("bki,bi->bk", E, bias)
    return Q + C, Q, C


def candidate_losses(w, g, H, P=None):
    """Loss of all 126 candidates for blocks w [B,16] (zero-trace rule applied): (L, Q, C)."""
    w = np.asarray(w, dtype=np.float64)
    H = np.array(H, dtype=np.float64)
    P = None if P is None else np.array(P, dtype=np.float64)
    dead = np.trace(H, axis1=1, axis2=2) == 0.0
    H[dead] = np.eye(BLOCK)
    if P is not None:
        P[dead] = 0.0
    return _candidate_losses(w, candidate_scales(np.asarray(g, dtype=np.float64)), H, P)


def sweep_blocks(w, g, H, P=None, hidx=None, chunk: int = 2048, allowed=None):
    """Core search on a list of blocks.

    w: [B,16] weights, g: [B] global scale of each block's matrix, H: [M,16,16] Hessians and
    P: [M,16,16] or None, with block b using H[hidx[b]] (hidx defaults to 0..B-1).  allowed: None
    (all 126 candidates) or a [B,126] mask of the candidates block b may take (the multiplier
    search); the others score +inf.  Returns a dict with code (uint8 E4M3 byte), nib [B,16], loss,
    and the runner-up data."""
    w = np.asarray(w, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    H = np.asarray(H, dtype=np.float64)
    P = None if P is None else np.asarray(P, dtype=np.float64)
    B = w.shape[0]
    hidx = np.arange(B) if hidx is None else np.asarray(hidx, dtype=np.int64)
    out = {k: np.zeros(B) for k in ("loss", "L1", "Q1", "C1", "L2", "Q2", "C2")}
    out["code"] = np.zeros(B, dtype=np.uint8)
    out["k2"] = np.zeros(B, dtype=np.int64)
    out["nib"] = np.zeros((B, BLOCK), dtype=np.uint8)
    eye = np.eye(BLOCK)
    for b0 in range(0, B, chunk):
        sl = slice(b0, min(B, b0 + chunk))
        wb, Hb = w[sl], H[hidx[sl]]
        Pb = None if P is None else P[hidx[sl]]
        dead = np.trace(Hb, axis1=1, axis2=2) == 0.0            # no activation energy
        Hb[dead] = eye
        if Pb is not None:
            Pb[dead] = 0.0
        s = candidate_scales(g[sl])                              # [b, 126]
        L, Q, C = _candidate_losses(wb, s, Hb, Pb)
        if allowed is not None:
            L = np.where(allowed[sl], L, np.inf)
        k1, info = _select(L, Q, C)
        nib, _, _ = fake_quant(wb, s[np.arange(len(k1)), k1][:, None])
        out["code"][sl] = (k1 + 1).astype(np.uint8)
        out["nib"][sl] = nib
        out["loss"][sl] = info["L1"]
        for k in ("L1", "Q1", "C1", "L2", "Q2", "C2", "k2"):
            out[k][sl] = info[k]
    return out


def sweep_blocks_diag(w, g, imp, chunk: int = 4096, allowed=None):
    """Diagonal search on a list of blocks: imp [B,16] importance of the block's channels;
    allowed as in sweep_blocks."""
    w = np.asarray(w, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    imp = np.asarray(imp, dtype=np.float64)
    B = w.shape[0]
    out = {k: np.zeros(B) for k in ("loss", "L1", "Q1", "C1", "L2", "Q2", "C2")}
    out["code"] = np.zeros(B, dtype=np.uint8)
    out["k2"] = np.zeros(B, dtype=np.int64)
    out["nib"] = np.zeros((B, BLOCK), dtype=np.uint8)
    for b0 in range(0, B, chunk):
        sl = slice(b0, min(B, b0 + chunk))
        wb, ib = w[sl], imp[sl].copy()
        ib[ib.sum(axis=1) == 0.0] = 1.0
        s = candidate_scales(g[sl])
        _, _, E = fake_quant(wb[:, None, :], s[:, :, None])
        L = np.einsum("bki,bi->bk", E * E, ib)
        if allowed is not None:
            L = np.where(allowed[sl], L, np.inf)
        k1, info = _select(L, np.where(np.isfinite(L), L, 0.0), np.zeros_like(L))
        nib, _, _ = fake_quant(wb, s[np.arange(len(k1)), k1][:, None])
        out["code"][sl] = (k1 + 1).astype(np.uint8)
        out["nib"][sl] = nib
        out["loss"][sl] = info["L1"]
        for k in ("L1", "Q1", "C1", "L2", "Q2", "C2", "k2"):
            out[k][sl] = info[k]
    return out


def _flatten_blocks(W):
    W = np.asarray(W, dtype=np.float64)
    G, cout, cin = W.shape
    nb = cin // BLOCK
    return W.reshape(G, cout, nb, BLOCK), G, cout, nb


def _reshape_out(res, G, cout, nb):
    out = {}
    for k, v in res.items():
        if k == "nib":
            out["fp4"] = pack_nibbles(v.reshape(G, cout, nb * BLOCK))
            out["nib"] = v.reshape(G, cout, nb, BLOCK)
        else:
            out[k] = v.reshape(G, cout, nb)
    return out


def _allowed(wl, gl, multipliers):
    """Candidate mask of the multiplier search for blocks wl [B,16] (None: all 126)."""
    if multipliers is None:
        return None
    return multiplier_allowed(np.abs(wl).max(axis=1), gl, multipliers)


def sweep(W, amax, H, P=None, norm: float = E4M3_MAX, multipliers=None):
    """Full-matrix sweep.  W [G,cout,cin], amax [G], H [G,nb,16,16], P same or None; norm the
    E4M3 value the global amax maps to (448, or 256 for "4/6"); multipliers None (the 126-candidate
    FP8 sweep) or the amax multipliers of the multiplier search.

    Returns code [G,cout,nb] (E4M3 byte), fp4 [G,cout,cin/2], loss, L1/L2/Q/C diagnostics."""
    Wb, G, cout, nb = _flatten_blocks(W)
    g = global_scale(amax, norm)
    H = np.asarray(H, dtype=np.float64)
    wl = Wb.reshape(-1, BLOCK)
    gl = np.repeat(g, cout * nb)
    # block (g, c, n) uses H[g, n]
    hidx = (np.arange(G)[:, None, None] * nb + np.arange(nb)[None, None, :]
            + np.zeros((1, cout, 1), dtype=np.int64)).reshape(-1)
    Ht = H.reshape(G * nb, BLOCK, BLOCK)
    Pt = None if P is None else np.asarray(P, dtype=np.float64).reshape(G * nb, BLOCK, BLOCK)
    return _reshape_out(sweep_blocks(wl, gl, Ht, Pt, hidx, allowed=_allowed(wl, gl, multipliers)), G, cout, nb)


def sweep_diag(W, amax, imp, norm: float = E4M3_MAX, multipliers=None):
    """Full-matrix diagonal sweep.  imp [G, cin]; norm and multipliers as in sweep."""
    Wb, G, cout, nb = _flatten_blocks(W)
    g = global_scale(amax, norm)
    imp = np.asarray(imp, dtype=np.float64).reshape(G, 1, nb, BLOCK)
    wl = Wb.reshape(-1, BLOCK)
    gl = np.repeat(g, cout * nb)
    il = np.broadcast_to(imp, (G, cout, nb, BLOCK)).reshape(-1, BLOCK)
    return _reshape_out(sweep_blocks_diag(wl, gl, il, allowed=_allowed(wl, gl, multipliers)), G, cout, nb)


def exempt_mask(res, rel: float = 1e-6) -> np.ndarray:
    """Blocks whose two best losses are closer than rel * max(Q+|C|) of the two (near-ties)."""
    scale = np.maximum(res["Q1"] + np.abs(res["C1"]), res["Q2"] + np.abs(res["C2"]))
    return np.abs(res["L2"] - res["L1"]) <= rel * scale
