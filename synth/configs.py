"""Seeded synthetic workloads shaped like the layers the pages calibrate.

The pages calibrate real checkpoints on real calibration text; none of that is available
here, so every tensor is drawn from a fixed-seed generator with the shapes and value
distributions below.  Five workloads are defined:

``c1``  tiny dense: W [64,128] fp32 ~N(0,0.02), X [256,128] fp32 ~N(0,1), full Hessian.
``c2``  dense 2048x2048: W bf16 ~N(0,0.02), X [8192,2048] bf16 ~N(0,1) whose 1% outlier
        channels (at least one) are multiplied by 20 before rounding to bf16; full Hessian.
``c3``  activation-aware up_proj: W [12288,4096] bf16 ~N(0,0.015), X [8192,4096] bf16
        Student-t(4); H and P, sweep with cross term.  Its X_q is not drawn here: it is the
        NVFP4 fake-quant of X by the layer's input quantizer (per-tensor amax max|X|), which the
        tests take from the oracle and the benchmark from the library
        (``lh_activation_fake_quant``); ``Workload.Xq`` stays None until a caller sets it.
``c4``  WMSE down_proj: W [4096,12288] bf16 ~N(0,0.01), X [8192,12288] bf16 ~N(0,1) with
        0.5% outlier channels (at least one) x30; importance vector only, diagonal sweep.
``c5``  fused-MoE gate_up: 512 experts, each W [1280,2560] bf16 ~N(0,0.02); 8192 tokens of
        hidden size 2560 bf16 ~N(0,1); each token routed to 10 distinct experts drawn by
        Gumbel-top-k on Zipf(1.1) logits; the per-expert token slices are concatenated in
        expert order (token order inside an expert) into X [sum T_g, 2560] with row
        offsets [513].

Every draw uses ``numpy.random.Generator(PCG64(SeedSequence([seed, config_id, stream,
*sub])))`` with streams 0 = weights, 1 = activations, 2 = outlier channels, 3 = routing.
Normal draws are float32 (``standard_normal(dtype=float32)``) scaled in float32; Student-t
draws are float64 cast to float32.  bf16 storage is produced by round-to-nearest-even of
the float32 value and kept as raw ``uint16`` bit patterns (numpy has no bf16 dtype).

Any workload can be shrunk (``make("c3", cout=96, rows=200)``) for parity tests: the
recipe and seeds stay the same, only the shapes change.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np

CONFIG_IDS = {"c1": 1, "c2": 2, "c3": 3, "c4": 4, "c5": 5}

# Full-size shapes.  mode: "full" = Hessian sweep, "act" = Hessian + cross term,
# "diag" = importance-weighted (diagonal) sweep.
CONFIGS = {
    "c1": dict(dtype="f32", mode="full", n_groups=1, cout=64, cin=128, rows=256, w_std=0.02),
    "c2": dict(dtype="bf16", mode="full", n_groups=1, cout=2048, cin=2048, rows=8192, w_std=0.02,
               outlier_frac=0.01, outlier_mul=20.0),
    "c3": dict(dtype="bf16", mode="act", n_groups=1, cout=12288, cin=4096, rows=8192, w_std=0.015,
               student_df=4.0),
    "c4": dict(dtype="bf16", mode="diag", n_groups=1, cout=4096, cin=12288, rows=8192, w_std=0.01,
               outlier_frac=0.005, outlier_mul=30.0),
    "c5": dict(dtype="bf16", mode="full", n_groups=512, cout=1280, cin=2560, tokens=8192, topk=10,
               zipf=1.1, w_std=0.02),
}

DESCRIPTIONS = {
    "c1": "tiny dense W[64,128] fp32, X[256,128], full H",
    "c2": "dense 2048x2048 bf16, X[8192,2048] with 1% outlier channels x20, full H",
    "c3": "activation-aware up_proj W[12288,4096] bf16, X[8192,4096] Student-t(4), H+P",
    "c4": "WMSE down_proj W[4096,12288] bf16, X[8192,12288] with 0.5% outliers x30, diagonal",
    "c5": "fused MoE gate_up 512 experts W[1280,2560] bf16, 8192 tokens top-10 Zipf(1.1)",
}


def rng_for(seed: int, config_id: int, stream: int, *sub: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, config_id, stream, *sub])))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bit patterns.

    Inputs are finite (the generators never make NaN/Inf)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _to_storage(a32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_from_f32(a32)
    return np.ascontiguousarray(a32, dtype=np.float32)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    return a


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str              # storage dtype of W, X, X_q: "f32" or "bf16"
    mode: str               # "full", "act" or "diag"
    n_groups: int
    cout: int
    cin: int
    W: np.ndarray           # [n_groups, cout, cin] (uint16 bf16 bits or float32)
    X: np.ndarray           # [rows, cin]
    Xq: Optional[np.ndarray]  # activation-aware input X_q; never made by the generator (see c3)
    offsets: np.ndarray     # int64 [n_groups + 1]; rows of group g are [off[g], off[g+1])
    description: str = ""

    @property
    def rows(self) -> int:
        return int(self.X.shape[0])

    @property
    def n_blocks(self) -> int:
        return self.cin // 16

    @property
    def weight_blocks(self) -> int:
        return self.n_groups * self.cout * self.n_blocks

    def _f64(self, a):
        if a is None:
            return None
        if self.dtype == "bf16":
            return f32_from_bf16_bits(a).astype(np.float64)
        return a.astype(np.float64)

    def W_f64(self, g: Optional[int] = None):
        return self._f64(self.W if g is None else self.W[g])

    def X_f64(self, r0: int = 0, r1: Optional[int] = None):
        return self._f64(self.X[r0:r1])

    def Xq_f64(self, r0: int = 0, r1: Optional[int] = None):
        return None if self.Xq is None else self._f64(self.Xq[r0:r1])

    def sha256(self) -> dict:
        out = {}
        for k in ("W", "X", "Xq", "offsets"):
            a = getattr(self, k)
            if a is not None:
                out[k] = hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
        return out


def _moe_routing(rng: np.random.Generator, n_tokens: int, n_experts: int, topk: int, zipf: float):
    """Expert lists per token: Gumbel-top-k over logits -zipf*ln(rank) of a seeded ranking."""
    rank = rng.permutation(n_experts) + 1                    # rank of expert e, 1-based
    logits = -zipf * np.log(rank.astype(np.float64))
    gumbel = rng.gumbel(size=(n_tokens, n_experts))
    scores = logits[None, :] + gumbel
    top = np.argpartition(-scores, topk - 1, axis=1)[:, :topk]
    return top                                               # [n_tokens, topk] distinct experts


def make(name: str, seed: int = 0, **over) -> Workload:
    """Build workload ``name`` (c1..c5); keyword overrides shrink shapes for tests."""
    cid = CONFIG_IDS[name]
    cfg = dict(CONFIGS[name])
    cfg.update(over)
    dtype, mode = cfg["dtype"], cfg["mode"]
    cout, cin = int(cfg["cout"]), int(cfg["cin"])
    if cin % 16:
        raise ValueError("cin must be a multiple of 16")

    if name == "c5":
        G = int(cfg["n_groups"])
        ntok, topk = int(cfg["tokens"]), int(cfg["topk"])
        hidden = _to_storage(_normal(rng_for(seed, cid, 1), (ntok, cin), 1.0), dtype)
        top = _moe_routing(rng_for(seed, cid, 3), ntok, G, topk, float(cfg["zipf"]))
        tok_of = [[] for _ in range(G)]
        for t in range(ntok):            # token order inside each expert
            for e in top[t]:
                tok_of[int(e)].append(t)
        counts = np.array([len(v) for v in tok_of], dtype=np.int64)
        offsets = np.zeros(G + 1, dtype=np.int64)
        offsets[1:] = np.cumsum(counts)
        idx = np.concatenate([np.asarray(v, dtype=np.int64) for v in tok_of]) if ntok else np.zeros(0, np.int64)
        X = np.ascontiguousarray(hidden[idx])
        W = np.empty((G, cout, cin), dtype=np.uint16 if dtype == "bf16" else np.float32)
        for g in range(G):
            W[g] = _to_storage(_normal(rng_for(seed, cid, 0, g), (cout, cin), cfg["w_std"]), dtype)
        return Workload(name, dtype, mode, G, cout, cin, W, X, None, offsets, DESCRIPTIONS[name])

    rows = int(cfg["rows"])
    W = _to_storage(_normal(rng_for(seed, cid, 0), (cout, cin), cfg["w_std"]), dtype)[None]
    if "student_df" in cfg:
        x32 = rng_for(seed, cid, 1).standard_t(cfg["student_df"], (rows, cin)).astype(np.float32)
    else:
        x32 = _normal(rng_for(seed, cid, 1), (rows, cin), 1.0)
    if "outlier_frac" in cfg:
        n_out = max(1, int(np.floor(cfg["outlier_frac"] * cin)))   # at least one, also when shrunk
        ch = rng_for(seed, cid, 2).choice(cin, size=n_out, replace=False)
        x32[:, ch] *= np.float32(cfg["outlier_mul"])
    X = _to_storage(x32, dtype)
    offsets = np.array([0, rows], dtype=np.int64)
    return Workload(name, dtype, mode, 1, cout, cin, W, X, None, offsets, DESCRIPTIONS[name])
