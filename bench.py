"""Benchmark of the whole calibration path on one MI355X.

One step = one pass of the hot path over one synthetic layer: max calibration of W (global amax),
Hessian / importance / cross-matrix accumulation over the layer's tokens, and the 126-candidate
E4M3 scale sweep over every weight block.  Inputs are resident in HBM before timing starts; X and W
rotate over enough copies (>= 1 GiB) that every step streams them from HBM rather than from the
256 MB Infinity Cache.

Prints ONE JSON line.  `value` is weight blocks scored per second for the whole step.  `roofline`
describes the dominant kernel (the sweep), timed with HIP events on the stream it runs on;
`accumulate` gives the accumulation's algorithmic HBM rate.  Each phase reports the mean of
back-to-back calls (the figure the roofline uses), the median, minimum and maximum of the same
calls timed one by one, and the latency of a single call on an idle GPU.  `cpu_baseline` is the
float64 oracle timed on this host's cores (see --help for the sample).

Default workload: the largest single-GPU layer, the fused MoE gate_up with 512 experts (W bf16
[512, 1280, 2560], 8192 tokens routed top-10 by Zipf(1.1), 81920 rows).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "16-elem blocks scored/sec (126 scales each) + Hessian accum GB/s, % roofline"
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E, GB/s
# fp32 vector peak of MI355X: 256 CU x 4 SIMD x 16 lanes x 2 flop (FMA) x 2 (packed fp32) x
# 2.4 GHz = 157.3 TFLOP/s (the dense fp32 matrix peak is the same figure).  The sweep's
# algorithmic fp32 flops are counted against it; its busy unit is the VALU (SQ counters).
FP32_PEAK_TFLOPS = 157.3
# algorithmic flops per block (126 candidates): fake-quant 2/elem, H e 512, e^T(He) 32 (+ 2 e^T b 32)
FLOPS_FULL = 126 * (32 + 512 + 32)
FLOPS_COUPLED = 126 * (32 + 512 + 32 + 32) + 512
FLOPS_DIAG = 126 * (32 + 48)
# The flop counts above score every one of the 126 candidates of every block.  The kernels prove
# for most blocks that a range of codes cannot hold the argmin and do not score those codes, so
# the algorithmic rate can exceed the fp32 peak; `counters` gives the share of VALU issue slots
# the kernel actually used.
WORK_NOTE_FULL = ("achieved counts all 126 candidates per block; codes 1-96 are skipped for blocks "
                  "where a proven lower bound (the column's certified smallest Hessian eigenvalue, or "
                  "the triangle inequality in its seminorm) rules them out, so achieved can exceed "
                  "peak; counters.valu_issue_frac is the issue share actually used")
WORK_NOTE_DIAG = ("achieved counts all 126 candidates per block; only a 32-code window proven to hold "
                  "the argmin is scored, so achieved can exceed peak; counters.valu_issue_frac is the "
                  "issue share actually used")


def code_digest(paths):
    """sha256 of kernel sources (one path or a list: the kernel file and the headers it includes)
    with comments and whitespace removed: it changes when the code changes, not when a comment
    does."""
    import hashlib
    import re
    if isinstance(paths, str):
        paths = [paths]
    parts = []
    for path in paths:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        parts.append(" ".join(text.split()))
    return hashlib.sha256("\n".join(parts).encode()).hexdigest()


def _record_current(v):
    """True when a counter record's kernel sources still have the digest it was taken with."""
    src = v.get("source")
    if not src:
        return False
    src = [src] if isinstance(src, str) else src
    try:
        return code_digest([os.path.join(ROOT, "nvfp4_scale_calibration_lh_amd", "csrc", s) for s in src]) \
            == v.get("code_sha256")
    except OSError:
        return False


def measured_traffic(cfg, prefix):
    """HBM bytes per call of the kernels whose names start with `prefix` (a string or a tuple of
    them), from the rocprofv3
    FETCH_SIZE / WRITE_SIZE passes recorded in profiles/traffic.json, scaled by the copy-kernel
    calibration factors.  None when no record exists or a kernel's code changed since."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    kern = rec.get("workloads", {}).get(cfg, {})
    total, found = 0.0, False
    for name, v in kern.items():
        if not name.startswith(prefix):
            continue
        if not _record_current(v):
            return None
        total += v["fetch_kib"] * 1024 * rec["fetch_factor"] + v["write_kib"] * 1024 * rec["write_factor"]
        found = True
    return total if found else None


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="c5", choices=list(synth.CONFIGS))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--fq", action="store_true",
                   help="activation-aware workload: make X_q from X inside the accumulation kernel "
                        "(lh_accumulate_act_aware_fq) instead of reading a stored X_q")
    p.add_argument("--cpu-sample-blocks", type=int, default=16384,
                   help="blocks per host core of the oracle's sweep timed for the CPU baseline")
    p.add_argument("--rotate-gib", type=float, default=1.0)
    p.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                   help="only run a plain elementwise copy (torch.neg) of MIB MiB, 5 times, for "
                        "calibrating HBM byte counters, and exit")
    return p.parse_args()


def to_dev(torch, a, dtype, dev):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(dev)


def _oracle_sweep_chunk(task):
    """Pool worker: the oracle's search over one chunk of blocks with one BLAS thread; returns the
    chunk's block count."""
    import oracle
    from threadpoolctl import threadpool_limits
    mode, w, g, H, P, hidx, imp = task
    with threadpool_limits(1):
        if mode == "diag":
            oracle.sweep_blocks_diag(w, g, imp)
        else:
            oracle.sweep_blocks(w, g, H, P, hidx=hidx)
    return len(w)


def cpu_baseline(wl, Xq64, per_core_blocks):
    """The float64 oracle as it stands, on this host's cores: absmax, accumulation over every row,
    and the 126-candidate search over a seeded sample of blocks spread over a Pool of one process
    per core (one BLAS thread each).  Grouped layers take the sample from a seeded set of whole
    experts that includes the largest and the smallest one; absmax is timed on those experts.
    Returns the whole-step blocks/s with the sampled phases projected per block (or element)."""
    import multiprocessing as mp

    import oracle
    from threadpoolctl import threadpool_limits
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    G, cout, nb = wl.n_groups, wl.cout, wl.n_blocks
    rng = np.random.default_rng(12345)
    if G == 1:
        groups = np.array([0])
    else:
        T = np.diff(wl.offsets)
        pick = set(rng.choice(G, size=min(6, G), replace=False).tolist())
        pick |= {int(np.argmax(T)), int(np.argmin(T))}
        groups = np.array(sorted(pick))
    W_s = [wl.W_f64(int(g)) for g in groups]
    with threadpool_limits(1):
        t0 = time.perf_counter()
        amax_s = np.array([oracle.absmax(w[None])[0] for w in W_s])
        t_abs = (time.perf_counter() - t0) * G / len(groups)
    X64 = wl.X_f64()
    with threadpool_limits(cores):
        t0 = time.perf_counter()
        if wl.mode == "act":
            H, P = oracle.accumulate_act_aware(X64, Xq64, wl.offsets)
        elif wl.mode == "diag":
            H, P = None, None
            _, imp = oracle.accumulate(X64, wl.offsets, want_h=False, want_imp=True)
        else:
            H, P = oracle.accumulate(X64, wl.offsets)[0], None
        t_acc = time.perf_counter() - t0
    del X64
    B = per_core_blocks * cores
    per_g = max(1, B // len(groups))
    tasks = []
    chunk = 2048
    for k, g in enumerate(groups):
        flat = rng.choice(cout * nb, size=min(per_g, cout * nb), replace=False)
        c, n = flat // nb, flat % nb
        w = W_s[k].reshape(cout, nb, 16)[c, n]
        gs = np.repeat(oracle.global_scale(amax_s[k:k + 1])[0], len(flat))
        for a in range(0, len(flat), chunk):
            sl = slice(a, a + chunk)
            if wl.mode == "diag":
                tasks.append(("diag", w[sl], gs[sl], None, None, None, imp[g].reshape(nb, 16)[n[sl]]))
            else:
                tasks.append(("full", w[sl], gs[sl], H[g], None if P is None else P[g], n[sl], None))
    ctx = mp.get_context("fork")
    with ctx.Pool(cores) as pool:
        pool.map(_oracle_sweep_chunk, tasks[:cores])          # start-up, not timed
        t0 = time.perf_counter()
        done = sum(pool.map(_oracle_sweep_chunk, tasks, chunksize=1))
        t_sw = time.perf_counter() - t0
    blocks = wl.weight_blocks
    step = t_abs + t_acc + t_sw / done * blocks
    where = (f"experts {groups.tolist()} of {G} (largest and smallest routed-token counts included)"
             if G > 1 else "the layer")
    return {"value": blocks / step, "unit": "blocks/s", "cores": cores, "kind": "oracle",
            "sample": (f"float64 NumPy oracle on {cores} host cores: accumulation over all {wl.rows} rows "
                       f"({t_acc:.2f} s, BLAS on {cores} threads); absmax of {where}, projected per element "
                       f"to all {G} group(s) ({t_abs:.2f} s projected); 126-candidate search of {done} seeded "
                       f"random blocks of {where} over a {cores}-process pool ({t_sw:.2f} s wall), projected "
                       f"per block to all {blocks} blocks"),
            "phases_s": {"absmax": t_abs, "accumulate": t_acc, "sweep_projected": t_sw / done * blocks}}


def sq_shares(cfg, kernel_prefix):
    """VALU-issue and MFMA-busy shares of the kernel's cycles from the rocprofv3 SQ counter record
    in profiles/sq_counters.json (None when absent or when the kernel's code changed since)."""
    try:
        with open(os.path.join(ROOT, "profiles", "sq_counters.json")) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    for name, v in rec.get("workloads", {}).get(cfg, {}).items():
        if not name.startswith(kernel_prefix):
            continue
        if not _record_current(v):
            return None
        return {"kernel": name, "valu_issue_frac": v["valu_issue_frac"], "mfma_busy_frac": v["mfma_busy_frac"]}
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus above 1 is not supported",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import nvfp4_scale_calibration_lh_amd as lh

    dev = torch.device("cuda:0")
    if args.copy_calib:
        n = args.copy_calib * 2 ** 20 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes_read": n * 4, "copy_calib_bytes_written": n * 4, "launches": 5}))
        return
    wl = synth.make(args.config)
    G, cout, cin, rows = wl.n_groups, wl.cout, wl.cin, wl.rows
    nb = cin // 16
    blocks = wl.weight_blocks
    esz = 2 if wl.dtype == "bf16" else 4
    x_bytes = rows * cin * esz * (2 if wl.mode == "act" and not args.fq else 1)   # X (and a stored X_q)
    w_bytes = G * cout * cin * esz
    copies = max(1, min(64, int(np.ceil(args.rotate_gib * 2 ** 30 / max(1, x_bytes + w_bytes)))))
    free = torch.cuda.mem_get_info(dev)[0]
    copies = max(1, min(copies, int(0.5 * free // max(1, x_bytes + w_bytes))))

    W0 = to_dev(torch, wl.W, wl.dtype, dev)
    X0 = to_dev(torch, wl.X, wl.dtype, dev)
    Ws = [W0] + [W0.clone() for _ in range(copies - 1)]
    Xs = [X0] + [X0.clone() for _ in range(copies - 1)]
    off = torch.from_numpy(wl.offsets).to(dev) if G > 1 else None
    act = wl.mode == "act"
    fq = args.fq and act
    if act:
        # the input quantizer's amax per group (its own max calibration), and for the two-input
        # form the stored X_q that quantizer emits, made once by the library before timing
        x_amax = torch.stack([X0[int(wl.offsets[g]):int(wl.offsets[g + 1])].abs().max().float()
                              for g in range(G)])
        if not fq:
            Xq0 = lh.lh_activation_fake_quant(X0, x_amax, offsets=off)
            Xqs = [Xq0] + [Xq0.clone() for _ in range(copies - 1)]

    amax = torch.empty(G, dtype=torch.float32, device=dev)
    H = torch.empty((G, nb, 16, 16), dtype=torch.float32, device=dev)
    P = torch.empty_like(H) if act else None
    imp = torch.empty((G, cin), dtype=torch.float32, device=dev)
    code = torch.empty((G, cout, nb), dtype=torch.uint8, device=dev)
    fp4 = torch.empty((G, cout, cin // 2), dtype=torch.uint8, device=dev)
    loss = torch.empty((G, cout, nb), dtype=torch.float32, device=dev)

    def absmax(j):
        lh.lh_absmax(Ws[j], amax)

    def accumulate(j):
        if fq:
            lh.lh_accumulate_act_aware_fq(Xs[j], x_amax, H=H, P=P, offsets=off)
        elif act:
            lh.lh_accumulate_act_aware(Xs[j], Xqs[j], H=H, P=P, offsets=off)
        elif wl.mode == "diag":
            lh.lh_accumulate(Xs[j], H=None, imp=imp, offsets=off, want_h=False, want_imp=True)
        else:
            lh.lh_accumulate(Xs[j], H=H, offsets=off)

    def sweep(j):
        if wl.mode == "diag":
            lh.lh_scale_sweep_diag(Ws[j], amax, imp, code, fp4, loss)
        else:
            lh.lh_scale_sweep(Ws[j], amax, H, P, code, fp4, loss)

    def step(i):
        j = i % copies
        absmax(j)
        accumulate(j)
        sweep(j)

    stream = torch.cuda.current_stream(dev)     # the stream the library launches on

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    gpu_ms_step = e0.elapsed_time(e1) / args.steps

    # Per-phase durations: the same calls back to back (rotating inputs) with an event on the
    # library's stream between every two calls, queued behind a ~2 ms spin so that for phases of a
    # few microseconds the events time the kernels rather than the host's launch rate.  The mean
    # over the calls is the steady-state launch duration (the roofline's figure); median, min and
    # max come from the individual intervals.  Single-call latency: one call on an idle GPU,
    # events around it, the median of five.
    def phase(fn):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        torch.cuda._sleep(4_000_000)
        ev[0].record(stream)
        for i in range(args.steps):
            fn(i % copies)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
        single = []
        for i in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record(stream)
            fn(i % copies)
            b.record(stream)
            torch.cuda.synchronize()
            single.append(a.elapsed_time(b))
        return {"avg_launch_ms": ev[0].elapsed_time(ev[-1]) / args.steps, "median_ms": float(np.median(per)),
                "min_ms": float(np.min(per)), "max_ms": float(np.max(per)),
                "single_call_ms": float(np.median(single))}

    t_abs = phase(absmax)
    t_acc = phase(accumulate)
    t_sw = phase(sweep)
    ms_abs, ms_acc, ms_sw = t_abs["avg_launch_ms"], t_acc["avg_launch_ms"], t_sw["avg_launch_ms"]
    # after the path: the fake-quantized bf16 weights and block amax the chosen codes define
    wq_buf = torch.empty((G, cout, cin), dtype=torch.bfloat16, device=dev)
    bam_buf = torch.empty((G, cout, nb), dtype=torch.float32, device=dev)
    t_dq = phase(lambda j: lh.lh_dequantize(code, fp4, amax, dtype=torch.bfloat16, Wq=wq_buf, block_amax=bam_buf))
    ms_dq = t_dq["avg_launch_ms"]
    del wq_buf, bam_buf
    dq_bytes = blocks * (1 + 8 + 32 + 4) + G * 4
    # grouped full-Hessian layers: the same accumulation and sweep in one launch with H kept on chip
    # (lh_accumulate_sweep), bit-identical results; timed as a phase of its own
    t_fused = None
    if G > 1 and wl.mode == "full" and cout <= 8192:
        t_fused = phase(lambda j: lh.lh_accumulate_sweep(Xs[j], Ws[j], amax, off, code, fp4, loss))
    # reference: a device-to-device copy of X (the same rotating sources), bytes read + written
    xdst = torch.empty_like(Xs[0])
    ms_copy = phase(lambda j: xdst.copy_(Xs[j]))["avg_launch_ms"]
    del xdst

    flops_blk = FLOPS_DIAG if wl.mode == "diag" else (FLOPS_COUPLED if act else FLOPS_FULL)
    sweep_tflops = flops_blk * blocks / (ms_sw * 1e-3) / 1e12
    acc_bytes = x_bytes + (G * cin * 4 if wl.mode == "diag" else G * nb * 1024 * (2 if act else 1))
    acc_gbs = acc_bytes / (ms_acc * 1e-3) / 1e9
    copy_gbs = 2 * Xs[0].numel() * Xs[0].element_size() / (ms_copy * 1e-3) / 1e9
    abs_gbs = w_bytes / (ms_abs * 1e-3) / 1e9
    rec = args.config + ("fq" if fq else "")   # key of the counter records
    roof = {"bound": "alu", "achieved": sweep_tflops, "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": sweep_tflops / FP32_PEAK_TFLOPS, "traffic": measured_traffic(rec, ("k_sweep", "k_column_mu")),
            "kernel": "sweep", "flops_per_block": flops_blk, "blocks_per_launch": blocks,
            "avg_launch_ms": ms_sw, "counters": sq_shares(rec, "k_sweep_diag_win" if wl.mode == "diag" else "k_sweep_full<"),
            "work_note": WORK_NOTE_DIAG if wl.mode == "diag" else WORK_NOTE_FULL}

    out = {
        "metric": METRIC,
        "value": blocks / (ms_step * 1e-3),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "gpu_ms_per_step": gpu_ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.description, "name": args.config, "n_groups": G, "cout": cout,
                   "cin": cin, "rows": rows, "blocks": blocks, "input_dtype": wl.dtype,
                   "mode": wl.mode, "rotating_copies": copies,
                   **({"x_q": "made in the accumulation kernel"} if fq else {})},
        "roofline": roof,
        "accumulate": {**t_acc, "algorithmic_bytes": acc_bytes, "achieved_gbs": acc_gbs,
                       "peak_gbs": HBM_PEAK_GBS, "frac": acc_gbs / HBM_PEAK_GBS,
                       "traffic": measured_traffic(rec, ("k_acc", "k_imp")),
                       "copy_gbs": copy_gbs, "frac_of_copy": acc_gbs / copy_gbs},
        "absmax": {**t_abs, "achieved_gbs": abs_gbs, "frac": abs_gbs / HBM_PEAK_GBS},
        "dequantize": {**t_dq, "algorithmic_bytes": dq_bytes,
                       "achieved_gbs": dq_bytes / (ms_dq * 1e-3) / 1e9,
                       "frac": dq_bytes / (ms_dq * 1e-3) / 1e9 / HBM_PEAK_GBS, "outside_step": True},
        "sweep": {**t_sw, "blocks_per_s": blocks / (ms_sw * 1e-3), "tflops": sweep_tflops},
    }
    if t_fused is not None:
        out["fused_accumulate_sweep"] = {**t_fused, "blocks_per_s": blocks / (t_fused["avg_launch_ms"] * 1e-3),
                                         "vs_two_calls": (ms_acc + ms_sw) / t_fused["avg_launch_ms"],
                                         "outside_step": True}
    if not args.no_cpu_baseline:
        del Ws, Xs, W0, X0
        if act:
            del x_amax
            if not fq:
                del Xqs, Xq0
        torch.cuda.empty_cache()
        Xq64 = None
        if act:   # the oracle's own X_q (an input of its accumulation, made before its timing)
            import oracle
            X64 = wl.X_f64()
            am = [np.abs(X64[wl.offsets[g]:wl.offsets[g + 1]]).max(initial=0.0) for g in range(G)]
            Xq64 = oracle.activation_fake_quant(X64, am, wl.offsets, bf16=wl.dtype == "bf16")
            del X64
        out["cpu_baseline"] = cpu_baseline(wl, Xq64, args.cpu_sample_blocks)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
