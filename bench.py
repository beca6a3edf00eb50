"""Benchmark of the whole calibration path on one MI355X.

One step = one pass of the hot path over one synthetic layer: max calibration of W (global amax),
Hessian / importance / cross-matrix accumulation over the layer's tokens, and the 126-candidate
E4M3 scale sweep over every weight block.  Inputs are resident in HBM before timing starts; X and W
rotate over enough copies (>= 1 GiB) that every step streams them from HBM rather than from the
256 MB Infinity Cache.

Prints ONE JSON line.  `value` is weight blocks scored per second for the whole step.  `roofline`
describes the dominant kernel (the sweep), timed with HIP events on the stream it runs on;
`accumulate` gives the accumulation's algorithmic HBM rate.  `cpu_baseline` is the float64 oracle
timed on this host (see --help for the sample).

Default workload: the dense 2048x2048 layer (bf16 W, 8192 tokens with 1% outlier channels).
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
FP32_PEAK_TFLOPS = 157.3           # MI355X dense fp32 matrix (MFMA) peak
VALU_FP32_TFLOPS = 78.6            # fp32 vector FMA without packed math: 256 CU x 4 SIMD x 16 lanes x 2 x 2.4 GHz
# algorithmic flops per block (126 candidates): fake-quant 2/elem, H e 512, e^T(He) 32 (+ 2 e^T b 32)
FLOPS_FULL = 126 * (32 + 512 + 32)
FLOPS_COUPLED = 126 * (32 + 512 + 32 + 32) + 512
FLOPS_DIAG = 126 * (32 + 48)


def code_digest(path):
    """sha256 of a kernel source with its comments and whitespace removed: it changes when the
    code changes, not when a comment does."""
    import hashlib
    import re
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


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
        src = os.path.join(ROOT, "nvfp4_scale_calibration_lh_amd", "csrc", v.get("source", ""))
        try:
            if code_digest(src) != v.get("code_sha256"):
                return None
        except OSError:
            return None
        total += v["fetch_kib"] * 1024 * rec["fetch_factor"] + v["write_kib"] * 1024 * rec["write_factor"]
        found = True
    return total if found else None


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="c2", choices=list(synth.CONFIGS))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--fq", action="store_true",
                   help="activation-aware workload: make X_q from X inside the accumulation kernel "
                        "(lh_accumulate_act_aware_fq) instead of reading a stored X_q")
    p.add_argument("--cpu-sample-blocks", type=int, default=65536,
                   help="blocks of the oracle's sweep timed for the CPU baseline")
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


def cpu_baseline(wl, sample_blocks):
    """The float64 oracle, single-threaded: full absmax and accumulation, sweep on a seeded sample
    of blocks; returns the projected whole-step blocks/s."""
    import oracle
    from threadpoolctl import threadpool_limits
    if wl.n_groups != 1:
        raise RuntimeError("the CPU baseline is defined for the dense workloads")
    with threadpool_limits(1):
        t0 = time.perf_counter()
        Wo = wl.W_f64()
        amax = oracle.absmax(Wo)
        t_abs = time.perf_counter() - t0
        t0 = time.perf_counter()
        if wl.mode == "act":
            H, P = oracle.accumulate_act_aware(wl.X_f64(), wl.Xq_f64(), wl.offsets)
        elif wl.mode == "diag":
            H, P = None, None
            _, imp = oracle.accumulate(wl.X_f64(), wl.offsets, want_h=False, want_imp=True)
        else:
            H, P = oracle.accumulate(wl.X_f64(), wl.offsets)[0], None
        t_acc = time.perf_counter() - t0
        rng = np.random.default_rng(12345)
        nb = wl.n_blocks
        B = min(sample_blocks, wl.cout * nb)
        flat = rng.choice(wl.cout * nb, size=B, replace=False)
        c, n = flat // nb, flat % nb
        w = Wo[0].reshape(wl.cout, nb, 16)[c, n]
        g = np.repeat(oracle.global_scale(amax)[0], B)
        t0 = time.perf_counter()
        if wl.mode == "diag":
            oracle.sweep_blocks_diag(w, g, imp[0].reshape(nb, 16)[n])
        else:
            oracle.sweep_blocks(w, g, H[0], None if P is None else P[0], hidx=n)
        t_sw = time.perf_counter() - t0
    blocks = wl.weight_blocks
    step = t_abs + t_acc + t_sw / B * blocks
    return {"value": blocks / step, "unit": "blocks/s", "cores": 1, "kind": "oracle",
            "sample": (f"float64 NumPy oracle, 1 thread: absmax and accumulation over the whole layer "
                       f"({t_abs + t_acc:.2f} s), sweep over {B} seeded random blocks ({t_sw:.2f} s); "
                       f"whole-step time projected per block to all {blocks} blocks")}


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
    Xq0 = to_dev(torch, wl.Xq, wl.dtype, dev) if wl.Xq is not None else None
    Ws = [W0] + [W0.clone() for _ in range(copies - 1)]
    Xs = [X0] + [X0.clone() for _ in range(copies - 1)]
    Xqs = ([Xq0] + [Xq0.clone() for _ in range(copies - 1)]) if Xq0 is not None and not args.fq else None
    off = torch.from_numpy(wl.offsets).to(dev) if G > 1 else None

    amax = torch.empty(G, dtype=torch.float32, device=dev)
    H = torch.empty((G, nb, 16, 16), dtype=torch.float32, device=dev)
    P = torch.empty_like(H) if wl.mode == "act" else None
    imp = torch.empty((G, cin), dtype=torch.float32, device=dev)
    code = torch.empty((G, cout, nb), dtype=torch.uint8, device=dev)
    fp4 = torch.empty((G, cout, cin // 2), dtype=torch.uint8, device=dev)
    loss = torch.empty((G, cout, nb), dtype=torch.float32, device=dev)

    def absmax(j):
        lh.lh_absmax(Ws[j], amax)

    fq = args.fq and wl.mode == "act"
    if fq:   # the input quantizer's amax comes from its own (earlier) max calibration
        x_amax = torch.stack([Xs[0][int(wl.offsets[g]):int(wl.offsets[g + 1])].abs().max().float()
                              for g in range(G)])

    def accumulate(j):
        if fq:
            lh.lh_accumulate_act_aware_fq(Xs[j], x_amax, H=H, P=P, offsets=off)
        elif wl.mode == "act":
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

    # per-phase launch durations: the same calls back to back (rotating inputs), between two
    # events on the library's stream, so each average is the kernel's steady-state duration
    # (a ~2 ms spin first keeps the GPU busy while the calls are queued, so for phases of a few
    # microseconds the events time the kernels rather than the host's launch rate)
    def phase_ms(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(4_000_000)
        a.record(stream)
        for i in range(args.steps):
            fn(i % copies)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    ms_abs = phase_ms(absmax)
    ms_acc = phase_ms(accumulate)
    ms_sw = phase_ms(sweep)
    # after the path: the fake-quantized bf16 weights and block amax the chosen codes define
    wq_buf = torch.empty((G, cout, cin), dtype=torch.bfloat16, device=dev)
    bam_buf = torch.empty((G, cout, nb), dtype=torch.float32, device=dev)
    ms_dq = phase_ms(lambda j: lh.lh_dequantize(code, fp4, amax, dtype=torch.bfloat16, Wq=wq_buf, block_amax=bam_buf))
    del wq_buf, bam_buf
    dq_bytes = blocks * (1 + 8 + 32 + 4) + G * 4
    # reference: a device-to-device copy of X (the same rotating sources), bytes read + written
    xdst = torch.empty_like(Xs[0])
    ms_copy = phase_ms(lambda j: xdst.copy_(Xs[j]))
    del xdst

    flops_blk = FLOPS_DIAG if wl.mode == "diag" else (FLOPS_COUPLED if wl.mode == "act" else FLOPS_FULL)
    sweep_tflops = flops_blk * blocks / (ms_sw * 1e-3) / 1e12
    acc_bytes = x_bytes + (G * cin * 4 if wl.mode == "diag" else G * nb * 1024 * (2 if wl.mode == "act" else 1))
    acc_gbs = acc_bytes / (ms_acc * 1e-3) / 1e9
    copy_gbs = 2 * Xs[0].numel() * Xs[0].element_size() / (ms_copy * 1e-3) / 1e9
    abs_gbs = w_bytes / (ms_abs * 1e-3) / 1e9
    if wl.mode == "diag":
        roof = {"bound": "alu", "achieved": sweep_tflops, "peak": VALU_FP32_TFLOPS, "unit": "TFLOP/s",
                "frac": sweep_tflops / VALU_FP32_TFLOPS, "traffic": None}
    else:
        roof = {"bound": "mfma", "achieved": sweep_tflops, "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": sweep_tflops / FP32_PEAK_TFLOPS, "traffic": None}
    rec = args.config + ("fq" if args.fq and wl.mode == "act" else "")   # key of the counter record
    roof["traffic"] = measured_traffic(rec, "k_sweep")
    roof.update({"kernel": "sweep", "flops_per_block": flops_blk, "blocks_per_launch": blocks,
                 "avg_launch_ms": ms_sw})

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
                   **({"x_q": "made in the accumulation kernel"} if args.fq and wl.mode == "act" else {})},
        "roofline": roof,
        "accumulate": {"avg_launch_ms": ms_acc, "algorithmic_bytes": acc_bytes, "achieved_gbs": acc_gbs,
                       "peak_gbs": HBM_PEAK_GBS, "frac": acc_gbs / HBM_PEAK_GBS,
                       "traffic": measured_traffic(rec, ("k_acc", "k_imp")),
                       "copy_gbs": copy_gbs, "frac_of_copy": acc_gbs / copy_gbs},
        "absmax": {"avg_launch_ms": ms_abs, "achieved_gbs": abs_gbs, "frac": abs_gbs / HBM_PEAK_GBS},
        "dequantize": {"avg_launch_ms": ms_dq, "algorithmic_bytes": dq_bytes,
                       "achieved_gbs": dq_bytes / (ms_dq * 1e-3) / 1e9,
                       "frac": dq_bytes / (ms_dq * 1e-3) / 1e9 / HBM_PEAK_GBS, "outside_step": True},
        "sweep": {"avg_launch_ms": ms_sw, "blocks_per_s": blocks / (ms_sw * 1e-3), "tflops": sweep_tflops},
    }
    if not args.no_cpu_baseline and G == 1:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample_blocks)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
