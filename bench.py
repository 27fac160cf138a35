"""Benchmark of the sparse MoE FFN layer forward on one MI355X.

A step is one whole layer forward (router + top-k, permute, grouped expert
FFNs, combine) over one batch of seeded synthetic tokens already resident in
HBM.  Prints ONE JSON line with tokens/s, the roofline position of the
dominant kernel (the grouped up-projection GEMM) measured with HIP events
on the stream it runs on, and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
MFMA_F32_PEAK_TFLOPS = 157.3     # MI355X fp32 vector/matrix
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_prefill")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="budget of the CPU-oracle sample (0 = skip)")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-shaped leg of the default run")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device copy first (a kernel of "
                         "known traffic for scaling HBM byte counters)")
    return ap.parse_args()


# the grouped-GEMM kernels and the headers they compile
GEMM_SOURCES = [os.path.join(ROOT, "sparse_mixture_experts_50_amd", "csrc", f)
                for f in ("gemm.hip", "gemm_tall.hip", "common.h", "kernels.h")]


def source_digest() -> str:
    h = hashlib.sha256()
    for path in GEMM_SOURCES:
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per launch of the up-projection GEMM from the committed
    counter summary of this workload, or None if there is none or the GEMM
    source changed since it was taken."""
    path = os.path.join(ROOT, "profiles",
                        f"gemm_up_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("gemm_source_sha256_16") != source_digest():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic(wl, counts, kept):
    """FLOPs and bytes of one forward (kept rows only, touched experts)."""
    import numpy as np
    es = wl.elem_bytes
    ew = 1 if wl.expert_fp8 else es        # bytes per expert-matrix weight
    sc = 4 if wl.expert_fp8 else 0         # fp32 scale per output channel
    nu = 2 if wl.activation == "swiglu" else 1   # up matrices (W1[, W3])
    rows = int(np.sum(kept)) + wl.n_shared * wl.T     # expert GEMM rows
    touched = int(np.sum(kept > 0)) + wl.n_shared
    flops = 2.0 * wl.T * wl.d * wl.E + 2.0 * (nu + 1) * rows * wl.d * wl.d_ff
    expert_bytes = ((nu + 1) * wl.d * wl.d_ff * ew + (wl.d + nu * wl.d_ff) * sc
                    + (wl.d + nu * wl.d_ff if wl.linear_biases else 0) * es)
    bytes_ = (wl.E * wl.d * es + touched * expert_bytes +
              2 * wl.T * wl.d * es)
    up_flops = 2.0 * nu * rows * wl.d * wl.d_ff
    up_bytes = (nu * touched * wl.d_ff * (wl.d * ew + sc) +
                rows * (wl.d + wl.d_ff) * es)
    return dict(flops=flops, bytes=bytes_, rows=rows, touched=touched,
                up_flops=up_flops, up_bytes=up_bytes)


def roofline_bound(alg, flops_peak_tflops) -> str:
    """The roofline bound of the up GEMM: whichever of its algorithmic
    bytes at the HBM peak and its FLOPs at the matrix peak takes longer
    (arithmetic intensity below or above the ridge point, 2500 / 8 = 312
    FLOP per byte for bf16)."""
    t_hbm = alg["up_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = alg["up_flops"] / (flops_peak_tflops * 1e12)
    return "hbm" if t_hbm > t_mfma else "mfma"


def dense_gemm_tflops(M, N, K, dev) -> float:
    """torch.matmul (hipBLASLt) bf16 rate on one dense M x N x K product."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    a = torch.randn(M, K, device=dev, dtype=torch.bfloat16, generator=g)
    b = torch.randn(N, K, device=dev, dtype=torch.bfloat16, generator=g)
    for _ in range(3):
        torch.matmul(a, b.t())
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        torch.matmul(a, b.t())
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    del a, b
    return 2.0 * M * N * K / (ms * 1e9)


def cpu_baseline(wl, inp, budget_s):
    """The oracle, as it stands, on the first n tokens of the same inputs
    (n sized to the time budget), through the whole layer."""
    import numpy as np
    import torch
    import oracle
    host = {k: (v.cpu() if isinstance(v, torch.Tensor) else v)
            for k, v in inp.items()}
    cores = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp:
        cores = min(cores, int(omp))

    def run(n):
        sub = dict(host)
        sub["x"] = host["x"][:n]
        t0 = time.perf_counter()
        if wl.routing == "expert_choice":
            C = min(n, oracle.capacity(n, wl.E, wl.capacity_factor))
            oracle.forward_expert_choice(sub, C, wl.alpha,
                                         activation=wl.activation)
        else:
            oracle.forward(sub, wl.k, wl.capacity_factor, wl.alpha,
                           activation=wl.activation)
        return time.perf_counter() - t0

    n = min(wl.T, max(1, cores))
    dt = run(n)
    while dt < budget_s / 2 and n < wl.T:
        n = min(wl.T, max(n + 1, int(n * min(8.0, budget_s / max(dt, 1e-3)
                                              / 2))))
        dt = run(n)
    return dict(value=n / dt, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"first {n} of {wl.T} tokens of {wl.name}, whole "
                       f"layer (router to combine) in fp64, {dt:.1f} s")


def time_layer(wl, layer, weights, xs, steps, warmup, stream):
    """Run ``warmup`` untimed and ``steps`` timed layer calls (call i on
    xs[i % len(xs)]) through the entry points moe_forward chains
    (moe_route_dispatch, moe_ffn_up, moe_ffn_down, moe_combine) on
    ``stream``.  The timed region holds only the calls, bracketed by two
    HIP events: an event recorded between two kernels holds the queue for
    ~5 us, a cost the layer itself does not have.  The up-projection GEMM's
    duration comes from ``steps`` back-to-back launches of it on the last
    call's routing, right after, bracketed the same way."""
    import torch

    import sparse_mixture_experts_50_amd as moe
    desc, r, ws, y = layer.buffers(wl.T)
    n_x = len(xs)

    def step(i):
        x = xs[i % n_x]
        moe.moe_route_dispatch(desc, x, weights, r, ws)
        moe.moe_ffn_up(desc, x, weights, r, ws)
        moe.moe_ffn_down(desc, weights, r, ws)
        moe.moe_combine(desc, r, y, ws)

    log(f"[bench] {wl.name}: warmup {warmup}")
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] {wl.name}: timing {steps} steps")
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    log(f"[bench] {wl.name}: {steps} launches of the up GEMM")
    x = xs[(steps - 1) % n_x]
    u0 = torch.cuda.Event(enable_timing=True)
    u1 = torch.cuda.Event(enable_timing=True)
    u0.record(stream)
    for i in range(steps):
        moe.moe_ffn_up(desc, x, weights, r, ws)
    u1.record(stream)
    torch.cuda.synchronize()
    counts = r.counts.cpu().numpy()
    kept = r.kept.cpu().numpy()
    assert int(counts.sum()) == wl.T * wl.k
    return dict(desc=desc, total_ms=total_ms, wall=wall,
                ms_per_step=total_ms / steps,
                up_avg_ms=u0.elapsed_time(u1) / steps,
                counts=counts, kept=kept)


def decode_leg(weights, dev, stream, warmup=10):
    """The Mixtral-shaped decode layer (32 tokens per call, the same expert
    weights as the prefill layer), timed over its 200 calls with distinct
    x: per-call time, tokens/s and the whole layer's algorithmic HBM bytes
    per call against the HBM peak, plus the up GEMM's own rate."""
    import numpy as np

    import sparse_mixture_experts_50_amd as moe
    import workloads
    wl = workloads.get("mixtral_decode")
    xs = [workloads.make_x(wl, dev, c) for c in range(wl.calls)]
    layer = moe.MoeLayer(weights, wl.k, wl.capacity_factor, wl.alpha,
                         routing=wl.routing, activation=wl.activation)
    m = time_layer(wl, layer, weights, xs, wl.calls, warmup, stream)
    # touched experts and kept rows vary by call: every one of the 200
    # calls touches all 8 experts of this workload (checked on the last)
    alg = algorithmic(wl, m["counts"], m["kept"])
    ms = m["ms_per_step"]
    layer_gbs = alg["bytes"] / (ms * 1e6)
    up_gbs = alg["up_bytes"] / (m["up_avg_ms"] * 1e6)
    return {
        "workload": wl.name, "calls": wl.calls, "warmup": warmup,
        "tokens_per_call": wl.T,
        "ms_per_call": ms,
        "tokens_per_s": wl.T / (ms / 1e3),
        "layer_bytes_per_call": alg["bytes"],
        "layer_hbm_gbs": layer_gbs,
        "layer_hbm_frac": layer_gbs / HBM_PEAK_GBS,
        "up_gemm_ms": m["up_avg_ms"],
        "up_gemm_gbs": up_gbs,
        "up_gemm_frac": up_gbs / HBM_PEAK_GBS,
        "experts_touched_last_call": int(np.sum(m["kept"] > 0)),
        "gemm_variants": [moe.moe_gemm_variant(m["desc"], True),
                          moe.moe_gemm_variant(m["desc"], False)],
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus "
              f"{args.gpus}); the layer is not sharded across GPUs",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import sparse_mixture_experts_50_amd as moe
    import workloads

    wl = workloads.get(args.workload)
    steps = args.steps if args.steps is not None else (
        wl.calls if wl.calls > 1 else 20)
    warmup = args.warmup
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    # measured HBM copy bandwidth (1 GiB read + 1 GiB write), beside the
    # nominal peak; with --copy-calibration this is also the known-size
    # kernel the byte counters are scaled by
    ca = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).fill_(1.0)
    cb = torch.empty_like(ca)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    copies = 1 if args.copy_calibration else 5
    e0.record()
    for _ in range(copies):
        cb.copy_(ca)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2.0 * (1 << 30) * copies / (e0.elapsed_time(e1) * 1e6)
    del ca, cb
    log(f"[bench] {wl.name}: generating inputs on {dev}")
    inp = workloads.make_inputs(wl, dev)
    n_x = wl.calls
    xs = [inp["x"]] + [workloads.make_x(wl, dev, c) for c in range(1, n_x)]
    weights = moe.Weights.from_dict(inp)
    layer = moe.MoeLayer(weights, wl.k, wl.capacity_factor, wl.alpha,
                         routing=wl.routing, activation=wl.activation)
    stream = torch.cuda.current_stream(dev)
    m = time_layer(wl, layer, weights, xs, steps, warmup, stream)
    desc = m["desc"]
    total_ms, wall = m["total_ms"], m["wall"]
    up_avg_ms = m["up_avg_ms"]
    ms_per_step = m["ms_per_step"]
    counts, kept = m["counts"], m["kept"]
    alg = algorithmic(wl, counts, kept)
    tokens_per_s = wl.T * steps / (total_ms / 1e3)
    flops_peak = MFMA_BF16_PEAK_TFLOPS if wl.dtype == "bf16" \
        else MFMA_F32_PEAK_TFLOPS
    gbs = alg["up_bytes"] / (up_avg_ms * 1e6)
    tflops = alg["up_flops"] / (up_avg_ms * 1e9)
    if roofline_bound(alg, flops_peak) == "hbm":
        roof = dict(bound="hbm", achieved=gbs, peak=HBM_PEAK_GBS, unit="GB/s")
    else:
        roof = dict(bound="mfma", achieved=tflops, peak=flops_peak,
                    unit="TFLOP/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    # the same launch against both peaks
    roof["hbm_frac"] = gbs / HBM_PEAK_GBS
    roof["mfma_frac"] = tflops / flops_peak
    if wl.dtype == "bf16" and float(np.sum(kept)) / wl.E > 48:
        # the vendor library's dense bf16 GEMM of the same FLOPs as the up
        # GEMM (rows x d_ff x d), measured here beside the nominal peak
        roof["measured_dense_gemm_tflops"] = dense_gemm_tflops(
            alg["rows"], wl.d_ff * (2 if wl.activation == "swiglu" else 1),
            wl.d, dev)
    roof["algorithmic_bytes"] = alg["up_bytes"]
    roof["traffic"] = recorded_traffic(wl.name)
    roof["kernel"] = "grouped GEMM up (moe_ffn_up)"
    # the library's kernel variant ids of the up and down GEMMs
    roof["gemm_variants"] = [moe.moe_gemm_variant(desc, True),
                             moe.moe_gemm_variant(desc, False)]
    roof["kernel_ms"] = up_avg_ms

    decode = None
    if wl.name == "mixtral_prefill" and not args.no_decode:
        # the metric's second half: the decode-shaped layer's HBM fraction,
        # on the same weights, in the same process
        decode = decode_leg(weights, dev, stream)

    cpu = None
    if args.cpu_seconds > 0:
        log("[bench] timing the CPU oracle on a sample")
        cpu = cpu_baseline(wl, inp, args.cpu_seconds)

    out = {
        "metric": "MoE-layer fwd tokens/s",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "d": wl.d, "E": wl.E,
                   "k": wl.k, "d_ff": wl.d_ff, "n_shared": wl.n_shared,
                   "capacity_factor": wl.capacity_factor,
                   "routing": wl.routing,
                   "expert_weights": "e4m3" if wl.expert_fp8 else wl.dtype,
                   "activation": wl.activation,
                   "parallelism": "single-gpu"},
        "layer_tflops": alg["flops"] / (ms_per_step * 1e9),
        "layer_hbm_gbs": alg["bytes"] / (ms_per_step * 1e6),
        "wall_s": wall,
        "measured_hbm_copy_gbs": copy_gbs,
        "roofline": roof,
        "decode": decode,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
