"""Benchmark of the MoE routing + Q4 grouped-GEMM hot path on one MI355X.

One step = moe_route (top-k, histogram, scan, block map, scatter) followed by
moe_grouped_gemm_q4 over the routed rows, on the prefill-chunk workload
(T=512 tokens, E=256 experts, top-8, K=2048 -> N=512, group-64 affine 4-bit
weights).  Inputs are seeded synthetic arrays already resident in HBM when
the timed region starts.

Cold weights: consecutive steps use different resident copies of the layer's
weights (like consecutive MoE layers), at least 1 GiB in all, so every GEMM
reads its weights from HBM rather than from the 256 MB Infinity Cache.

Prints one JSON line with the throughput of the whole step, the roofline of
the grouped-GEMM kernel (timed with HIP events on its launch stream; HBM
traffic from the committed rocprofv3 counter summary when it matches the
kernel source) and the CPU oracle timed on the host cores.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload 2|4|1]
                    [--block-rows BM] [--layers L] [--no-cpu-baseline] [--cpu-reps R]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE q4 grouped-GEMM TFLOP/s + weight GB/s at T=512/4096; % of roofline"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published


def q4_bytes(N: int, K: int) -> int:
    """Packed codes + bf16 scale and bias per 64 weights."""
    return N * K // 2 + (N * K // 64) * 4


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel source (else None)."""
    from quantized_grouped_gemm_amd.profiling import kernel_source_hash
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
        ent = d[kernel][workload]
        if ent.get("source_hash") != kernel_source_hash():
            return None
        return ent["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(p, w, bm, reps):
    import oracle
    t_all = []
    for _ in range(reps):
        t0 = time.perf_counter()
        ids, _ = oracle.topk_softmax(p.logits, w.k)
        rt = oracle.route(ids, w.E, bm)
        oracle.grouped_gemm_q4(p.X, w.k, p.Wq, p.S, p.B, rt["perm"], rt["offsets"])
        t_all.append(time.perf_counter() - t0)
    t = float(np.median(t_all))
    flops = 2.0 * w.T * w.k * w.N * w.K
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"the whole step (route + grouped GEMM) of the same workload, median of {reps} runs, "
                      f"{t:.2f} s each"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--block-rows", type=int, default=0)
    ap.add_argument("--layers", type=int, default=0, help="resident weight copies used in turn (0: >= 1 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=40)
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the path is single-GPU "
                                   "(expert-parallel sharding is described in DESIGN.md)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import quantized_grouped_gemm_amd as q
    import workloads as W

    w = W.WORKLOADS[args.workload]
    assert not w.ffn, "bench.py times the single-projection workloads (1, 2, 4)"
    p = W.make_problem(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def d(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    T, E, k, K, N = w.T, w.E, w.k, w.K, w.N
    # Cold weights, as in a model: consecutive MoE layers each read their own
    # weights.  `layers` resident copies (>= 1 GiB in all, four times the
    # 256 MB Infinity Cache) are used in turn, so a step's weights were last
    # touched a whole rotation earlier and come from HBM.
    w_layer = E * q4_bytes(N, K)
    layers = args.layers or max(2, -(-(1 << 30) // w_layer))
    packed0 = q.prepack(d(p.Wq), d(p.S), d(p.B))     # one-time re-tiling at load time
    packs = [packed0] + [tuple(t.clone() for t in packed0) for _ in range(layers - 1)]
    logits, X = d(p.logits), d(p.X)
    rt = q.alloc_route(T, E, k, args.block_rows, device=dev)
    Y = torch.empty((T * k, N), dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        q.route(logits, k, bufs=rt, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        q.grouped_gemm_q4(X, k, packs[i % layers], rt, Y=Y, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed: exactly `steps` steps back to back between two synchronisations;
    # HIP events on the launch stream split each step into route and GEMM
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, ev[i])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ev_step_ms = float(np.mean([a.elapsed_time(c) for a, b, c in ev]))
    route_ms = float(np.mean([a.elapsed_time(b) for a, b, c in ev]))
    gemm_all = np.array([b.elapsed_time(c) for a, b, c in ev])
    gemm_ms = float(gemm_all.mean())

    counts = rt["counts"].cpu().numpy()
    touched = int((counts > 0).sum())
    A = T * k
    flops = 2.0 * A * N * K
    w_bytes = touched * q4_bytes(N, K)
    alg_bytes = w_bytes + T * K * 2 + A * N * 2
    achieved_gbps = alg_bytes / (gemm_ms * 1e-3) / 1e9
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    hbm_bound = flops / alg_bytes < ridge
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": achieved_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved_gbps / HBM_PEAK_GBPS}
    else:
        roof = {"bound": "mfma", "achieved": gemm_tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": gemm_tflops / BF16_PEAK_TFLOPS}
    roof["traffic"] = load_traffic("k_gemm_q4", w.name)
    roof["kernel"] = "k_gemm_q4"
    roof["algorithmic_bytes_per_launch"] = alg_bytes
    roof["algorithmic_flops_per_launch"] = flops

    out = {
        "metric": METRIC,
        "value": flops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded numpy PCG64; logits N(0,1)" + (f" + Zipf expert bias, alpha {w.skew_alpha}"
                if w.skew_alpha else "") + ", activations bf16 N(0,1), uniform 4-bit codes, bf16 scale "
                "|N(0,0.02)|, bias -8*scale + N(0,0.002))",
        "config": {"workload": w.name, "T": T, "E": E, "top_k": k, "K": K, "N": N,
                   "block_rows": rt["block_rows"], "group": 64, "parallelism": "single GPU"},
        "weight_GBps_step": w_bytes / (ms_per_step * 1e-3) / 1e9,
        "gemm": {"us": gemm_ms * 1e3, "TFLOP/s": gemm_tflops, "weight_GB/s": w_bytes / (gemm_ms * 1e-3) / 1e9,
                 "experts_touched": touched, "rows_max_over_mean": float(counts.max() / counts.mean()),
                 "experts_below_2_rows": float((counts < 2).mean())},
        "route_us": route_ms * 1e3,
        "event_ms_per_step": ev_step_ms,
        "timing": f"steps back to back, wall clock between two synchronisations; weights rotate over {layers} "
                  f"resident copies ({layers * w_layer / 2**30:.2f} GiB) so each GEMM reads them from HBM; "
                  "route and GEMM split by HIP events on the launch stream",
        "gemm_us_p10_p90": [float(np.percentile(gemm_all, 10)) * 1e3, float(np.percentile(gemm_all, 90)) * 1e3],
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p, w, rt["block_rows"], args.cpu_reps)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
