"""Benchmark of the MoE routing + Q4 grouped-GEMM hot path on one MI355X.

Default (the prefill-chunk workload: T=512 tokens, E=256 experts, top-8,
K=2048 -> N=512, group-64 affine 4-bit weights): one step = the routing (top-k,
histogram, scan, block map, scatter) and the grouped GEMM over the routed rows,
as one moe_route_grouped_gemm_q4 call (its GEMM launch ranks each expert's rows
itself; at other shapes moe_route then moe_grouped_gemm_q4); the same JSON
line also carries, under "c3", the expert-FFN
step at T=4096 below (the metric is quoted at T=512 and T=4096), with its own
roofline and CPU baseline (--no-c3 leaves it out).  Other workloads:
  --workload 4   the same step at T=16384 with Zipf-skewed routing
  --workload 3   one step = moe_route + moe_expert_ffn_q4 (gate+up, SwiGLU,
                 down, weighted combine, shared expert) at T=4096, H=2048, I=512
  --workload 5   one step = one batch-1 decode step (moe_decode_ffn_q4:
                 routing, 8 of 256 experts + the shared expert) with fresh
                 logits and activations every step
Inputs are seeded synthetic arrays already resident in HBM when the timed
region starts.

Cold weights: consecutive steps use different resident copies of the layer's
weights (like consecutive MoE layers), so every step reads its weights from
HBM rather than from the 256 MB Infinity Cache: at least 1 GiB of copies for
the prefill workloads, and for decode enough copies that more than 256 MB of
other weights are read between two uses of a copy.

Steps are replayed from HIP graphs unless --no-graph: each graph holds a chain
of consecutive steps, each on its own weight copy (and, for decode, its own
fresh token), as consecutive layers run in one captured forward pass; an eager
run of the same steps gives the per-kernel event times.

Prints one JSON line: the throughput of the whole step, the roofline of the
dominant kernel (timed with HIP events on its launch stream; HBM traffic from
the committed rocprofv3 counter summary when it matches the kernel source)
and the CPU oracle timed on the host cores.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload 2|4|3|5|1]
                    [--block-rows BM] [--layers L] [--no-graph] [--no-cpu-baseline] [--cpu-reps R]
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
DATA = ("synthetic (seeded numpy PCG64; logits N(0,1){skew}, activations bf16 N(0,1), uniform 4-bit codes, "
        "bf16 scale |N(0,0.02)|, bias -8*scale + N(0,0.002))")


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


_CEILINGS = None


def measured_ceilings(torch, q) -> dict:
    """What this GPU sustains, measured here beside the published peaks: a 1 GiB
    device-to-device copy (HBM read + write) and the library's MFMA-only loop
    (independent 32x32x16 bf16 MFMAs on every SIMD)."""
    global _CEILINGS
    if _CEILINGS is not None:
        return _CEILINGS
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * (1 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    wgs, iters = 256 * 8, 2000
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    q.moe_calibrate_mfma(wgs, 10, out)
    torch.cuda.synchronize()
    e0.record()
    q.moe_calibrate_mfma(wgs, iters, out)
    e1.record()
    torch.cuda.synchronize()
    mfma_tflops = wgs * 4 * iters * 8 * 32768 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    _CEILINGS = {"hbm_copy_GBps": copy_gbps, "mfma_bf16_TFLOPs": mfma_tflops,
                 "how": "1 GiB device copy (read + write bytes / time, torch copy kernel); "
                        "moe_calibrate_mfma: 2048 workgroups x 4 waves of independent 32x32x16 bf16 MFMAs"}
    return _CEILINGS


def roofline(flops: float, alg_bytes: float, kernel_ms: float, kernel: str, workload: str) -> dict:
    gbps = alg_bytes / (kernel_ms * 1e-3) / 1e9
    tflops = flops / (kernel_ms * 1e-3) / 1e12
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    if flops / alg_bytes < ridge:
        roof = {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": gbps / HBM_PEAK_GBPS}
    else:
        roof = {"bound": "mfma", "achieved": tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": tflops / BF16_PEAK_TFLOPS}
    roof["traffic"] = load_traffic(kernel, workload)
    if _CEILINGS is not None:
        ceil = _CEILINGS["hbm_copy_GBps"] if roof["bound"] == "hbm" else _CEILINGS["mfma_bf16_TFLOPs"]
        roof["measured_ceiling"] = ceil
        roof["frac_of_measured_ceiling"] = roof["achieved"] / ceil
    roof["kernel"] = kernel
    roof["algorithmic_bytes_per_launch"] = alg_bytes
    roof["algorithmic_flops_per_launch"] = flops
    return roof


class Timer:
    """Times exactly `steps` calls of step(i, ev) back to back between two
    synchronisations; ev holds HIP events recorded on the launch stream."""

    def __init__(self, torch, nev):
        self.torch, self.nev = torch, nev

    def run(self, step, warmup, steps):
        torch = self.torch
        for i in range(warmup):
            step(i, None)
        torch.cuda.synchronize()
        ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(self.nev)) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(warmup + i, ev[i])
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
        seg = [np.array([e[j].elapsed_time(e[j + 1]) for e in ev]) for j in range(self.nev - 1)]
        return ms_per_step, seg


def graph_ms_per_step(torch, args, capture_step, layers):
    """Whole-step wall time with the steps replayed from HIP graphs captured
    from the same library calls: one graph runs a chain of `layers` consecutive
    steps (each on its own resident weight copy, as consecutive MoE layers of a
    model run back to back in one captured forward pass), and single-step
    graphs run the remainder, so exactly args.steps steps execute and their
    small kernels start back to back without host launch gaps."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # warm the calls once outside capture
        capture_step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    chain = torch.cuda.CUDAGraph()
    with torch.cuda.graph(chain):
        for l in range(layers):
            capture_step(l)
    singles = []
    for l in range(layers):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            capture_step(l)
        singles.append(g)
    for i in range(max(1, args.warmup // layers)):
        chain.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps // layers):
        chain.replay()
    for l in range(args.steps % layers):
        singles[l].replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / args.steps


def graph_split_ms(torch, pre, call, layers, reps, rounds=3, whole=None):
    """Time of `call` inside the step it belongs to: HIP graphs hold a chain of
    `layers` steps (pre(l) then call(l), or whole(l): one call that does pre's
    work and then the call's, each on its own resident weight copy) and the
    same chain of pre(l) alone; both are replayed `reps` times back to back
    between two HIP events on the launch stream, alternating over `rounds`
    rounds, and the call's time per step is the difference of the two
    per-step times.  A back-to-back chain of the call alone would time it in
    another context than the step's (at the prefill shapes the GEMMs then run
    several percent slower).  Returns (step ms, pre ms, call ms)."""
    def step(l):
        if whole is not None:
            whole(l)
        else:
            pre(l)
            call(l)

    s = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(s)
    with torch.cuda.stream(side):       # warm the calls once outside capture
        pre(0)
        step(0)
    s.wait_stream(side)
    torch.cuda.synchronize()
    g_step, g_pre = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_step):
        for l in range(layers):
            step(l)
    with torch.cuda.graph(g_pre):
        for l in range(layers):
            pre(l)
    g_step.replay()
    g_pre.replay()
    torch.cuda.synchronize()
    tot = {"step": 0.0, "pre": 0.0}
    for _ in range(rounds):
        for name, g in (("step", g_step), ("pre", g_pre)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for _ in range(reps):
                g.replay()
            e1.record(s)
            torch.cuda.synchronize()
            tot[name] += e0.elapsed_time(e1)
    n = rounds * reps * layers
    step_ms, pre_ms = tot["step"] / n, tot["pre"] / n
    return step_ms, pre_ms, step_ms - pre_ms


def decode_graph_ms_per_step(torch, args, capture_step, layers):
    """Decode steps replayed from HIP graphs: steps warmup .. warmup+steps-1 in
    chains of `layers` consecutive steps, each captured with its own inputs and
    weight copy (a decode pass through consecutive layers in one graph).
    capture_step(i) launches step i on torch's current stream.  Returns
    (wall-clock ms per step, HIP-event ms per step) over the replays."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        capture_step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    chains = []
    for c0 in range(args.warmup, args.warmup + args.steps, layers):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(c0, min(c0 + layers, args.warmup + args.steps)):
                capture_step(i)
        chains.append(g)
    chains[0].replay()                   # warm the graph path once
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(s)
    for g in chains:
        g.replay()
    e1.record(s)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / args.steps
    return wall, e0.elapsed_time(e1) / args.steps


def base_line(args, w, value, ms_per_step, config, roof):
    return {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": DATA.format(skew=f" + Zipf expert bias, alpha {w.skew_alpha}" if w.skew_alpha else ""),
        "config": config, "roofline": roof,
    }


# ------------------------------------------------------------ single projection
def bench_gemm(args, torch, q, W, w, d):
    p = W.make_problem(w)
    T, E, k, K, N = w.T, w.E, w.k, w.K, w.N
    w_layer = E * q4_bytes(N, K)
    layers = args.layers or max(2, -(-(1 << 30) // w_layer))
    packed0 = q.prepack(d(p.Wq), d(p.S), d(p.B))     # one-time re-tiling at load time
    packs = [packed0] + [tuple(t.clone() for t in packed0) for _ in range(layers - 1)]
    logits, X = d(p.logits), d(p.X)
    rt = q.alloc_route(T, E, k, args.block_rows, device=X.device)
    Y = torch.empty((T * k, N), dtype=torch.int16, device=X.device)
    stream = torch.cuda.current_stream()
    # 64-row blocks up to MOEQ4_ROUTE_IN_LAUNCH_MAX assignments: one call, whose
    # GEMM launch ranks each expert's rows itself after the top-k
    # (moe_route_grouped_gemm_q4); the routing that precedes the GEMM launch is
    # then the top-k alone
    fused = rt["block_rows"] == 64 and 0 < T * k <= q.MOEQ4_ROUTE_IN_LAUNCH_MAX
    cur = torch.cuda.current_stream

    def pre(l, st=None):
        if fused:
            q.topk_softmax(logits, k, rt, stream=st or cur())
        else:
            q.route(logits, k, bufs=rt, stream=st or cur())

    def whole(l, st=None):
        if fused:
            q.route_grouped_gemm_q4(logits, X, k, packs[l], rt, Y=Y, stream=st or cur())
        else:
            q.route(logits, k, bufs=rt, stream=st or cur())
            q.grouped_gemm_q4(X, k, packs[l], rt, Y=Y, stream=st or cur())

    def step(i, ev):
        if ev is not None:
            ev[0].record(stream)
        whole(i % layers, stream)
        if ev is not None:
            ev[1].record(stream)

    def pre_step(i, ev):
        if ev is not None:
            ev[0].record(stream)
        pre(i, stream)
        if ev is not None:
            ev[1].record(stream)

    # eager: the steps between HIP events, then (separately) the routing that
    # precedes the GEMM launch on its own
    eager_ms, (whole_all,) = Timer(torch, 2).run(step, args.warmup, args.steps)
    _, (route_all,) = Timer(torch, 2).run(pre_step, 2, min(args.steps, 20))
    gemm_all = whole_all - float(route_all.mean())
    gemm_ms = float(gemm_all.mean())
    gemm_eager_ms = gemm_ms
    ms_per_step = eager_ms
    if not args.no_graph:
        ms_per_step = graph_ms_per_step(torch, args, whole, layers)
        split_step_ms, split_pre_ms, gemm_ms = graph_split_ms(torch, pre, None, layers, max(1, args.steps // layers),
                                                              whole=whole)
    counts = rt["counts"].cpu().numpy()
    touched = int((counts > 0).sum())
    A = T * k
    flops = 2.0 * A * N * K
    w_bytes = touched * q4_bytes(N, K)
    alg_bytes = w_bytes + T * K * 2 + A * N * 2
    out = base_line(args, w, flops / (ms_per_step * 1e-3) / 1e12, ms_per_step,
                    {"workload": w.name, "T": T, "E": E, "top_k": k, "K": K, "N": N,
                     "block_rows": rt["block_rows"], "group": 64, "parallelism": "single GPU"},
                    roofline(flops, alg_bytes, gemm_ms, "k_gemm_q4", w.name))
    out["roofline"]["kernel_detail"] = (
        "the GEMM launch that also ranks each expert's rows (moe_route_grouped_gemm_q4)" if fused
        else "the grouped GEMM launch after moe_route")
    out.update({
        "weight_GBps_step": w_bytes / (ms_per_step * 1e-3) / 1e9,
        "gemm": {"us": gemm_ms * 1e3, "eager_event_us": gemm_eager_ms * 1e3, "TFLOP/s": flops / (gemm_ms * 1e-3) / 1e12,
                 "split_step_us": None if args.no_graph else split_step_ms * 1e3,
                 "split_pre_us": None if args.no_graph else split_pre_ms * 1e3,
                 "weight_GB/s": w_bytes / (gemm_ms * 1e-3) / 1e9, "experts_touched": touched,
                 "rows_max_over_mean": float(counts.max() / counts.mean()),
                 "experts_below_2_rows": float((counts < 2).mean())},
        "route_us": float(route_all.mean()) * 1e3,
        "eager_ms_per_step": eager_ms,
        "step_call": ("moe_route_grouped_gemm_q4 (top-k launch, then one GEMM launch that ranks each expert's "
                      "rows itself)" if fused else "moe_route then moe_grouped_gemm_q4"),
        "timing": f"steps back to back" +
                  ("" if args.no_graph else f", replayed from HIP graphs each holding a chain of {layers} steps "
                   "(the step's launches, one weight copy each), wall clock between two synchronisations") +
                  f"; weights rotate over {layers} resident copies ({layers * w_layer / 2**30:.2f} GiB) so each "
                  "GEMM reads them from HBM; GEMM time (gemm.us, the roofline's) by HIP events around graph replays: "
                  "a chain of steps minus the same chain of the routing that precedes the GEMM launch ("
                  + ("moe_topk_softmax" if fused else "moe_route") + "), per step" +
                  (" (eager: the step and the routing alone by HIP events)" if
                  args.no_graph else "; route_us and gemm.eager_event_us by HIP events in eager runs (the "
                   "step, then the routing alone)"),
        "gemm_us_p10_p90": [float(np.percentile(gemm_all, 10)) * 1e3, float(np.percentile(gemm_all, 90)) * 1e3],
    })
    if not args.no_cpu_baseline:
        import oracle
        t = []
        while len(t) < args.cpu_reps and (not t or sum(t) < args.cpu_seconds):
            t0 = time.perf_counter()
            ids, _ = oracle.topk_softmax(p.logits, k)
            r = oracle.route(ids, E, rt["block_rows"])
            oracle.grouped_gemm_q4(p.X, k, p.Wq, p.S, p.B, r["perm"], r["offsets"])
            t.append(time.perf_counter() - t0)
            print(f"cpu baseline: run {len(t)} took {t[-1]:.2f} s", file=sys.stderr, flush=True)
        ts = float(np.median(t))
        out["cpu_baseline"] = {"value": flops / ts / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
                               "kind": "oracle",
                               "sample": f"the whole step (route + grouped GEMM) of the same workload, median of "
                                         f"{len(t)} runs, {ts:.2f} s each"}
    return out


def ffn_flops(T, H, I, k, shared):
    """gate+up (2I x H) and down (H x I) per routed row, plus the shared expert per token."""
    per_row = 2.0 * (2 * I * H + H * I)
    return per_row * T * k + (per_row * T if shared else 0.0)


def pack_ffn(q, d, p):
    return (q.prepack(d(p.gu_q), d(p.gu_s), d(p.gu_b)), q.prepack(d(p.dn_q), d(p.dn_s), d(p.dn_b)),
            q.prepack(d(p.sh_gu_q), d(p.sh_gu_s), d(p.sh_gu_b)), q.prepack(d(p.sh_dn_q), d(p.sh_dn_s), d(p.sh_dn_b)))


def clone_pack(pk):
    return tuple(tuple(t.clone() for t in m) for m in pk)


# ----------------------------------------------------------------- expert FFN
def bench_ffn(args, torch, q, W, w, d):
    p = W.make_problem(w)
    T, E, k, H, I = w.T, w.E, w.k, w.K, w.N
    expert_bytes = q4_bytes(2 * I, H) + q4_bytes(H, I)
    w_layer = (E + 1) * expert_bytes
    layers = args.layers or max(2, -(-(1 << 30) // w_layer))
    pk0 = pack_ffn(q, d, p)
    packs = [pk0] + [clone_pack(pk0) for _ in range(layers - 1)]
    logits, X = d(p.logits), d(p.X)
    rt = q.alloc_route(T, E, k, args.block_rows, device=X.device)
    bufs = q.alloc_ffn(T, H, I, E, k, True, device=X.device)
    stream = torch.cuda.current_stream()
    chunked = None
    if args.chunk:  # the same step as a sequence of bounded chunks (moe_prefill_ffn_chunked_q4)
        chunked = q.alloc_chunked(T, args.chunk, H, I, E, k, args.block_rows, True, device=X.device)

    def step(i, ev):
        if ev is not None:
            ev[0].record(stream)
        if chunked is not None:
            if ev is not None:
                ev[1].record(stream)
            q.prefill_ffn_chunked(logits, X, k, *packs[i % layers], bufs=chunked, stream=stream)
        else:
            q.route(logits, k, bufs=rt, stream=stream)
            if ev is not None:
                ev[1].record(stream)
            q.expert_ffn(X, k, rt, *packs[i % layers], bufs=bufs, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    def graph_step(l):
        s = torch.cuda.current_stream()
        if chunked is not None:
            q.prefill_ffn_chunked(logits, X, k, *packs[l], bufs=chunked, stream=s)
        else:
            q.route(logits, k, bufs=rt, stream=s)
            q.expert_ffn(X, k, rt, *packs[l], bufs=bufs, stream=s)

    eager_ms, (route_all, ffn_all) = Timer(torch, 3).run(step, args.warmup, args.steps)
    ffn_ms = float(ffn_all.mean())
    ffn_eager_ms = ffn_ms
    ms_per_step = eager_ms
    if not args.no_graph:
        ms_per_step = graph_ms_per_step(torch, args, graph_step, layers)
        if chunked is None:  # the FFN inside its step (a chunked call routes each chunk itself)
            _, _, ffn_ms = graph_split_ms(
                torch, lambda l: q.route(logits, k, bufs=rt, stream=torch.cuda.current_stream()),
                lambda l: q.expert_ffn(X, k, rt, *packs[l], bufs=bufs, stream=torch.cuda.current_stream()),
                layers, max(1, args.steps // layers))
    if chunked is not None:
        q.route(logits, k, bufs=rt, stream=stream)   # expert counts of the whole batch, for the byte count
    counts = rt["counts"].cpu().numpy()
    touched = int((counts > 0).sum())
    flops = ffn_flops(T, H, I, k, True)
    w_bytes = (touched + 1) * expert_bytes
    alg_bytes = w_bytes + T * H * 2 * 2   # weights, X once, out once
    out = base_line(args, w, flops / (ms_per_step * 1e-3) / 1e12, ms_per_step,
                    {"workload": w.name, "T": T, "E": E, "top_k": k, "H": H, "I": I, "shared_expert": True,
                     "block_rows": rt["block_rows"], "group": 64, "parallelism": "single GPU",
                     **({"chunk_tokens": args.chunk} if args.chunk else {})},
                    roofline(flops, alg_bytes, ffn_ms, "expert_ffn" + ("_chunked" if args.chunk else ""), w.name))
    out.update({
        "weight_GBps_step": w_bytes / (ms_per_step * 1e-3) / 1e9,
        "ffn": {"us": ffn_ms * 1e3, "eager_event_us": ffn_eager_ms * 1e3, "TFLOP/s": flops / (ffn_ms * 1e-3) / 1e12,
                "experts_touched": touched,
                "kernels": "routed + shared gate+up (SwiGLU) in one launch, routed (x routing weight) + "
                           "shared down in one launch, combine"},
        "route_us": float(route_all.mean()) * 1e3,
        "eager_ms_per_step": eager_ms,
        "scratch_bytes": (chunked["ws_bytes"] if chunked is not None else
                          rt["ws_bytes"] + bufs["ws_bytes"] + sum(rt[n].numel() * rt[n].element_size() for n in
                                                                 ("topk_ids", "topk_w", "counts", "offsets", "perm",
                                                                  "inv_perm", "blocks", "num_blocks"))),
        "timing": f"steps back to back, wall clock between two synchronisations" +
                  ("" if args.no_graph else f", replayed from HIP graphs each holding a chain of {layers} steps "
                   "(route + FFN launches, one weight copy each)") +
                  f"; weights rotate over {layers} resident copies ({layers * w_layer / 2**30:.2f} GiB); FFN time "
                  "(ffn.us, the roofline's) by HIP events around graph replays: a chain of route + FFN steps minus "
                  "the same chain of routing alone, per step"
                  + (" (eager or chunked: route and FFN split by HIP events)" if (args.no_graph or args.chunk) else
                     "; route_us and ffn.eager_event_us by HIP events in an eager run"),
    })
    if not args.no_cpu_baseline:
        import oracle
        sh = (p.sh_gu_q, p.sh_gu_s, p.sh_gu_b, p.sh_dn_q, p.sh_dn_s, p.sh_dn_b)
        t0 = time.perf_counter()
        ids, wts = oracle.topk_softmax(p.logits, k)
        oracle.expert_ffn_grouped_q4(p.X, ids, wts, p.gu_q, p.gu_s, p.gu_b, p.dn_q, p.dn_s, p.dn_b, sh=sh)
        ts = time.perf_counter() - t0
        print(f"cpu baseline (expert FFN): {ts:.2f} s", file=sys.stderr, flush=True)
        out["cpu_baseline"] = {"value": flops / ts / 1e12, "unit": "TFLOP/s",
                               "cores": oracle.num_threads(), "kind": "oracle",
                               "sample": f"the whole step of the same workload (top-k + softmax, then every "
                                         f"token's FFN expert by expert, shared expert included), one run, "
                                         f"{ts:.2f} s"}
    return out


# ------------------------------------------------------------- few-row groups
def bench_crossover(args, torch, q, W, d):
    """Groups of T = 1..8 rows at the decode shapes (top-8 of 256 + shared
    expert, H=2048, I=512), fresh rows every step, as a speculative
    verification step hands the layer: the few-token path
    (moe_small_batch_ffn_q4), the prefill path (moe_route + moe_expert_ffn_q4)
    and, at T=1, the decode step.  Microseconds per step from HIP graph replays;
    weights rotate over resident copies as in the decode benchmark."""
    w = W.WORKLOADS[5]
    p = W.make_problem(w)
    E, k, H, I = w.E, w.k, w.K, w.N
    expert_bytes = q4_bytes(2 * I, H) + q4_bytes(H, I)
    layers = args.layers or max(2, -(-(384 << 20) // ((k + 1) * expert_bytes)))
    pk0 = pack_ffn(q, d, p)
    packs = [pk0] + [clone_pack(pk0) for _ in range(layers - 1)]
    nst = args.warmup + args.steps
    rows = []
    sizes = [int(v) for v in args.crossover_rows.split(",")] if args.crossover_rows else \
        list(range(1, q.MOEQ4_SMALL_MAX_T + 1))
    for T in sizes:
        lg = d(np.stack([W.gen_logits(w.cid, T, E, 1000 * T + s) for s in range(nst)]))
        xs = d(np.stack([W.gen_acts(w.cid, T, H, 1000 * T + s) for s in range(nst)]))
        sb = q.alloc_small(T, E, k, H, I, True, device=xs.device)
        rt = q.alloc_route(T, E, k, 0, device=xs.device)
        fb = q.alloc_ffn(T, H, I, E, k, True, device=xs.device)

        def small_step(i):
            q.small_batch_ffn(lg[i], xs[i], k, *packs[i % layers], bufs=sb, stream=torch.cuda.current_stream())

        def prefill_step(i):
            s = torch.cuda.current_stream()
            q.route(lg[i], k, bufs=rt, stream=s)
            q.expert_ffn(xs[i], k, rt, *packs[i % layers], bufs=fb, stream=s)

        # distinct experts per step, from the few-token path's own routing output
        distinct = []
        for i in range(min(nst, 32)):
            small_step(i)
            distinct.append(len(np.unique(sb["topk_ids"].cpu().numpy())))
        u = float(np.mean(distinct))
        row = {"T": T, "distinct_experts_mean": u}
        row["small_us"] = decode_graph_ms_per_step(torch, args, small_step, layers)[0] * 1e3
        row["prefill_path_us"] = decode_graph_ms_per_step(torch, args, prefill_step, layers)[0] * 1e3
        if T == 1:
            db = q.alloc_decode(E, k, H, I, True, device=xs.device)
            row["decode_us"] = decode_graph_ms_per_step(
                torch, args, lambda i: q.decode_ffn(lg[i][0], xs[i][0], k, *packs[i % layers], bufs=db,
                                                    stream=torch.cuda.current_stream()), layers)[0] * 1e3
        row["small_weight_GBps"] = (u + 1) * expert_bytes / (row["small_us"] * 1e-6) / 1e9
        row["small_us_per_row"] = row["small_us"] / T
        rows.append(row)
        print(f"# T={T}: few-token {row['small_us']:.1f} us, prefill path {row['prefill_path_us']:.1f} us",
              file=sys.stderr, flush=True)
    return {"metric": "few-row MoE layer (groups of T rows at the decode shapes): us per step", "unit": "us",
            "higher_is_better": False, "data": "synthetic", "dtype": "bf16",
            "config": {"workload": "few-row groups T=1..8 E=256 k=8 H=2048 I=512 + shared",
                       "steps_per_T": args.steps, "weight_copies": layers},
            "rows": rows,
            "timing": "steps back to back from HIP graphs of consecutive steps, each with fresh rows and its own "
                      "weight copy; wall clock between two synchronisations"}


# ------------------------------------------------------------------ ablations
def unfused_layout(counts, offsets, perm, k, T):
    """Row sources of the unfused arm's batched GEMM: per expert, its routed
    tokens (perm order) padded with row T (a zero row) to a common multiple of 16."""
    E = len(counts)
    mmax = int(counts.max()) if E else 0
    mpad = max(16, -(-mmax // 16) * 16)
    src_row = np.full((E, mpad), T, np.int64)
    for e in range(E):
        c = int(counts[e])
        src_row[e, :c] = perm[offsets[e]: offsets[e] + c] // k
    return src_row


def unfused_gemm(torch, Wbf, Xz, src_row):
    """The unfused arm's GEMM: every expert's rebuilt bf16 weights [E, N, K]
    (from moe_dequant_q4) times its gathered rows, one vendor batched GEMM
    (torch.bmm -> hipBLASLt) with the right operand contiguous.  [E, N, mpad] bf16."""
    xt = Xz[src_row].transpose(1, 2).contiguous()            # [E, K, mpad]
    return torch.bmm(Wbf.view(torch.bfloat16), xt)


def host_block_map(counts, bm):
    """The host-synced arm's block map, built on the CPU from the expert counts
    copied back from the GPU: int32 [nb * 4] entries {expert, first sorted row,
    rows, block index} and nb."""
    cnt = np.asarray(counts, np.int64)
    E = len(cnt)
    nbe = (cnt + bm - 1) // bm
    offs = np.concatenate([[0], np.cumsum(cnt)])
    e_of = np.repeat(np.arange(E), nbe)
    j = np.arange(int(nbe.sum())) - np.repeat(np.cumsum(nbe) - nbe, nbe)
    blk = np.stack([e_of, offs[e_of] + j * bm, np.minimum(bm, cnt[e_of] - j * bm), j], 1)
    return blk.astype(np.int32).reshape(-1), int(nbe.sum())


def bench_ablation(args, torch, q, W, T, d):
    """The pages' two prefill mechanisms, each against its unfused alternative,
    on the single-projection shape (E=256, k=8, K=2048, N=512) at T tokens:
      fused     moe_route + moe_grouped_gemm_q4 (the product path as two calls; every arm
                routes with the same moe_route call);
      unfused   moe_route + moe_dequant_q4 (every weight rebuilt as bf16 into
                HBM) + a bf16 grouped GEMM on the expanded weights: the vendor
                batched GEMM (torch.bmm -> hipBLASLt) over per-expert padded
                rows, gathered through perm; its HBM floor is printed beside it;
      hostsync  moe_route, then the expert counts copied to the host, the block
                map built there and copied back before moe_grouped_gemm_q4
                (the CPU round trip the GPU-resident routing removes).
    Every variant runs the same seeded inputs and a fresh weight copy per step."""
    w = W.custom(2, T, 256, 8, 2048, 512)
    p = W.make_problem(w)
    E, k, K, N = w.E, w.k, w.K, w.N
    w_layer = E * q4_bytes(N, K)
    layers = args.layers or max(2, -(-(1 << 30) // w_layer))
    packed0 = q.prepack(d(p.Wq), d(p.S), d(p.B))
    packs = [packed0] + [tuple(t.clone() for t in packed0) for _ in range(layers - 1)]
    logits, X = d(p.logits), d(p.X)
    rt = q.alloc_route(T, E, k, args.block_rows, device=X.device)
    Y = torch.empty((T * k, N), dtype=torch.int16, device=X.device)
    stream = torch.cuda.current_stream()
    # the routing is the same every step (same logits): the padded layout of the
    # unfused GEMM is taken from it once, outside the timed region
    q.route(logits, k, bufs=rt, stream=stream)
    torch.cuda.synchronize()
    counts = rt["counts"].cpu().numpy()
    offsets = rt["offsets"].cpu().numpy()
    perm = rt["perm"].cpu().numpy()
    mmax = int(counts.max())
    src_row = torch.from_numpy(unfused_layout(counts, offsets, perm, k, T)).to(X.device)   # row T of Xz is zeros
    Xz = torch.cat([X.view(torch.bfloat16), torch.zeros((1, K), dtype=torch.bfloat16, device=X.device)])
    Wbf = torch.empty((E, N, K), dtype=torch.int16, device=X.device)
    blocks_host = torch.empty(rt["blocks"].numel(), dtype=torch.int32).pin_memory()
    nb_host = torch.empty(4, dtype=torch.int32).pin_memory()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(step_fn, n):
        for i in range(args.warmup):
            step_fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            step_fn(args.warmup + i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n

    def fused(i):
        q.route(logits, k, bufs=rt, stream=stream)
        q.grouped_gemm_q4(X, k, packs[i % layers], rt, Y=Y, stream=stream)

    def unfused(i):
        q.route(logits, k, bufs=rt, stream=stream)
        q.dequant(packs[i % layers], E, N, K, out=Wbf, stream=stream)
        unfused_gemm(torch, Wbf, Xz, src_row)

    def hostsync(i):
        q.route(logits, k, bufs=rt, stream=stream)
        cnt = rt["counts"].cpu().numpy()                        # the CPU wait
        blk, nb = host_block_map(cnt, rt["block_rows"])
        blocks_host[: blk.size] = torch.from_numpy(blk)
        nb_host[0] = nb
        rt["blocks"][: blk.size].copy_(blocks_host[: blk.size], non_blocking=True)
        rt["num_blocks"][:1].copy_(nb_host[:1], non_blocking=True)
        q.grouped_gemm_q4(X, k, packs[i % layers], rt, Y=Y, stream=stream)

    steps = args.steps
    res = {"fused_us": timed(fused, steps) * 1e3, "unfused_us": timed(unfused, steps) * 1e3,
           "hostsync_us": timed(hostsync, steps) * 1e3}
    # kernel-level split of the unfused path (events around the dequant and the GEMM)
    e3 = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    dq, gm = [], []
    for i in range(10):
        q.route(logits, k, bufs=rt, stream=stream)
        e3[0].record()
        q.dequant(packs[i % layers], E, N, K, out=Wbf, stream=stream)
        e3[1].record()
        unfused_gemm(torch, Wbf, Xz, src_row)
        e3[2].record()
        torch.cuda.synchronize()
        dq.append(e3[0].elapsed_time(e3[1]))
        gm.append(e3[0].elapsed_time(e3[2]) - e3[0].elapsed_time(e3[1]))
    bf16_bytes = E * N * K * 2
    res.update({
        "unfused_dequant_kernel_us": float(np.median(dq)) * 1e3,
        "unfused_gemm_us": float(np.median(gm)) * 1e3,
        "unfused_hbm_floor_us": (w_layer + 2 * bf16_bytes) / 5.1e12 * 1e6,
        "speedup_fused_vs_unfused": res["unfused_us"] / res["fused_us"],
        "speedup_gpu_routing_vs_hostsync": res["hostsync_us"] / res["fused_us"],
    })
    return {"ablation": "in-GEMM dequant and GPU-resident routing vs their unfused alternatives", "T": T,
            "config": {"workload": w.name, "E": E, "top_k": k, "K": K, "N": N, "block_rows": rt["block_rows"],
                       "rows_per_expert_max": mmax},
            "steps": steps, "warmup": args.warmup, "weight_copies": layers, "results_us": res,
            "notes": "unfused GEMM = torch.bmm (hipBLASLt) over per-expert rows padded to a multiple of 16, "
                     "activations gathered through perm; unfused_hbm_floor_us = (q4 read + bf16 write + bf16 read) "
                     "at 5.1 TB/s (the measured copy rate); hostsync = D2H of the counts (synchronizing), block map "
                     "on the host, H2D of the map, then the same grouped GEMM"}


# --------------------------------------------------------------------- decode
def bench_decode(args, torch, q, W, w, d):
    p = W.make_problem(w)
    E, k, H, I = w.E, w.k, w.K, w.N
    expert_bytes = q4_bytes(2 * I, H) + q4_bytes(H, I)
    step_bytes = (k + 1) * expert_bytes
    # a copy's weights are read again only after > 256 MB of other weights
    layers = args.layers or max(2, -(-(384 << 20) // step_bytes))
    pk0 = pack_ffn(q, d, p)
    packs = [pk0] + [clone_pack(pk0) for _ in range(layers - 1)]
    steps_total = args.warmup + args.steps
    lg = d(np.stack([W.gen_logits(w.cid, 1, E, s)[0] for s in range(steps_total)]))
    xs = d(np.stack([W.gen_acts(w.cid, 1, H, s)[0] for s in range(steps_total)]))
    bufs = q.alloc_decode(E, k, H, I, True, device=xs.device)
    stream = torch.cuda.current_stream()

    def step(i, ev):
        if ev is not None:
            ev[0].record(stream)
        gu, dn, sg, sd = packs[i % layers]
        q.decode_ffn(lg[i], xs[i], k, gu, dn, sg, sd, bufs=bufs, stream=stream)
        if ev is not None:
            ev[1].record(stream)

    eager_ms, (dec_all,) = Timer(torch, 2).run(step, args.warmup, args.steps)
    dec_ms = dec_eager_ms = float(dec_all.mean())
    ms_per_step = eager_ms
    if not args.no_graph:
        ms_per_step, dec_ms = decode_graph_ms_per_step(
            torch, args, lambda i: q.decode_ffn(lg[i], xs[i], k, *packs[i % layers], bufs=bufs,
                                                stream=torch.cuda.current_stream()), layers)
    flops = ffn_flops(1, H, I, k, True)
    alg_bytes = step_bytes + H * 2 * 2 + E * 4
    out = base_line(args, w, flops / (ms_per_step * 1e-3) / 1e12, ms_per_step,
                    {"workload": w.name, "T": 1, "E": E, "top_k": k, "H": H, "I": I, "shared_expert": True,
                     "steps_of_fresh_tokens": args.steps, "group": 64, "parallelism": "single GPU"},
                    roofline(flops, alg_bytes, dec_ms, "decode_step", w.name))
    out.update({
        "weight_GBps_step": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "decode": {"us_per_step_kernels": dec_ms * 1e3, "eager_event_us": dec_eager_ms * 1e3,
                   "weight_GB/s": step_bytes / (dec_ms * 1e-3) / 1e9,
                   "weight_bytes_per_step": step_bytes,
                   "kernels": "k_decode_gateup (routing + gate/up + SwiGLU), k_decode_down (down + combine)"},
        "timing": f"steps back to back, wall clock between two synchronisations" +
                  ("" if args.no_graph else f", replayed from HIP graphs each holding {layers} consecutive steps "
                   "(every step its own fresh logits and activations and its own weight copy)") +
                  f"; weights rotate over {layers} resident copies so more than 256 MB "
                  "of other weights are read between two uses of a copy; kernel time (decode.us_per_step_kernels, "
                  "the roofline's) by HIP events around the graph replays" + (" (eager run)" if args.no_graph else
                  "; decode.eager_event_us by HIP events in an eager run"),
        "eager_ms_per_step": eager_ms,
        "p10_p90_us": [float(np.percentile(dec_all, 10)) * 1e3, float(np.percentile(dec_all, 90)) * 1e3],
    })
    if not args.no_cpu_baseline:
        import oracle
        sh = (p.sh_gu_q, p.sh_gu_s, p.sh_gu_b, p.sh_dn_q, p.sh_dn_s, p.sh_dn_b)
        n = 20
        inputs = [(W.gen_logits(w.cid, 1, E, s), W.gen_acts(w.cid, 1, H, s)) for s in range(n)]
        t0 = time.perf_counter()
        for lgs, xs1 in inputs:
            ids, wts = oracle.topk_softmax(lgs, k)
            oracle.expert_ffn_q4(xs1, ids, wts, p.gu_q, p.gu_s, p.gu_b, p.dn_q, p.dn_s, p.dn_b, sh=sh)
        ts = (time.perf_counter() - t0) / n
        out["cpu_baseline"] = {"value": flops / ts / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
                               "kind": "oracle",
                               "sample": f"the first {n} decode steps of the same workload (inputs generated "
                                         f"before the clock starts), {ts * 1e3:.1f} ms each"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 50; 1000 for decode)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--block-rows", type=int, default=0)
    ap.add_argument("--layers", type=int, default=0, help="resident weight copies used in turn (0: automatic)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of HIP graph replays")
    ap.add_argument("--ablation", type=int, default=0,
                    help="T: run the fused / unfused-dequant / host-synced-routing comparison at T tokens instead")
    ap.add_argument("--crossover", action="store_true",
                    help="time groups of 1..8 rows on the few-token, prefill and decode paths instead")
    ap.add_argument("--chunk", type=int, default=0,
                    help="expert-FFN workload: run the step as chunks of this many tokens (moe_prefill_ffn_chunked_q4)")
    ap.add_argument("--crossover-rows", default="", help="comma-separated T values for --crossover (default 1..8)")
    ap.add_argument("--no-c3", action="store_true",
                    help="default workload: leave out the expert-FFN step at T=4096 that rides in the same line")
    ap.add_argument("--c3-steps", type=int, default=20, help="timed steps of that expert-FFN step")
    ap.add_argument("--cpu-reps", type=int, default=40)
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="stop repeating the CPU oracle once this much time is spent (at least one run)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the path measured here is the "
                                   "single-GPU hot path", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import quantized_grouped_gemm_amd as q
    import workloads as W

    w = W.WORKLOADS[args.workload]
    if args.steps is None:
        args.steps = 1000 if (w.ffn and w.T == 1) else 50   # decode: the workload's 1000 fresh tokens
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def d(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    if args.ablation:
        print(json.dumps(bench_ablation(args, torch, q, W, args.ablation, d)), flush=True)
        return
    if args.crossover:
        print(json.dumps(bench_crossover(args, torch, q, W, d)), flush=True)
        return
    ceilings = measured_ceilings(torch, q)
    if w.ffn and w.T == 1:
        out = bench_decode(args, torch, q, W, w, d)
    elif w.ffn:
        out = bench_ffn(args, torch, q, W, w, d)
    else:
        out = bench_gemm(args, torch, q, W, w, d)
        if args.workload == 2 and not args.no_c3:
            # the metric is quoted at T=512 and T=4096: the expert-FFN step at
            # T=4096 rides in the same line, with its own roofline and baseline
            c3 = argparse.Namespace(**vars(args))
            c3.steps, c3.warmup, c3.block_rows, c3.chunk = args.c3_steps, min(args.warmup, 5), 0, 0
            r = bench_ffn(c3, torch, q, W, W.WORKLOADS[3], d)
            out["c3"] = {key: r[key] for key in ("value", "unit", "ms_per_step", "steps", "warmup", "config",
                                                "roofline", "ffn", "route_us", "cpu_baseline", "timing")
                         if key in r}
    out["measured_ceilings"] = ceilings
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
