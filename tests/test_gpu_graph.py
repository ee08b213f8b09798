"""The library's launches captured in a HIP graph: each replay, with fresh
inputs written into the captured buffers between replays (eager work between
them), must equal the eager result bit for bit.  The calls enqueue kernels
only (no host synchronisation, allocation or memset), so they can be captured."""
import numpy as np
import pytest

import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts only to be skipped
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_util import dev, host  # noqa: E402
import quantized_grouped_gemm_amd as q  # noqa: E402


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def _check_replays(g, set_inputs, run_eager, outputs, reps=3):
    """outputs: functions returning host copies of what must match (only the
    defined part of each output: block-map entries past num_blocks are unspecified)."""
    for r in range(reps):
        set_inputs(r)
        g.replay()
        torch.cuda.synchronize()
        got = [f() for f in outputs]
        run_eager()
        torch.cuda.synchronize()
        for a, f in zip(got, outputs):
            np.testing.assert_array_equal(a, f())


def test_graph_route_and_grouped_gemm():
    w = W.custom(80, 200, 16, 4, 256, 128)
    p = W.make_problem(w)
    logits, X = dev(p.logits), dev(p.X)
    packed = q.prepack(dev(p.Wq), dev(p.S), dev(p.B))
    rt = q.alloc_route(w.T, w.E, w.k, 32)
    Y = torch.empty((w.T * w.k, w.N), dtype=torch.int16, device="cuda")

    def run():
        s = torch.cuda.current_stream()
        q.route(logits, w.k, bufs=rt, stream=s)
        q.grouped_gemm_q4(X, w.k, packed, rt, Y=Y, stream=s)

    def set_inputs(r):
        logits.copy_(dev(W.gen_logits(80, w.T, w.E, step=r + 1)))
        X.copy_(dev(W.gen_acts(80, w.T, w.K, step=r + 1)))

    g = _capture(run)
    def blocks():
        nb = int(host(rt["num_blocks"])[0])
        return host(rt["blocks"])[: 4 * nb].copy()

    _check_replays(g, set_inputs, run, [lambda: host(Y).copy(), lambda: host(rt["perm"]).copy(), blocks,
                                        lambda: host(rt["topk_ids"]).copy(), lambda: host(rt["num_blocks"])[:1].copy()])


def test_graph_route_and_expert_ffn():
    w = W.custom(81, 120, 16, 2, 256, 128, ffn=True)
    p = W.make_problem(w)
    logits, X = dev(p.logits), dev(p.X)
    gu = q.prepack(dev(p.gu_q), dev(p.gu_s), dev(p.gu_b))
    dn = q.prepack(dev(p.dn_q), dev(p.dn_s), dev(p.dn_b))
    sg = q.prepack(dev(p.sh_gu_q), dev(p.sh_gu_s), dev(p.sh_gu_b))
    sd = q.prepack(dev(p.sh_dn_q), dev(p.sh_dn_s), dev(p.sh_dn_b))
    rt = q.alloc_route(w.T, w.E, w.k, 16)
    bufs = q.alloc_ffn(w.T, w.K, w.N, w.E, w.k, True)

    def run():
        s = torch.cuda.current_stream()
        q.route(logits, w.k, bufs=rt, stream=s)
        q.expert_ffn(X, w.k, rt, gu, dn, sg, sd, bufs=bufs, stream=s)

    def set_inputs(r):
        logits.copy_(dev(W.gen_logits(81, w.T, w.E, step=r + 1)))
        X.copy_(dev(W.gen_acts(81, w.T, w.K, step=r + 1)))

    g = _capture(run)
    _check_replays(g, set_inputs, run, [lambda: host(bufs["out"]).copy()])


def test_graph_decode_step():
    w = W.custom(82, 1, 64, 4, 256, 128, ffn=True)
    p = W.make_problem(w)
    gu = q.prepack(dev(p.gu_q), dev(p.gu_s), dev(p.gu_b))
    dn = q.prepack(dev(p.dn_q), dev(p.dn_s), dev(p.dn_b))
    sg = q.prepack(dev(p.sh_gu_q), dev(p.sh_gu_s), dev(p.sh_gu_b))
    sd = q.prepack(dev(p.sh_dn_q), dev(p.sh_dn_s), dev(p.sh_dn_b))
    lg, x = dev(p.logits[0]), dev(p.X[0])
    bufs = q.alloc_decode(w.E, w.k, w.K, w.N, True)

    def run():
        q.decode_ffn(lg, x, w.k, gu, dn, sg, sd, bufs=bufs, stream=torch.cuda.current_stream())

    def set_inputs(r):
        lg.copy_(dev(W.gen_logits(82, 1, w.E, step=r + 1)[0]))
        x.copy_(dev(W.gen_acts(82, 1, w.K, step=r + 1)[0]))

    g = _capture(run)
    _check_replays(g, set_inputs, run, [lambda: host(bufs["out"]).copy(), lambda: host(bufs["topk_ids"]).copy()])


def _ffn_weights(p):
    return (q.prepack(dev(p.gu_q), dev(p.gu_s), dev(p.gu_b)), q.prepack(dev(p.dn_q), dev(p.dn_s), dev(p.dn_b)),
            q.prepack(dev(p.sh_gu_q), dev(p.sh_gu_s), dev(p.sh_gu_b)),
            q.prepack(dev(p.sh_dn_q), dev(p.sh_dn_s), dev(p.sh_dn_b)))


@pytest.mark.parametrize("T", [2, 5])
def test_graph_small_batch(T):
    # the few-token layer: routing, distinct-expert plan, gate/up, split down
    # and combine, all on the device
    w = W.custom(83, T, 64, 4, 256, 128, ffn=True)
    p = W.make_problem(w)
    gu, dn, sg, sd = _ffn_weights(p)
    lg, x = dev(p.logits), dev(p.X)
    bufs = q.alloc_small(T, w.E, w.k, w.K, w.N, True)

    def run():
        q.small_batch_ffn(lg, x, w.k, gu, dn, sg, sd, bufs=bufs, stream=torch.cuda.current_stream())

    def set_inputs(r):
        lg.copy_(dev(W.gen_logits(83, T, w.E, step=r + 1)))
        x.copy_(dev(W.gen_acts(83, T, w.K, step=r + 1)))

    g = _capture(run)
    _check_replays(g, set_inputs, run, [lambda: host(bufs["out"]).copy(), lambda: host(bufs["topk_ids"]).copy()])


def test_graph_chunked_prefill():
    # route + FFN per chunk (with the tallest-first block order of 64-row blocks)
    w = W.custom(84, 300, 32, 4, 256, 128, ffn=True)
    p = W.make_problem(w)
    gu, dn, sg, sd = _ffn_weights(p)
    lg, X = dev(p.logits), dev(p.X)
    bufs = q.alloc_chunked(w.T, 128, w.K, w.N, w.E, w.k, 64, True)

    def run():
        q.prefill_ffn_chunked(lg, X, w.k, gu, dn, sg, sd, bufs=bufs, stream=torch.cuda.current_stream())

    def set_inputs(r):
        lg.copy_(dev(W.gen_logits(84, w.T, w.E, step=r + 1)))
        X.copy_(dev(W.gen_acts(84, w.T, w.K, step=r + 1)))

    g = _capture(run)
    _check_replays(g, set_inputs, run, [lambda: host(bufs["out"])[: w.T].copy(),
                                        lambda: host(bufs["topk_ids"])[: w.T].copy()])
