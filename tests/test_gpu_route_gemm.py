"""GPU parity of moe_route_grouped_gemm_q4: routing and the grouped GEMM in one
call.  Its routing tables must equal the oracle's bit for bit, its routing
weights within 1e-6 and Y the oracle's within the GEMM tolerance
(tests/parity.py).  Y must also equal, bit for bit, what moe_route followed by
moe_grouped_gemm_q4 write: the same rebuild and the same order of sums.  The
call ranks each expert's rows inside the GEMM launch (64-row blocks, up to
4096 assignments); the other shapes here take the two-call path."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import compare_bf16, report

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts only to be skipped
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_util import dev, gpu_gemm, gpu_route, host, nan_filled  # noqa: E402
import quantized_grouped_gemm_amd as q  # noqa: E402

TABLES = ("topk_ids", "counts", "offsets", "perm", "inv_perm", "blocks", "num_blocks")


def _hot_logits(T, E, seed):
    # expert 3 wins every token's first slot: one expert holds T rows
    l = np.random.default_rng([seed, T, E]).standard_normal((T, E)).astype(np.float32)
    l[:, 3] = 50.0
    return l


def _fused(w, p, logits, bm, rt=None, packed=None):
    T, E = logits.shape
    A = T * w.k
    rt = rt or q.alloc_route(T, E, w.k, bm)
    for key in TABLES:
        rt[key].fill_(-7)
    packed = packed or q.prepack(dev(p.Wq), dev(p.S), dev(p.B))
    Y = nan_filled((max(A, 1), w.N))
    lg = dev(np.ascontiguousarray(logits, np.float32)) if T else torch.empty((0, E), device="cuda")
    X = dev(p.X) if T else torch.empty((0, w.K), dtype=torch.int16, device="cuda")
    q.route_grouped_gemm_q4(lg, X, w.k, packed, rt, Y=Y)
    torch.cuda.synchronize()
    nb = int(host(rt["num_blocks"])[0])
    return dict(
        ids=host(rt["topk_ids"])[:A].reshape(T, w.k), w=host(rt["topk_w"])[:A].reshape(T, w.k),
        counts=host(rt["counts"]), offsets=host(rt["offsets"]), perm=host(rt["perm"])[:A],
        inv_perm=host(rt["inv_perm"])[:A], num_blocks=nb, blocks=host(rt["blocks"]).reshape(-1, 4)[:nb],
        Y=host(Y, np.uint16)[:A], block_rows=rt["block_rows"], rt=rt, packed=packed)


def _check(w, bm, logits=None, name=None, against_two_calls=True):
    p = W.make_problem(w)
    logits = p.logits if logits is None else logits
    g = _fused(w, p, logits, bm)
    ids, wt = oracle.topk_softmax(logits, w.k)
    ref = oracle.route(ids, w.E, g["block_rows"])
    np.testing.assert_array_equal(g["ids"], ids)
    if w.T:
        assert np.abs(g["w"].astype(np.float64) - wt).max() <= 1e-6
    for key in ("counts", "offsets", "perm", "inv_perm"):
        np.testing.assert_array_equal(g[key], ref[key], err_msg=key)
    assert g["num_blocks"] == ref["num_blocks"]
    np.testing.assert_array_equal(g["blocks"], ref["blocks"])
    if w.T == 0:
        return g
    Yref = oracle.grouped_gemm_q4(p.X, w.k, p.Wq, p.S, p.B, ref["perm"], ref["offsets"])
    ok, st = compare_bf16(g["Y"], Yref)
    if name:
        report(name, st)
    assert ok, st
    if against_two_calls:
        r = gpu_route(logits, w.k, g["block_rows"])
        Y2 = gpu_gemm(p.X, w.k, p.Wq, p.S, p.B, r["dev"])
        np.testing.assert_array_equal(g["Y"], Y2[: w.T * w.k])
    return g


def test_route_gemm_prefill_chunk_full_size():
    # the prefill-chunk workload (T=512, 8 of 256 experts, 2048 -> 512) at its
    # default block height (64 rows): every table entry and all 2,097,152 outputs
    w = W.WORKLOADS[2]
    assert q.moe_default_block_rows(w.T, w.E, w.k) == 64
    _check(w, 0, name=f"{w.name} (routing in the GEMM launch)")


@pytest.mark.parametrize("T,E,k,K,N", [
    (64, 16, 2, 256, 128),     # the tiny workload's shape
    (200, 8, 3, 320, 272),     # 75 rows per expert: two passes; odd groups; a partial N tile
    (1, 256, 8, 2048, 512),    # one token: 248 experts without rows
    (5, 256, 8, 256, 64),      # 40 assignments over 256 experts
    (100, 1024, 8, 128, 32),   # the largest expert count: four histogram entries per thread
    (1024, 256, 4, 128, 64),   # 4096 assignments, the most one launch ranks
    (512, 8, 8, 128, 64),      # k = E: every token picks every expert (8 passes each)
    (40, 4, 2, 64, 32),        # one group of K: no full chunk to start early
    (700, 64, 4, 256, 48),     # 11 rounds of 256 assignments; a 48-column tile
    (64, 1024, 64, 128, 32),   # the widest top-k over the most experts: 4096 assignments
])
def test_route_gemm_shapes(T, E, k, K, N):
    _check(W.custom(90, T, E, k, K, N), 64)


def _random_shape(seed):
    # a seeded shape inside the one-launch limits (T*k <= 4096), weights kept small
    r = np.random.default_rng([98, seed])
    E = int(r.choice([1, 3, 8, 17, 64, 200, 256, 511, 1024]))
    k = int(r.integers(1, min(E, 64) + 1))
    T = int(r.integers(1, 4096 // k + 1))
    K = 64 * int(r.integers(1, 9))
    N = 16 * int(r.integers(1, 17))
    while E * N * K > (1 << 24):  # halve N, then K, in whole tiles
        if N > 16:
            N = 16 * max(1, N // 32)
        else:
            K = 64 * max(1, K // 128)
    return T, E, k, K, N


@pytest.mark.parametrize("seed", range(12))
def test_route_gemm_random_shapes(seed):
    # seeded shapes across the limits: tables against the oracle, Y against the
    # oracle and bit for bit against the two calls
    T, E, k, K, N = _random_shape(seed)
    print(f"route+gemm random case {seed}: T={T} E={E} k={k} K={K} N={N}", flush=True)
    _check(W.custom(100 + seed, T, E, k, K, N), 64)


def test_route_gemm_hot_expert_many_passes():
    # one expert takes all 500 tokens: its workgroups run 8 passes of 64 rows
    w = W.custom(91, 500, 256, 8, 256, 128)
    g = _check(w, 64, logits=_hot_logits(w.T, w.E, 91))
    assert g["counts"][3] == w.T


def test_route_gemm_tied_logits():
    # logits on a coarse grid: most tokens hold exact ties inside and at the
    # edge of their top k, settled by the lower expert id as in the oracle
    w = W.custom(97, 256, 64, 6, 128, 64)
    l = np.random.default_rng([97, 256, 64]).standard_normal((256, 64))
    _check(w, 64, logits=(np.round(l * 2) / 2).astype(np.float32))


@pytest.mark.parametrize("T,E,k,bm", [
    (4097, 1, 1, 64),    # past 4096 assignments: the two-call path
    (1000, 256, 8, 64),  # 8000 assignments at 64-row blocks: the two-call path
    (300, 16, 2, 128),   # taller blocks: the two-call path
    (64, 16, 2, 16),
])
def test_route_gemm_two_call_path(T, E, k, bm):
    _check(W.custom(92, T, E, k, 128, 64), bm)


def test_route_gemm_empty_prompt():
    E, k, K, N = 16, 2, 128, 64
    rt = q.alloc_route(0, E, k, 64)
    for key in TABLES:
        rt[key].fill_(-7)
    w = W.custom(93, 1, E, k, K, N)
    p = W.make_problem(w)
    packed = q.prepack(dev(p.Wq), dev(p.S), dev(p.B))
    q.route_grouped_gemm_q4(torch.empty((0, E), device="cuda"), torch.empty((0, K), dtype=torch.int16, device="cuda"),
                            k, packed, rt, Y=nan_filled((1, N)))
    torch.cuda.synchronize()
    assert int(host(rt["num_blocks"])[0]) == 0
    assert not host(rt["counts"]).any() and not host(rt["offsets"]).any()


def test_route_gemm_reuses_buffers():
    # one set of buffers and weights, call after call with new logits: every
    # table entry is rewritten (nothing stale from the previous routing)
    w = W.custom(94, 300, 32, 4, 256, 64)
    p = W.make_problem(w)
    rt = q.alloc_route(w.T, w.E, w.k, 64)
    packed = q.prepack(dev(p.Wq), dev(p.S), dev(p.B))
    for s in range(3):
        logits = W.gen_logits(94, w.T, w.E, step=s)
        g = _fused(w, p, logits, 64, rt=rt, packed=packed)
        ids, _ = oracle.topk_softmax(logits, w.k)
        ref = oracle.route(ids, w.E, 64)
        for key in ("counts", "offsets", "perm", "inv_perm"):
            np.testing.assert_array_equal(g[key], ref[key], err_msg=key)
        np.testing.assert_array_equal(g["blocks"], ref["blocks"])
        Yref = oracle.grouped_gemm_q4(p.X, w.k, p.Wq, p.S, p.B, ref["perm"], ref["offsets"])
        ok, st = compare_bf16(g["Y"], Yref)
        assert ok, st


def test_route_gemm_graph_replays():
    # captured once, replayed with fresh logits and activations: each replay
    # equals the eager call bit for bit
    from test_gpu_graph import _capture, _check_replays
    w = W.custom(95, 400, 64, 8, 256, 128)
    p = W.make_problem(w)
    logits, X = dev(p.logits), dev(p.X)
    packed = q.prepack(dev(p.Wq), dev(p.S), dev(p.B))
    rt = q.alloc_route(w.T, w.E, w.k, 64)
    Y = torch.empty((w.T * w.k, w.N), dtype=torch.int16, device="cuda")

    def run():
        q.route_grouped_gemm_q4(logits, X, w.k, packed, rt, Y=Y, stream=torch.cuda.current_stream())

    def set_inputs(r):
        logits.copy_(dev(W.gen_logits(95, w.T, w.E, step=r + 1)))
        X.copy_(dev(W.gen_acts(95, w.T, w.K, step=r + 1)))

    def blocks():
        nb = int(host(rt["num_blocks"])[0])
        return host(rt["blocks"])[: 4 * nb].copy()

    g = _capture(run)
    _check_replays(g, set_inputs, run, [lambda: host(Y).copy(), lambda: host(rt["perm"]).copy(),
                                        lambda: host(rt["inv_perm"]).copy(), blocks,
                                        lambda: host(rt["counts"]).copy(), lambda: host(rt["offsets"]).copy()])


@pytest.mark.parametrize("T,E,k", [(512, 256, 8), (77, 16, 4), (1, 1024, 64), (3000, 64, 2)])
def test_topk_softmax_alone(T, E, k):
    # moe_topk_softmax writes exactly moe_route's ids and weights
    logits = W.gen_logits(96, T, E)
    rt = q.alloc_route(T, E, k, 64)
    rt["topk_ids"].fill_(-7)
    q.topk_softmax(dev(logits), k, rt)
    torch.cuda.synchronize()
    ids, wt = oracle.topk_softmax(logits, k)
    np.testing.assert_array_equal(host(rt["topk_ids"])[: T * k].reshape(T, k), ids)
    assert np.abs(host(rt["topk_w"])[: T * k].reshape(T, k).astype(np.float64) - wt).max() <= 1e-6
    g = gpu_route(logits, k, 64)
    np.testing.assert_array_equal(host(rt["topk_w"])[: T * k].reshape(T, k), g["w"])
