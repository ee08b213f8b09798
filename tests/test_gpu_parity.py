"""GPU parity: the HIP path against the CPU oracle on identical seeded inputs.

Routing tables must match bit for bit; routing weights within 1e-6; grouped
GEMM outputs within tol = 1e-2*rms(oracle) + 1e-3 (rounding-aware, see
tests/parity.py).  Every call goes through the C ABI (ctypes binding)."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import compare_bf16, report

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts only to be skipped
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_util import dev, gpu_gemm, gpu_route, host, tiled_layout  # noqa: E402
import quantized_grouped_gemm_amd as q  # noqa: E402


def _check_route(logits, k, bm):
    T, E = logits.shape
    ids, w = oracle.topk_softmax(logits, k)
    ref = oracle.route(ids, E, bm)
    g = gpu_route(logits, k, bm)
    np.testing.assert_array_equal(g["ids"], ids)
    if T:
        assert np.abs(g["w"].astype(np.float64) - w).max() <= 1e-6
    np.testing.assert_array_equal(g["counts"], ref["counts"])
    np.testing.assert_array_equal(g["offsets"], ref["offsets"])
    np.testing.assert_array_equal(g["perm"], ref["perm"])
    np.testing.assert_array_equal(g["inv_perm"], ref["inv_perm"])
    assert g["num_blocks"] == ref["num_blocks"]
    np.testing.assert_array_equal(g["blocks"], ref["blocks"])
    assert g["num_blocks"] <= g["max_blocks"]
    return g, ids, w, ref


def _logits(kind, T, E, seed=0):
    r = np.random.default_rng([seed, T, E])
    if kind == "normal":
        return r.standard_normal((T, E)).astype(np.float32)
    if kind == "ties":          # few distinct values: many exact ties, and both signed zeros
        l = r.integers(-2, 3, (T, E)).astype(np.float32)
        l[l == 0] = np.where(r.random(int((l == 0).sum())) < 0.5, -0.0, 0.0).astype(np.float32)
        return l
    if kind == "hot":           # expert 3 wins every token's first slot
        l = r.standard_normal((T, E)).astype(np.float32)
        l[:, 3] = 50.0
        return l
    if kind == "constant":      # all equal: selection by expert id only
        return np.full((T, E), 0.5, np.float32)
    raise ValueError(kind)


ROUTE_CASES = [
    ("normal", 64, 16, 2), ("normal", 512, 256, 8), ("normal", 4096, 256, 8), ("normal", 1, 256, 8),
    ("ties", 300, 256, 8), ("ties", 77, 16, 4), ("hot", 1000, 256, 8), ("hot", 50, 64, 1),
    ("constant", 40, 32, 5), ("normal", 3, 1, 1), ("normal", 33, 8, 8), ("normal", 129, 1024, 64),
    ("normal", 200, 300, 6), ("normal", 5, 256, 8), ("normal", 1000, 128, 3), ("normal", 2500, 512, 16),
    # T*k on both sides of 2^16: the scan kernel's packed single scan stops at 65535
    ("normal", 13107, 64, 5), ("normal", 8192, 256, 8),
    # T*k on both sides of 8192, where one workgroup stops ranking from the ids
    # alone; the largest expert count on that path; one expert taking them all
    ("normal", 1024, 256, 8), ("normal", 8193, 1, 1), ("normal", 100, 1024, 64), ("hot", 8192, 64, 1),
    # more chunks than the chunk scan's waves hold in registers (313 chunks of 128 tokens);
    # an expert count that leaves the chunk scan's last workgroup partly idle
    ("normal", 40000, 64, 16), ("normal", 3000, 300, 6),
]


@pytest.mark.parametrize("kind,T,E,k", ROUTE_CASES)
@pytest.mark.parametrize("bm", [16, 128, 160, 256])
def test_route_bit_exact(kind, T, E, k, bm):
    _check_route(_logits(kind, T, E), k, bm)


def test_route_empty_prompt():
    g = gpu_route(np.zeros((0, 16), np.float32), 2, 16)
    assert g["num_blocks"] == 0
    assert np.all(g["counts"] == 0) and np.all(g["offsets"] == 0)


@pytest.mark.parametrize("cid", [1, 2, 4])
def test_route_workloads(cid):
    w = W.WORKLOADS[cid]
    logits = W.gen_logits(cid, w.T, w.E, 0, w.skew_alpha, w.zipf_s)
    bm = {1: 16, 2: 32, 4: 128}[cid]
    g, *_ = _check_route(logits, w.k, bm)
    if cid == 4:   # the skewed workload really is skewed
        c = g["counts"]
        assert c.max() > 10 * c.mean() and (c < 2).mean() > 0.1


def test_route_repeated_calls_reuse_workspace():
    # one set of buffers serves call after call (different inputs, same buffers)
    T, E, k, bm = 700, 64, 4, 32
    b = q.alloc_route(T, E, k, bm)
    for s in range(4):
        lg = _logits("normal", T, E, seed=s)
        d = torch.from_numpy(lg).cuda()
        q.route(d, k, bufs=b)
        torch.cuda.synchronize()
        ids, _ = oracle.topk_softmax(lg, k)
        ref = oracle.route(ids, E, bm)
        np.testing.assert_array_equal(b["perm"].cpu().numpy(), ref["perm"])
        nb = int(b["num_blocks"][0])
        assert nb == ref["num_blocks"]
        np.testing.assert_array_equal(b["blocks"].cpu().numpy().reshape(-1, 4)[:nb], ref["blocks"])


def test_route_decode_steps():
    w = W.WORKLOADS[5]
    for s in range(20):
        _check_route(W.gen_logits(5, 1, w.E, s), w.k, 16)


# ---------------------------------------------------------------- prepack --

@pytest.mark.parametrize("E,N,K", [(3, 32, 256), (2, 48, 192), (1, 16, 64), (4, 64, 320)])
def test_prepack_layout_bit_exact(E, N, K):
    w = W.custom(40, 1, E, 1, K, N)
    p = W.make_problem(w)
    ct, st, bt = q.prepack(dev(p.Wq), dev(p.S), dev(p.B))
    torch.cuda.synchronize()
    rc, rs, rb = tiled_layout(p.Wq, p.S, p.B)
    np.testing.assert_array_equal(host(ct), rc)
    np.testing.assert_array_equal(host(st, np.uint16), rs)
    np.testing.assert_array_equal(host(bt, np.uint16), rb)


# ---------------------------------------------------------------- dequant --

def _bf16_bits(w64):
    """bf16 bit patterns of float64 values that are bf16 numbers."""
    return (w64.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("E,N,K", [(3, 32, 256), (2, 48, 192), (1, 16, 64), (4, 64, 320)])
def test_dequant_bit_exact(E, N, K):
    # every weight rebuilt into memory equals the oracle's bf16(scale*code + bias)
    w = W.custom(41, 1, E, 1, K, N)
    p = W.make_problem(w)
    out = q.dequant(q.prepack(dev(p.Wq), dev(p.S), dev(p.B)), E, N, K)
    torch.cuda.synchronize()
    got = host(out, np.uint16)
    for e in range(E):
        np.testing.assert_array_equal(got[e], _bf16_bits(oracle.dequant_q4(p.Wq[e], p.S[e], p.B[e])))


def test_dequant_prefill_weights_full():
    # every weight of the 256-expert [512 x 2048] prefill workload
    w = W.WORKLOADS[2]
    p = W.make_problem(w)
    out = q.dequant(q.prepack(dev(p.Wq), dev(p.S), dev(p.B)), w.E, w.N, w.K)
    torch.cuda.synchronize()
    for e in range(w.E):
        np.testing.assert_array_equal(host(out[e], np.uint16), _bf16_bits(oracle.dequant_q4(p.Wq[e], p.S[e], p.B[e])))


# ----------------------------------------------------------- grouped GEMM --

def _gemm_full(w, bm, seed_logits=None, name=None):
    p = W.make_problem(w)
    logits = p.logits if seed_logits is None else seed_logits
    g, ids, _, ref = _check_route(logits, w.k, bm)
    Y = gpu_gemm(p.X, w.k, p.Wq, p.S, p.B, g["dev"])
    Yref = oracle.grouped_gemm_q4(p.X, w.k, p.Wq, p.S, p.B, ref["perm"], ref["offsets"])
    ok, st = compare_bf16(Y[: w.T * w.k], Yref)
    if name:
        report(name, st)
    assert ok, st
    return Y, g, p


@pytest.mark.parametrize("bm", [16, 32, 64, 128, 160, 256])
def test_gemm_tiny_workload(bm):
    _gemm_full(W.WORKLOADS[1], bm)


@pytest.mark.parametrize("bm", [16, 32, 64, 128, 160, 256])
def test_gemm_ragged(bm):
    # N = 272 leaves a partial N tile; K = 320 is five K chunks; blocks end mid sub-tile
    _gemm_full(W.custom(31, 200, 8, 3, 320, 272), bm)


@pytest.mark.parametrize("T,E,k,K,N,bm", [
    (40, 1, 1, 192, 48, 16),     # dense: one expert, every token
    (1, 16, 2, 64, 16, 16),      # one token, minimum K and N
    (6, 4, 4, 128, 32, 128),     # k = E, T*k < BM
    (90, 3, 2, 256, 64, 32),     # few experts, many rows each
    (300, 3, 2, 192, 80, 256),   # 256-row blocks: one full, partial ones; odd groups
])
def test_gemm_edge_shapes(T, E, k, K, N, bm):
    _gemm_full(W.custom(32, T, E, k, K, N), bm)


@pytest.mark.parametrize("T,E,k,K,N", [
    (200, 8, 3, 512, 272),      # four chunks; a partial 512-column tile
    (300, 16, 2, 1024, 128),    # narrower than one workgroup's 512 columns
    (100, 64, 8, 2048, 512),    # the prefill shape with a few rows per expert
    (50, 4, 2, 1536, 48),       # twelve chunks; three 16-column tiles
    (40, 2, 1, 512, 16),        # one 16-column tile
    (64, 16, 2, 4096, 64),      # activations too large for LDS: the streaming kernel
])
def test_gemm_short_blocks_lds_resident(T, E, k, K, N):
    # 32-row blocks whose activations fit in LDS for all of K (K a multiple of
    # 512, 32*K*2 <= 128 KB) run the LDS-resident kernel; others the streaming one
    _gemm_full(W.custom(35, T, E, k, K, N), 32)


def test_gemm_hot_expert():
    w = W.custom(33, 300, 16, 2, 256, 128)
    _gemm_full(w, 32, seed_logits=_logits("hot", 300, 16))


def test_gemm_prefill_chunk_full_size():
    # the prefill-chunk workload (T=512, 8 of 256 experts, 2048 -> 512) at its
    # default block height: every one of the 2,097,152 outputs against the oracle
    w = W.WORKLOADS[2]
    Y, g, p = _gemm_full(w, q.moe_default_block_rows(w.T, w.E, w.k), name=w.name)


@pytest.mark.parametrize("bm", [32, 64])
def test_gemm_prefill_chunk_full_size_other_heights(bm):
    w = W.WORKLOADS[2]
    _gemm_full(w, bm, name=f"{w.name} BM={bm}")


@pytest.mark.parametrize("bm", [128, 160, 256])
def test_gemm_skewed_full_size(bm):
    # the skewed workload (T=16384, Zipf-biased logits): all 67,108,864 outputs
    w = W.WORKLOADS[4]
    _gemm_full(w, bm, name=f"{w.name} BM={bm}")


def test_gemm_deterministic():
    w = W.custom(34, 333, 32, 4, 512, 256)
    p = W.make_problem(w)
    g = gpu_route(p.logits, w.k, 32)
    Y1 = gpu_gemm(p.X, w.k, p.Wq, p.S, p.B, g["dev"])
    Y2 = gpu_gemm(p.X, w.k, p.Wq, p.S, p.B, g["dev"], reps=3)
    np.testing.assert_array_equal(Y1, Y2)
    g2 = gpu_route(p.logits, w.k, 32)
    for key in ("ids", "counts", "offsets", "perm", "inv_perm", "blocks"):
        np.testing.assert_array_equal(g[key], g2[key])
