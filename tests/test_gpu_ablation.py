"""The two comparison arms that `bench.py --ablation` times against the fused
path, checked against the CPU oracle on the prefill-chunk shape (T=512, 8 of
256 experts, 2048 -> 512), so that their timings compare equal work:
  * unfused dequant: moe_dequant_q4 writes every rebuilt bf16 weight to HBM,
    then the vendor batched GEMM multiplies the gathered rows;
  * host-synced routing: the block map built on the host from the expert
    counts copied back, then the grouped GEMM.
Outputs within tol = 1e-2*rms(oracle) + 1e-3 (rounding-aware); the host-built
block map bit-exact against moe_route's."""
import numpy as np
import pytest

import bench
import oracle
import workloads as W
from parity import compare_bf16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts only to be skipped
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_util import dev, gpu_route, host, nan_filled  # noqa: E402
import quantized_grouped_gemm_amd as q  # noqa: E402


def _problem(T):
    w = W.custom(2, T, 256, 8, 2048, 512)
    p = W.make_problem(w)
    ids, _ = oracle.topk_softmax(p.logits, w.k)
    ref = oracle.route(ids, w.E, q.moe_default_block_rows(T, w.E, w.k))
    Yref = oracle.grouped_gemm_q4(p.X, w.k, p.Wq, p.S, p.B, ref["perm"], ref["offsets"])
    return w, p, ref, Yref


@pytest.mark.parametrize("T", [512])
def test_unfused_arm_matches_oracle(T):
    w, p, ref, Yref = _problem(T)
    E, k, K, N = w.E, w.k, w.K, w.N
    packed = q.prepack(dev(p.Wq), dev(p.S), dev(p.B))
    Wbf = q.dequant(packed, E, N, K)
    X = dev(p.X)
    Xz = torch.cat([X.view(torch.bfloat16), torch.zeros((1, K), dtype=torch.bfloat16, device="cuda")])
    src_row = torch.from_numpy(bench.unfused_layout(ref["counts"], ref["offsets"], ref["perm"], k, T)).cuda()
    out = bench.unfused_gemm(torch, Wbf, Xz, src_row)            # [E, N, mpad]
    torch.cuda.synchronize()
    o = out.view(torch.int16).cpu().numpy().view(np.uint16)
    Y = np.full((T * k, N), 0x7FC0, np.uint16)
    for e in range(E):
        c = int(ref["counts"][e])
        Y[ref["offsets"][e]: ref["offsets"][e] + c] = o[e, :, :c].T
    ok, st = compare_bf16(Y, Yref)
    assert ok, st


@pytest.mark.parametrize("T", [512])
def test_hostsync_arm_block_map_and_output(T):
    w, p, ref, Yref = _problem(T)
    k = w.k
    g = gpu_route(p.logits, k, 0)
    blk, nb = bench.host_block_map(g["counts"], g["block_rows"])
    assert nb == g["num_blocks"]
    np.testing.assert_array_equal(blk.reshape(-1, 4), g["blocks"])
    # the grouped GEMM over the host-built map (copied into a poisoned table)
    rt = dict(g["dev"])
    rt["blocks"] = torch.full_like(rt["blocks"], -3)
    rt["blocks"][: blk.size].copy_(torch.from_numpy(blk))
    rt["num_blocks"] = torch.tensor([nb, 0, 0, 0], dtype=torch.int32, device="cuda")
    Y = nan_filled((T * k, w.N))
    q.grouped_gemm_q4(dev(p.X), k, q.prepack(dev(p.Wq), dev(p.S), dev(p.B)), rt, Y=Y)
    torch.cuda.synchronize()
    ok, st = compare_bf16(host(Y, np.uint16), Yref)
    assert ok, st
