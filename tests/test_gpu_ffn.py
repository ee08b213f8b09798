"""GPU parity of the prefill expert FFN (moe_expert_ffn_q4, after moe_route)
against the CPU oracle on identical seeded inputs: the layer output within
tol = 1e-2*rms(oracle) + 1e-3 (rounding-aware, tests/parity.py).  Every call
goes through the C ABI."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import compare_bf16, report

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts only to be skipped
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_util import dev, gpu_route, host, nan_filled  # noqa: E402
import quantized_grouped_gemm_amd as q  # noqa: E402


class Layer:
    def __init__(self, w, shared=True):
        self.w, self.shared = w, shared
        p = W.make_problem(w, shared=shared)
        self.p = p
        self.gu = q.prepack(dev(p.gu_q), dev(p.gu_s), dev(p.gu_b))
        self.dn = q.prepack(dev(p.dn_q), dev(p.dn_s), dev(p.dn_b))
        if shared:
            self.sh_gu = q.prepack(dev(p.sh_gu_q), dev(p.sh_gu_s), dev(p.sh_gu_b))
            self.sh_dn = q.prepack(dev(p.sh_dn_q), dev(p.sh_dn_s), dev(p.sh_dn_b))
            self.sh_host = (p.sh_gu_q, p.sh_gu_s, p.sh_gu_b, p.sh_dn_q, p.sh_dn_s, p.sh_dn_b)
        else:
            self.sh_gu = self.sh_dn = self.sh_host = None
        self.Xd = dev(p.X)

    def gpu(self, bm, logits=None, max_blocks=None):
        lg = self.p.logits if logits is None else logits
        g = gpu_route(lg, self.w.k, bm)
        T, H, I, E, k = self.w.T, self.w.K, self.w.N, self.w.E, self.w.k
        bufs = q.alloc_ffn(T, H, I, E, k, self.shared)
        bufs["out"] = nan_filled((max(T, 1), H))   # rows the kernels skip stay NaN
        rt = g["dev"]
        if max_blocks is not None:                 # a bound larger than this T needs
            rt = dict(rt, max_blocks=max_blocks, blocks=torch.cat(
                [rt["blocks"], torch.full((4 * max_blocks - rt["blocks"].numel(),), -5, dtype=torch.int32,
                                          device="cuda")]))
        b = q.expert_ffn(self.Xd, k, rt, self.gu, self.dn, self.sh_gu, self.sh_dn, bufs=bufs)
        torch.cuda.synchronize()
        return g, host(b["out"], np.uint16)[:T]

    def reference(self, logits=None):
        w, p = self.w, self.p
        lg = p.logits if logits is None else logits
        ids, wts = oracle.topk_softmax(lg, w.k)
        return ids, oracle.expert_ffn_grouped_q4(p.X, ids, wts, p.gu_q, p.gu_s, p.gu_b, p.dn_q, p.dn_s, p.dn_b,
                                                 sh=self.sh_host)

    def check(self, bm, logits=None, ref=None, name=None, max_blocks=None):
        g, out = self.gpu(bm, logits, max_blocks=max_blocks)
        ids, r = ref if ref is not None else self.reference(logits)
        np.testing.assert_array_equal(g["ids"], ids)
        ok, st = compare_bf16(out, r)
        if name:
            report(name, st)
        assert ok, st
        return out


@pytest.mark.parametrize("bm", [16, 32, 64, 128, 160, 256])
def test_ffn_small(bm):
    Layer(W.custom(70, 64, 16, 2, 256, 128, ffn=True)).check(bm)


@pytest.mark.parametrize("bm", [32, 128, 160, 256])
def test_ffn_odd_groups(bm):
    # H = 320 and I = 192: odd group counts in both matrices; T*k not a multiple of BM
    Layer(W.custom(71, 200, 8, 3, 320, 192, ffn=True)).check(bm)


@pytest.mark.parametrize("bm", [16, 128, 256])
def test_ffn_no_shared(bm):
    Layer(W.custom(72, 100, 16, 4, 256, 128, ffn=True), shared=False).check(bm)


@pytest.mark.parametrize("bm", [16, 64, 160])
def test_ffn_smallest_dims(bm):
    # H = I = 64: one scale group along each contraction, one 64-column tile
    Layer(W.custom(75, 50, 8, 2, 64, 64, ffn=True)).check(bm)


def test_ffn_most_experts_widest_topk():
    # E = 1024 experts, k = 64 of them per token
    Layer(W.custom(76, 20, 1024, 64, 128, 64, ffn=True)).check(64)


def test_ffn_few_tokens():
    Layer(W.custom(73, 3, 32, 8, 256, 128, ffn=True)).check(16)


def test_ffn_hot_expert():
    w = W.custom(74, 300, 16, 2, 256, 128, ffn=True)
    lg = np.random.default_rng(5).standard_normal((300, 16)).astype(np.float32)
    lg[:, 3] = 50.0
    Layer(w).check(64, logits=lg)


def test_ffn_deterministic():
    L = Layer(W.custom(75, 333, 32, 4, 256, 128, ffn=True))
    _, a = L.gpu(32)
    _, b = L.gpu(32)
    np.testing.assert_array_equal(a, b)


def test_ffn_oversized_block_bound():
    # max_blocks far above moe_max_blocks (routing buffers sized for a longer
    # batch) with the workspace at its exact size: the launch grid follows the
    # bound of this T, so nothing reads past the workspace or the block map
    L = Layer(W.custom(76, 3, 16, 8, 256, 128, ffn=True))
    L.check(64, max_blocks=100)
    L.check(16, max_blocks=500)


_C3_REF = {}


@pytest.mark.parametrize("bm", [128, 160, 256])
def test_ffn_workload_full_size(bm):
    # the expert-FFN workload: T=4096, 8 of 256 experts + shared, H=2048, I=512;
    # every one of the 4096 x 2048 outputs against the oracle
    w = W.WORKLOADS[3]
    L = Layer(w)
    if "ref" not in _C3_REF:
        _C3_REF["ref"] = L.reference()
    L.check(bm, ref=_C3_REF["ref"], name=f"{w.name} BM={bm}")
