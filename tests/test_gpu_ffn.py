"""GPU parity of the prefill expert FFN (moe_expert_ffn_q4, after moe_route)
against the CPU oracle on identical seeded inputs: the layer output within
tol = 1e-2*rms(oracle) + 1e-3 (rounding-aware, tests/parity.py).  Every call
goes through the C ABI."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import compare_bf16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts only to be skipped
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_util import dev, gpu_route, host  # noqa: E402
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

    def gpu(self, bm, logits=None):
        lg = self.p.logits if logits is None else logits
        g = gpu_route(lg, self.w.k, bm)
        b = q.expert_ffn(self.Xd, self.w.k, g["dev"], self.gu, self.dn, self.sh_gu, self.sh_dn)
        torch.cuda.synchronize()
        return g, host(b["out"], np.uint16)[: self.w.T]

    def check(self, bm, tokens=None, logits=None):
        w, p = self.w, self.p
        lg = p.logits if logits is None else logits
        g, out = self.gpu(bm, lg)
        ids, wts = oracle.topk_softmax(lg, w.k)
        np.testing.assert_array_equal(g["ids"], ids)
        ref = oracle.expert_ffn_q4(p.X, ids, wts, p.gu_q, p.gu_s, p.gu_b, p.dn_q, p.dn_s, p.dn_b,
                                   sh=self.sh_host, tokens=tokens)
        got = out if tokens is None else out[tokens]
        ok, st = compare_bf16(got, ref)
        assert ok, st
        return out


@pytest.mark.parametrize("bm", [16, 32, 64, 128, 256])
def test_ffn_small(bm):
    Layer(W.custom(70, 64, 16, 2, 256, 128, ffn=True)).check(bm)


@pytest.mark.parametrize("bm", [32, 128, 256])
def test_ffn_odd_groups(bm):
    # H = 320 and I = 192: odd group counts in both matrices; T*k not a multiple of BM
    Layer(W.custom(71, 200, 8, 3, 320, 192, ffn=True)).check(bm)


@pytest.mark.parametrize("bm", [16, 128, 256])
def test_ffn_no_shared(bm):
    Layer(W.custom(72, 100, 16, 4, 256, 128, ffn=True), shared=False).check(bm)


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


@pytest.mark.parametrize("bm", [128, 256])
def test_ffn_workload_full_size_sampled(bm):
    # the expert-FFN workload: T=4096, 8 of 256 experts + shared, H=2048, I=512;
    # the oracle checks a sample of tokens
    w = W.WORKLOADS[3]
    L = Layer(w)
    tokens = np.random.default_rng(3).choice(w.T, size=48, replace=False).astype(np.int32)
    out = L.check(bm, tokens=np.sort(tokens))
    assert np.isfinite(out.view(np.int16).astype(np.float32)).all()
