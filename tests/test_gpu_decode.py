"""GPU parity of the batch-1 decode step (moe_decode_ffn_q4) against the CPU
oracle on identical seeded inputs: routing ids bit-exact, routing weights
within 1e-6, the layer output within tol = 1e-2*rms(oracle) + 1e-3
(rounding-aware, tests/parity.py).  Every call goes through the C ABI."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import compare_bf16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts only to be skipped
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_util import dev, host  # noqa: E402
import quantized_grouped_gemm_amd as q  # noqa: E402


class Model:
    """Weights of one workload on the host (for the oracle) and prepacked on the device."""

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

    def gpu(self, logits, x, bufs=None):
        b = q.decode_ffn(dev(logits), dev(x), self.w.k, self.gu, self.dn, self.sh_gu, self.sh_dn, bufs=bufs)
        torch.cuda.synchronize()
        return b

    def check(self, step=0, logits=None):
        w, p = self.w, self.p
        s = W.make_problem(w, step=step, weights=False)
        lg = s.logits if logits is None else logits
        b = self.gpu(lg[0], s.X[0])
        ids, wts = oracle.topk_softmax(lg, w.k)
        np.testing.assert_array_equal(host(b["topk_ids"]), ids[0])
        assert np.abs(host(b["topk_w"]).astype(np.float64) - wts[0]).max() <= 1e-6
        ref = oracle.expert_ffn_q4(s.X, ids, wts, p.gu_q, p.gu_s, p.gu_b, p.dn_q, p.dn_s, p.dn_b,
                                   sh=self.sh_host)
        ok, st = compare_bf16(host(b["out"], np.uint16)[None], ref)
        assert ok, (step, st)
        return b


@pytest.fixture(scope="module")
def decode_model():
    return Model(W.WORKLOADS[5])


def test_decode_workload_steps(decode_model):
    # the decode workload: top-8 of 256 + shared expert, H=2048, I=512; fresh
    # logits and activations every step
    for s in range(12):
        decode_model.check(step=s)


def test_decode_deterministic(decode_model):
    s = W.make_problem(decode_model.w, step=3, weights=False)
    a = host(decode_model.gpu(s.logits[0], s.X[0])["out"]).copy()
    for _ in range(3):
        np.testing.assert_array_equal(host(decode_model.gpu(s.logits[0], s.X[0])["out"]), a)


def test_decode_tied_logits(decode_model):
    # all logits equal: the k lowest expert ids, equal weights
    lg = np.full((1, 256), 0.25, np.float32)
    b = decode_model.check(step=0, logits=lg)
    np.testing.assert_array_equal(host(b["topk_ids"]), np.arange(8))


@pytest.mark.parametrize("E,k,H,I,shared", [
    (16, 2, 320, 192, True),     # odd group counts in both matrices (half-size last chunks)
    (64, 4, 512, 256, False),    # no shared expert
    (8, 1, 256, 128, False),     # a single expert: one half of each output tile is empty
    (8, 1, 256, 128, True),
    (1024, 64, 256, 128, True),  # the largest expert count and top-k
    (32, 32, 128, 128, True),    # k = E, smallest sizes
    (8, 2, 8192, 128, True),     # the largest H: x staged as two 16-byte pieces per thread
    (64, 63, 256, 512, True),    # J * I = 32768, the most h one down workgroup stages (64 KB of LDS)
])
def test_decode_shapes(E, k, H, I, shared):
    m = Model(W.custom(60 + k, 1, E, k, H, I, ffn=True), shared=shared)
    for s in range(3):
        m.check(step=s)
