"""GPU parity of the few-token layer (moe_small_batch_ffn_q4, 1 <= T <= 8)
against the CPU oracle on identical seeded inputs: routing ids bit-exact,
routing weights within 1e-6, the layer output within tol = 1e-2*rms(oracle) +
1e-3 (rounding-aware, tests/parity.py).  Every call goes through the C ABI."""
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

    def gpu(self, logits, x):
        b = q.small_batch_ffn(dev(np.ascontiguousarray(logits, np.float32)), dev(x), self.w.k, self.gu, self.dn,
                              self.sh_gu, self.sh_dn)
        torch.cuda.synchronize()
        return b

    def check(self, logits, x):
        w, p = self.w, self.p
        b = self.gpu(logits, x)
        ids, wts = oracle.topk_softmax(logits, w.k)
        np.testing.assert_array_equal(host(b["topk_ids"]), ids)
        assert np.abs(host(b["topk_w"]).astype(np.float64) - wts).max() <= 1e-6
        ref = oracle.expert_ffn_q4(x, ids, wts, p.gu_q, p.gu_s, p.gu_b, p.dn_q, p.dn_s, p.dn_b, sh=self.sh_host)
        ok, st = compare_bf16(host(b["out"], np.uint16), ref)
        assert ok, (logits.shape, st)
        return b


def decode_group(w, T, first_step):
    """T consecutive decode steps' inputs of workload w, as one group of rows."""
    ss = [W.make_problem(w, step=first_step + i, weights=False) for i in range(T)]
    return np.concatenate([s.logits for s in ss]), np.concatenate([s.X for s in ss])


@pytest.fixture(scope="module")
def decode_model():
    return Model(W.WORKLOADS[5])


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 8])
def test_small_batch_decode_shapes(decode_model, T):
    # top-8 of 256 + shared expert, H=2048, I=512: groups of T rows such as a
    # speculative verification step hands the layer
    for first in (0, 11):
        lg, x = decode_group(decode_model.w, T, first)
        decode_model.check(lg, x)


def test_small_batch_shared_experts(decode_model):
    # rows that select the same experts (repeated rows, and all-equal logits:
    # the k lowest ids for every row): each distinct expert is read once for
    # every row that selected it
    lg, x = decode_group(decode_model.w, 4, 3)
    lg2 = np.concatenate([lg[:2], lg[:2]])
    decode_model.check(lg2, x)
    tied = np.full((5, 256), -0.5, np.float32)
    b = decode_model.check(tied, decode_group(decode_model.w, 5, 7)[1])
    np.testing.assert_array_equal(host(b["topk_ids"]), np.tile(np.arange(8), (5, 1)))


def test_small_batch_matches_decode_step(decode_model):
    # one row: the same layer as the batch-1 decode step (fp32 sums in another
    # order, so compared to the rounding-aware tolerance)
    lg, x = decode_group(decode_model.w, 1, 5)
    a = host(decode_model.gpu(lg, x)["out"], np.uint16)[0]
    b = q.decode_ffn(dev(lg[0]), dev(x[0]), 8, decode_model.gu, decode_model.dn, decode_model.sh_gu,
                     decode_model.sh_dn)
    torch.cuda.synchronize()
    from parity import bf16_to_f64
    ok, st = compare_bf16(a, bf16_to_f64(host(b["out"], np.uint16)))
    assert ok, st


def test_small_batch_deterministic(decode_model):
    lg, x = decode_group(decode_model.w, 5, 2)
    a = host(decode_model.gpu(lg, x)["out"]).copy()
    for _ in range(3):
        np.testing.assert_array_equal(host(decode_model.gpu(lg, x)["out"]), a)


@pytest.mark.parametrize("T,E,k,H,I,shared", [
    (3, 16, 2, 320, 192, True),     # odd group counts in both matrices (half-size last chunks)
    (5, 64, 4, 512, 256, False),    # no shared expert
    (8, 8, 8, 256, 128, True),      # k = E: every row selects every expert
    (7, 8, 1, 256, 128, False),     # more rows than distinct experts can be
    (2, 1024, 64, 256, 128, True),  # the largest expert count and top-k
    (8, 128, 6, 1024, 640, True),   # other sizes, eight rows
    (8, 64, 11, 2048, 512, True),   # the largest staged h: 8 x 12 x 512 values, 96 KB of LDS
])
def test_small_batch_shapes(T, E, k, H, I, shared):
    w = W.custom(70 + T, T, E, k, H, I, ffn=True)
    m = Model(w, shared=shared)
    for s in range(2):
        pr = W.make_problem(w, step=s, weights=False)
        m.check(pr.logits, pr.X)
