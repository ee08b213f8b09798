"""GPU parity of the chunked prefill (moe_prefill_ffn_chunked_q4): the routed
FFN + shared expert of a prompt run as bounded chunks that reuse one chunk's
scratch.  Against the CPU oracle (routing ids bit-exact, weights within 1e-6,
output within tol = 1e-2*rms(oracle) + 1e-3, rounding-aware), and bit-exact
against the same chunks run one by one through moe_route + moe_expert_ffn_q4
(the driver only moves pointers).  Every call goes through the C ABI."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import compare_bf16, report

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts only to be skipped
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_util import dev, host, nan_filled  # noqa: E402
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
        self.Ld, self.Xd = dev(p.logits), dev(p.X)

    def chunked(self, chunk, bm=0):
        T, H, I, E, k = self.w.T, self.w.K, self.w.N, self.w.E, self.w.k
        bufs = q.alloc_chunked(T, chunk, H, I, E, k, bm, self.shared)
        bufs["out"] = nan_filled((max(T, 1), H))   # rows the kernels skip stay NaN
        b = q.prefill_ffn_chunked(self.Ld, self.Xd, self.w.k, self.gu, self.dn, self.sh_gu, self.sh_dn,
                                  chunk_tokens=chunk, block_rows=bm, bufs=bufs)
        torch.cuda.synchronize()
        T = self.w.T
        return host(b["topk_ids"])[:T], host(b["topk_w"])[:T], host(b["out"], np.uint16)[:T]

    def one_by_one(self, chunk, bm):
        outs = []
        for t0 in range(0, self.w.T, chunk):
            rt = q.route(self.Ld[t0:t0 + chunk].contiguous(), self.w.k, block_rows=bm)
            b = q.expert_ffn(self.Xd[t0:t0 + chunk].contiguous(), self.w.k, rt, self.gu, self.dn, self.sh_gu,
                             self.sh_dn)
            torch.cuda.synchronize()
            outs.append(host(b["out"], np.uint16)[: min(chunk, self.w.T - t0)])
        return np.concatenate(outs)

    def check_oracle(self, chunk, bm=0, name=None):
        p, k = self.p, self.w.k
        ids, wts, out = self.chunked(chunk, bm)
        rid, rw = oracle.topk_softmax(p.logits, k)
        np.testing.assert_array_equal(ids, rid)
        assert np.abs(wts.astype(np.float64) - rw).max() <= 1e-6
        ref = oracle.expert_ffn_grouped_q4(p.X, rid, rw, p.gu_q, p.gu_s, p.gu_b, p.dn_q, p.dn_s, p.dn_b,
                                           sh=self.sh_host)
        ok, st = compare_bf16(out, ref)
        if name:
            report(name, st)
        assert ok, (chunk, st)
        return out


@pytest.mark.parametrize("chunk,bm", [(256, 0), (256, 32), (100, 16), (1000, 64), (4096, 0)])
def test_chunked_matches_oracle(chunk, bm):
    # T=1000: chunks of 256 leave a 232-token tail; 100 gives ten chunks; a
    # chunk at least as long as T is one call
    Layer(W.custom(80, 1000, 64, 4, 256, 128, ffn=True)).check_oracle(chunk, bm)


@pytest.mark.parametrize("chunk,bm", [(256, 32), (100, 16), (1000, 64)])
def test_chunked_equals_chunks_one_by_one(chunk, bm):
    L = Layer(W.custom(81, 1000, 64, 4, 320, 192, ffn=True))
    _, _, out = L.chunked(chunk, bm)
    np.testing.assert_array_equal(out, L.one_by_one(chunk, bm))


def test_chunked_no_shared_expert():
    Layer(W.custom(82, 777, 32, 2, 256, 128, ffn=True), shared=False).check_oracle(128, 32)


def test_chunked_deterministic():
    L = Layer(W.custom(83, 600, 64, 4, 256, 128, ffn=True))
    a = L.chunked(128)[2]
    np.testing.assert_array_equal(L.chunked(128)[2], a)


def test_chunked_expert_ffn_workload_full_size():
    # the expert-FFN workload (T=4096, 8 of 256 + shared, H=2048, I=512) in
    # chunks of 1024 tokens: every output against the oracle
    w = W.WORKLOADS[3]
    Layer(w).check_oracle(1024, 0, name=f"{w.name} in chunks of 1024")
