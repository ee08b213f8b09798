"""moe_decode_ffn_q4_noalloc (the decode step on the library's static per-GPU
scratch, for callers that cannot allocate) against moe_decode_ffn_q4 (the same
step on a caller workspace): outputs and routing bit-exact, on two calls in a
row through the C ABI, the second with a smaller problem (fewer experts, a
smaller top-k and hidden size, no shared expert), so that what the first call
left in the scratch cannot stand in for the second's results."""
import numpy as np
import pytest

import workloads as W
from parity import bf16_to_f64

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts only to be skipped
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_util import dev, host  # noqa: E402
import quantized_grouped_gemm_amd as q  # noqa: E402


def _case(cid, E, k, H, I, shared, step):
    w = W.custom(cid, 1, E, k, H, I, ffn=True)
    p = W.make_problem(w, step=step, shared=shared)
    pk = lambda a, b, c: q.prepack(dev(a), dev(b), dev(c))  # noqa: E731
    gu, dn = pk(p.gu_q, p.gu_s, p.gu_b), pk(p.dn_q, p.dn_s, p.dn_b)
    sg = pk(p.sh_gu_q, p.sh_gu_s, p.sh_gu_b) if shared else (None, None, None)
    sd = pk(p.sh_dn_q, p.sh_dn_s, p.sh_dn_b) if shared else (None, None, None)
    return dict(E=E, k=k, H=H, I=I, logits=dev(p.logits[0]), x=dev(p.X[0]), gu=gu, dn=dn, sg=sg, sd=sd,
                shared=shared)


def _with_workspace(c):
    b = q.alloc_decode(c["E"], c["k"], c["H"], c["I"], c["shared"])
    b["out"].fill_(0x7FC0)
    q.moe_decode_ffn_q4(c["logits"], c["x"], c["E"], c["k"], c["H"], c["I"], *c["gu"], *c["dn"], *c["sg"],
                        *c["sd"], b["topk_ids"], b["topk_w"], b["out"], b["workspace"], b["ws_bytes"])
    torch.cuda.synchronize()
    return host(b["out"], np.uint16), host(b["topk_ids"]), host(b["topk_w"])


def _no_alloc(c):
    out = torch.full((c["H"],), 0x7FC0, dtype=torch.int16, device="cuda")
    ids = torch.full((c["k"],), -1, dtype=torch.int32, device="cuda")
    wts = torch.full((c["k"],), -1.0, dtype=torch.float32, device="cuda")
    q.moe_decode_ffn_q4_noalloc(c["logits"], c["x"], c["E"], c["k"], c["H"], c["I"], *c["gu"], *c["dn"],
                                *c["sg"], *c["sd"], ids, wts, out)
    torch.cuda.synchronize()
    return host(out, np.uint16), host(ids), host(wts)


def test_no_alloc_decode_matches_workspace_call_twice():
    big = _case(90, 256, 8, 2048, 512, True, 0)       # the decode workload's shape
    small = _case(91, 64, 4, 1024, 256, False, 1)     # a smaller second call
    assert q.moe_decode_workspace_bytes(256, 8, 2048, 512, True) <= q.MOEQ4_DECODE_SCRATCH_BYTES
    for c in (big, small):
        got = _no_alloc(c)
        want = _with_workspace(c)
        for g, w_ in zip(got, want):
            np.testing.assert_array_equal(g, w_)
        assert not np.isnan(bf16_to_f64(got[0])).any()   # every output written
