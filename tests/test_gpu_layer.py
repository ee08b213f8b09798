"""GPU parity of the layer call (moe_layer_ffn_q4), which picks its kernels
from the number of rows: the one-row decode step at T=1, the few-row step at
2 <= T <= 8 and routing + the expert FFN above.  Against the CPU oracle
(routing ids bit-exact, weights within 1e-6, output within tol =
1e-2*rms(oracle) + 1e-3, rounding-aware), and bit-exact against the entry
point each path calls directly.  Every call goes through the C ABI."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import compare_bf16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts only to be skipped
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_util import dev, host, nan_filled  # noqa: E402
import quantized_grouped_gemm_amd as q  # noqa: E402

_LAYER = {}


def _layer():
    # the decode-workload weights: 8 of 256 experts + shared, H=2048, I=512
    if not _LAYER:
        w = W.WORKLOADS[5]
        p = W.make_problem(w)
        _LAYER.update(
            w=w, p=p, gu=q.prepack(dev(p.gu_q), dev(p.gu_s), dev(p.gu_b)),
            dn=q.prepack(dev(p.dn_q), dev(p.dn_s), dev(p.dn_b)),
            sg=q.prepack(dev(p.sh_gu_q), dev(p.sh_gu_s), dev(p.sh_gu_b)),
            sd=q.prepack(dev(p.sh_dn_q), dev(p.sh_dn_s), dev(p.sh_dn_b)),
            sh=(p.sh_gu_q, p.sh_gu_s, p.sh_gu_b, p.sh_dn_q, p.sh_dn_s, p.sh_dn_b))
    return _LAYER


@pytest.mark.parametrize("T,path", [(1, q.MOEQ4_PATH_DECODE), (3, q.MOEQ4_PATH_FEW_ROWS),
                                    (8, q.MOEQ4_PATH_FEW_ROWS), (64, q.MOEQ4_PATH_PREFILL),
                                    (9, q.MOEQ4_PATH_PREFILL)])
def test_layer_call_matches_oracle_and_direct_path(T, path):
    L = _layer()
    w, p = L["w"], L["p"]
    E, k, H, I = w.E, w.k, w.K, w.N
    logits = W.gen_logits(w.cid, T, E, 500 + T)
    X = W.gen_acts(w.cid, T, H, 500 + T)
    ld, xd = dev(logits), dev(X)
    b = q.alloc_layer(T, H, I, E, k)
    assert b["path"] == path
    b["out"] = nan_filled((T, H))
    q.layer_ffn(ld, xd, k, L["gu"], L["dn"], L["sg"], L["sd"], bufs=b)
    torch.cuda.synchronize()
    out = host(b["out"], np.uint16)
    ids, wts = oracle.topk_softmax(logits, k)
    np.testing.assert_array_equal(host(b["topk_ids"]), ids)
    assert np.abs(host(b["topk_w"]).astype(np.float64) - wts).max() <= 1e-6
    ref = oracle.expert_ffn_q4(X, ids, wts, p.gu_q, p.gu_s, p.gu_b, p.dn_q, p.dn_s, p.dn_b, sh=L["sh"])
    ok, st = compare_bf16(out, ref)
    assert ok, st
    # the same bits as the entry point of the path
    if path == q.MOEQ4_PATH_DECODE:
        direct = q.decode_ffn(ld[0], xd[0], k, L["gu"], L["dn"], L["sg"], L["sd"])["out"].reshape(1, H)
    elif path == q.MOEQ4_PATH_FEW_ROWS:
        direct = q.small_batch_ffn(ld, xd, k, L["gu"], L["dn"], L["sg"], L["sd"])["out"]
    else:
        rt = q.route(ld, k)
        direct = q.expert_ffn(xd, k, rt, L["gu"], L["dn"], L["sg"], L["sd"])["out"]
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out, host(direct, np.uint16)[:T])
