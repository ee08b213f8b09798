"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments on the host before enqueueing
anything.  No compute call is made here."""
import ctypes
import os
import re

import pytest

import oracle
import quantized_grouped_gemm_amd as q

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moeq4.h")


def _declared():
    src = open(HDR).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert {"moe_route", "moe_grouped_gemm_q4", "moe_strerror"} <= set(names)
    raw = ctypes.CDLL(q.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(names) == set(q.SIGNATURES), "binding and header disagree"


def test_limits_match_header():
    src = open(HDR).read()
    for name in ("MOEQ4_MAX_EXPERTS", "MOEQ4_MAX_TOPK", "MOEQ4_SMALL_MAX_T", "MOEQ4_ROUTE_IN_LAUNCH_MAX"):
        m = re.search(r"#define\s+%s\s+(\d+)" % name, src)
        assert m and int(m.group(1)) == getattr(q, name), name


def test_strerror_covers_codes():
    for c in range(0, -7, -1):
        assert q.strerror(c) != "unknown status"
    assert q.strerror(-99) == "unknown status"


@pytest.mark.parametrize("T,E,k", [(64, 16, 2), (512, 256, 8), (4096, 256, 8), (16384, 256, 8), (1, 256, 8),
                                   (0, 16, 2), (7, 1, 1), (100, 1024, 64)])
def test_host_helpers(T, E, k):
    bm = q.moe_default_block_rows(T, E, k)
    assert bm in (16, 32, 64, 128, 160, 256)
    for b in (16, 32, 64, 128, 160, 256):
        assert q.moe_max_blocks(T, E, k, b) == oracle.max_blocks_bound(T * k, E, b)
    assert q.moe_max_blocks(T, E, k, 0) == q.moe_max_blocks(T, E, k, bm)
    assert q.moe_route_workspace_bytes(T, E, k, 0) >= 4 * T * k


def test_default_block_rows_follows_expert_load():
    assert q.moe_default_block_rows(512, 256, 8) == 64     # ~16 rows per expert: one 64-row block each
    assert q.moe_default_block_rows(4096, 256, 8) == 160   # ~128 rows per expert: one block each
    assert q.moe_default_block_rows(16384, 256, 8) == 160  # heavy and skewed
    assert q.moe_default_block_rows(2048, 256, 8) == 128   # ~64 rows per expert
    assert q.moe_default_block_rows(1024, 256, 8) == 64    # ~32 rows per expert
    assert q.moe_default_block_rows(64, 16, 2) == 64       # ~8 rows per expert


def test_invalid_shapes_rejected():
    L = q.lib()
    assert L.moe_max_blocks(-1, 16, 2, 16) == q.MOEQ4_ERR_SHAPE
    assert L.moe_max_blocks(8, 16, 17, 16) == q.MOEQ4_ERR_SHAPE        # k > E
    assert L.moe_max_blocks(8, 16, 0, 16) == q.MOEQ4_ERR_SHAPE
    assert L.moe_max_blocks(8, 2048, 2, 16) == q.MOEQ4_ERR_SHAPE       # E > 1024
    assert L.moe_max_blocks(8, 128, 65, 16) == q.MOEQ4_ERR_UNSUPPORTED  # k > 64
    assert L.moe_max_blocks(8, 16, 2, 24) == q.MOEQ4_ERR_SHAPE         # block_rows
    assert L.moe_route_workspace_bytes(8, 16, 17, 16) == 0


FAKE = 1 << 20   # 16-B aligned host-side stand-ins: never dereferenced, the calls fail first


def _route(**kw):
    a = dict(logits=FAKE, T=8, E=16, k=2, block_rows=16, topk_ids=FAKE, topk_w=FAKE, counts=FAKE,
             offsets=FAKE, perm=FAKE, inv_perm=FAKE, blocks=FAKE, num_blocks=FAKE, workspace=FAKE,
             ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return q.lib().moe_route(*a.values())


def test_route_validation():
    assert _route(T=-1) == q.MOEQ4_ERR_SHAPE
    assert _route(k=0) == q.MOEQ4_ERR_SHAPE
    assert _route(block_rows=48) == q.MOEQ4_ERR_SHAPE
    assert _route(logits=None) == q.MOEQ4_ERR_NULL
    assert _route(perm=None) == q.MOEQ4_ERR_NULL
    assert _route(num_blocks=None) == q.MOEQ4_ERR_NULL
    assert _route(ws_bytes=0) == q.MOEQ4_ERR_WORKSPACE
    assert _route(workspace=None) == q.MOEQ4_ERR_NULL
    assert _route(topk_w=FAKE + 4) == q.MOEQ4_ERR_ALIGN


def _gemm(**kw):
    a = dict(X=FAKE, T=8, K=256, N=128, E=16, k=2, Wq=FAKE, scales=FAKE, biases=FAKE, perm=FAKE,
             blocks=FAKE, num_blocks=FAKE, max_blocks=1000, block_rows=16, Y=FAKE, stream=None)
    a.update(kw)
    return q.lib().moe_grouped_gemm_q4(*a.values())


def test_gemm_validation():
    assert _gemm(K=96) == q.MOEQ4_ERR_SHAPE
    assert _gemm(K=0) == q.MOEQ4_ERR_SHAPE
    assert _gemm(N=120) == q.MOEQ4_ERR_SHAPE
    assert _gemm(max_blocks=q.moe_max_blocks(8, 16, 2, 16) - 1) == q.MOEQ4_ERR_SHAPE
    assert _gemm(block_rows=8) == q.MOEQ4_ERR_SHAPE
    assert _gemm(Wq=None) == q.MOEQ4_ERR_NULL
    assert _gemm(Y=None) == q.MOEQ4_ERR_NULL
    assert _gemm(Y=FAKE + 2) == q.MOEQ4_ERR_ALIGN
    assert _gemm(T=0, X=None, Y=None) == q.MOEQ4_OK     # nothing to do: no launch


def test_topk_validation():
    f = q.lib().moe_topk_softmax
    assert f(FAKE, 8, 16, 0, FAKE, FAKE, None) == q.MOEQ4_ERR_SHAPE
    assert f(FAKE, 8, 16, 17, FAKE, FAKE, None) == q.MOEQ4_ERR_SHAPE
    assert f(FAKE, 8, 2048, 8, FAKE, FAKE, None) == q.MOEQ4_ERR_SHAPE        # E > MOEQ4_MAX_EXPERTS
    assert f(FAKE, 8, 256, 65, FAKE, FAKE, None) == q.MOEQ4_ERR_UNSUPPORTED   # k > MOEQ4_MAX_TOPK
    assert f(None, 8, 16, 2, FAKE, FAKE, None) == q.MOEQ4_ERR_NULL
    assert f(FAKE, 8, 16, 2, FAKE + 4, FAKE, None) == q.MOEQ4_ERR_ALIGN
    assert f(None, 0, 16, 2, None, None, None) == q.MOEQ4_OK                # T = 0: nothing to do


def _route_gemm(**kw):
    a = dict(logits=FAKE, X=FAKE, T=8, K=256, N=128, E=16, k=2, Wq=FAKE, scales=FAKE, biases=FAKE,
             block_rows=64, topk_ids=FAKE, topk_w=FAKE, counts=FAKE, offsets=FAKE, perm=FAKE, inv_perm=FAKE,
             blocks=FAKE, num_blocks=FAKE, max_blocks=1000, Y=FAKE, workspace=FAKE, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return q.lib().moe_route_grouped_gemm_q4(*a.values())


def test_route_gemm_validation():
    assert _route_gemm(K=96) == q.MOEQ4_ERR_SHAPE
    assert _route_gemm(N=120) == q.MOEQ4_ERR_SHAPE
    assert _route_gemm(k=0) == q.MOEQ4_ERR_SHAPE
    assert _route_gemm(block_rows=48) == q.MOEQ4_ERR_SHAPE
    assert _route_gemm(max_blocks=q.moe_max_blocks(8, 16, 2, 64) - 1) == q.MOEQ4_ERR_SHAPE
    assert _route_gemm(logits=None) == q.MOEQ4_ERR_NULL
    assert _route_gemm(X=None) == q.MOEQ4_ERR_NULL
    assert _route_gemm(inv_perm=None) == q.MOEQ4_ERR_NULL
    assert _route_gemm(num_blocks=None) == q.MOEQ4_ERR_NULL
    assert _route_gemm(ws_bytes=0, block_rows=128) == q.MOEQ4_ERR_WORKSPACE
    assert _route_gemm(Y=FAKE + 2) == q.MOEQ4_ERR_ALIGN
    assert _route_gemm(topk_w=FAKE + 4) == q.MOEQ4_ERR_ALIGN


def test_single_hip_runtime_in_process():
    # torch's HIP runtime must be the one libmoeq4 binds to (streams and
    # pointers come from torch); two copies of libamdhip64 would not share them
    q.lib()
    with open("/proc/self/maps") as f:
        paths = {ln.split()[-1] for ln in f if "libamdhip64" in ln}
    assert len(paths) == 1, paths


def _prepack(**kw):
    a = dict(codes=FAKE, scales=FAKE, biases=FAKE, E=2, N=32, K=128, codes_t=FAKE, scales_t=FAKE,
             biases_t=FAKE, stream=None)
    a.update(kw)
    return q.lib().moe_prepack_q4(*a.values())


def test_prepack_validation():
    assert _prepack(N=24) == q.MOEQ4_ERR_SHAPE
    assert _prepack(K=96) == q.MOEQ4_ERR_SHAPE
    assert _prepack(E=0) == q.MOEQ4_ERR_SHAPE
    assert _prepack(codes_t=None) == q.MOEQ4_ERR_NULL
    assert _prepack(scales=FAKE + 8) == q.MOEQ4_ERR_ALIGN


def _decode(**kw):
    a = dict(logits=FAKE, x=FAKE, E=16, k=2, H=256, I=128, gu_q=FAKE, gu_s=FAKE, gu_b=FAKE, dn_q=FAKE,
             dn_s=FAKE, dn_b=FAKE, sh_gu_q=None, sh_gu_s=None, sh_gu_b=None, sh_dn_q=None, sh_dn_s=None,
             sh_dn_b=None, topk_ids=None, topk_w=None, out=FAKE, workspace=FAKE,
             ws_bytes=q.moe_decode_workspace_bytes(16, 2, 256, 128, False), stream=None)
    a.update(kw)
    return q.lib().moe_decode_ffn_q4(*a.values())


def test_decode_validation():
    assert q.moe_decode_workspace_bytes(256, 8, 2048, 512, True) > 0
    assert q.moe_decode_workspace_bytes(256, 8, 64, 512, True) == 0     # H below 128
    assert q.moe_decode_workspace_bytes(256, 8, 2048, 96, True) == 0    # I not a multiple of 64
    assert _decode(H=192 + 8) == q.MOEQ4_ERR_SHAPE
    assert _decode(k=17) == q.MOEQ4_ERR_SHAPE                           # k > E
    assert _decode(E=128, k=65) == q.MOEQ4_ERR_UNSUPPORTED               # k > 64
    assert _decode(logits=None) == q.MOEQ4_ERR_NULL
    assert _decode(out=None) == q.MOEQ4_ERR_NULL
    assert _decode(sh_gu_q=FAKE) == q.MOEQ4_ERR_NULL                    # shared: all six or none
    assert _decode(x=FAKE + 4) == q.MOEQ4_ERR_ALIGN
    assert _decode(ws_bytes=16) == q.MOEQ4_ERR_WORKSPACE
    assert _decode(E=128, k=64, I=1088) == q.MOEQ4_ERR_UNSUPPORTED      # h of 32 experts: beyond LDS


def _small(**kw):
    # every call below carries one invalid argument: rejected before any launch
    a = dict(logits=FAKE, x=FAKE, T=3, E=16, k=2, H=256, I=128, gu_q=FAKE, gu_s=FAKE, gu_b=FAKE, dn_q=FAKE,
             dn_s=FAKE, dn_b=FAKE, sh_gu_q=None, sh_gu_s=None, sh_gu_b=None, sh_dn_q=None, sh_dn_s=None,
             sh_dn_b=None, topk_ids=None, topk_w=None, out=FAKE, workspace=FAKE,
             ws_bytes=q.moe_small_batch_workspace_bytes(3, 16, 2, 256, 128, False), stream=None)
    a.update(kw)
    return q.lib().moe_small_batch_ffn_q4(*a.values())


def test_small_batch_validation():
    assert q.moe_small_batch_workspace_bytes(5, 256, 8, 2048, 512, True) > 0
    assert q.moe_small_batch_workspace_bytes(8, 256, 8, 2048, 512, True) > 0   # the decode shapes, 8 tokens
    # the plan, the routing and the gated outputs: grows with T and with the distinct-expert slots
    assert (q.moe_small_batch_workspace_bytes(8, 256, 8, 2048, 512, True) >
            q.moe_small_batch_workspace_bytes(2, 256, 8, 2048, 512, True))
    assert q.moe_small_batch_workspace_bytes(0, 256, 8, 2048, 512, True) == 0    # T = 0
    assert q.moe_small_batch_workspace_bytes(9, 256, 8, 2048, 512, True) == 0    # T above 8
    assert q.moe_small_batch_workspace_bytes(8, 256, 8, 4096, 512, True) == 0    # x of 8 tokens beyond LDS
    assert q.moe_small_batch_workspace_bytes(8, 256, 16, 2048, 512, True) == 0   # h beyond LDS
    assert q.moe_small_batch_workspace_bytes(2, 256, 8, 2048, 96, True) == 0     # I not a multiple of 64
    assert _small(T=0) == q.MOEQ4_ERR_SHAPE
    assert _small(T=q.MOEQ4_SMALL_MAX_T + 1) == q.MOEQ4_ERR_UNSUPPORTED
    assert _small(k=17) == q.MOEQ4_ERR_SHAPE                            # k > E
    assert _small(E=128, k=65) == q.MOEQ4_ERR_UNSUPPORTED                # k > 64
    assert _small(H=192 + 8) == q.MOEQ4_ERR_SHAPE
    assert _small(T=8, H=4096) == q.MOEQ4_ERR_UNSUPPORTED
    assert _small(logits=None) == q.MOEQ4_ERR_NULL
    assert _small(out=None) == q.MOEQ4_ERR_NULL
    assert _small(sh_dn_b=FAKE) == q.MOEQ4_ERR_NULL                     # shared: all six or none
    assert _small(x=FAKE + 4) == q.MOEQ4_ERR_ALIGN
    assert _small(topk_w=FAKE + 8) == q.MOEQ4_ERR_ALIGN
    assert _small(ws_bytes=16) == q.MOEQ4_ERR_WORKSPACE


def _chunked(**kw):
    # every call below carries one invalid argument: rejected before any launch
    a = dict(logits=FAKE, X=FAKE, T=1000, H=256, I=128, E=16, k=2, gu_q=FAKE, gu_s=FAKE, gu_b=FAKE, dn_q=FAKE,
             dn_s=FAKE, dn_b=FAKE, sh_gu_q=None, sh_gu_s=None, sh_gu_b=None, sh_dn_q=None, sh_dn_s=None,
             sh_dn_b=None, chunk_tokens=256, block_rows=0, topk_ids=None, topk_w=None, out=FAKE, workspace=FAKE,
             ws_bytes=q.moe_prefill_ffn_chunked_workspace_bytes(1000, 256, 256, 128, 16, 2, 0, False), stream=None)
    a.update(kw)
    return q.lib().moe_prefill_ffn_chunked_q4(*a.values())


def test_chunked_validation():
    ws = q.moe_prefill_ffn_chunked_workspace_bytes
    assert ws(16384, 1024, 2048, 512, 256, 8, 0, True) > 0
    # the scratch is that of one chunk: it does not grow with the prompt
    assert ws(16384, 1024, 2048, 512, 256, 8, 0, True) == ws(4096, 1024, 2048, 512, 256, 8, 0, True)
    assert ws(16384, 1024, 2048, 512, 256, 8, 0, True) < q.moe_expert_ffn_workspace_bytes(16384, 2048, 512, 256, 8,
                                                                                          True)
    assert ws(1000, 6, 256, 128, 16, 2, 0, False) == 0       # chunk not a multiple of 4
    assert ws(1000, 0, 256, 128, 16, 2, 0, False) == 0
    assert ws(1000, 256, 256, 96, 16, 2, 0, False) == 0      # I not a multiple of 64
    assert ws(1000, 256, 256, 128, 16, 2, 24, False) == 0    # block rows
    assert _chunked(chunk_tokens=0) == q.MOEQ4_ERR_SHAPE
    assert _chunked(chunk_tokens=130) == q.MOEQ4_ERR_SHAPE
    assert _chunked(T=-1) == q.MOEQ4_ERR_SHAPE
    assert _chunked(k=17) == q.MOEQ4_ERR_SHAPE
    assert _chunked(block_rows=48) == q.MOEQ4_ERR_SHAPE
    assert _chunked(logits=None) == q.MOEQ4_ERR_NULL
    assert _chunked(out=None) == q.MOEQ4_ERR_NULL
    assert _chunked(sh_gu_b=FAKE) == q.MOEQ4_ERR_NULL
    assert _chunked(X=FAKE + 2) == q.MOEQ4_ERR_ALIGN
    assert _chunked(topk_ids=FAKE + 4) == q.MOEQ4_ERR_ALIGN
    assert _chunked(ws_bytes=1024) == q.MOEQ4_ERR_WORKSPACE
    assert _chunked(T=0, logits=None, X=None, out=None) == q.MOEQ4_OK   # nothing to do: no launch


def _ffn(**kw):
    a = dict(X=FAKE, T=8, H=256, I=128, E=16, k=2, gu_q=FAKE, gu_s=FAKE, gu_b=FAKE, dn_q=FAKE, dn_s=FAKE,
             dn_b=FAKE, sh_gu_q=None, sh_gu_s=None, sh_gu_b=None, sh_dn_q=None, sh_dn_s=None, sh_dn_b=None,
             topk_w=FAKE, perm=FAKE, blocks=FAKE, num_blocks=FAKE, max_blocks=1000, block_rows=16, out=FAKE,
             workspace=FAKE, ws_bytes=q.moe_expert_ffn_workspace_bytes(8, 256, 128, 16, 2, False), stream=None)
    a.update(kw)
    return q.lib().moe_expert_ffn_q4(*a.values())


def test_ffn_validation():
    assert q.moe_expert_ffn_workspace_bytes(4096, 2048, 512, 256, 8, True) >= 2 * 4096 * 8 * (512 + 2048)
    assert q.moe_expert_ffn_workspace_bytes(8, 100, 128, 16, 2, True) == 0   # H not a multiple of 64
    assert _ffn(I=96) == q.MOEQ4_ERR_SHAPE
    assert _ffn(k=17) == q.MOEQ4_ERR_SHAPE
    assert _ffn(block_rows=24) == q.MOEQ4_ERR_SHAPE
    assert _ffn(max_blocks=1) == q.MOEQ4_ERR_SHAPE
    assert _ffn(perm=None) == q.MOEQ4_ERR_NULL
    assert _ffn(sh_dn_b=FAKE) == q.MOEQ4_ERR_NULL                            # shared: all six or none
    assert _ffn(out=FAKE + 2) == q.MOEQ4_ERR_ALIGN
    assert _ffn(ws_bytes=64) == q.MOEQ4_ERR_WORKSPACE
    assert _ffn(T=0, X=None, out=None) == q.MOEQ4_OK                         # nothing to do: no launch


def test_calibrate_mfma_validation():
    L = q.lib()
    assert L.moe_calibrate_mfma(8, 10, None, None) == q.MOEQ4_ERR_NULL
    assert L.moe_calibrate_mfma(0, 10, FAKE, None) == q.MOEQ4_ERR_SHAPE
    assert L.moe_calibrate_mfma(8, -1, FAKE, None) == q.MOEQ4_ERR_SHAPE
    assert L.moe_calibrate_mfma(8, 10, FAKE + 4, None) == q.MOEQ4_ERR_ALIGN


def test_dequant_validation():
    L = q.lib()
    assert L.moe_dequant_q4(FAKE, FAKE, FAKE, 0, 32, 128, FAKE, None) == q.MOEQ4_ERR_SHAPE
    assert L.moe_dequant_q4(FAKE, FAKE, FAKE, 2, 24, 128, FAKE, None) == q.MOEQ4_ERR_SHAPE
    assert L.moe_dequant_q4(FAKE, FAKE, FAKE, 2, 32, 96, FAKE, None) == q.MOEQ4_ERR_SHAPE
    assert L.moe_dequant_q4(None, FAKE, FAKE, 2, 32, 128, FAKE, None) == q.MOEQ4_ERR_NULL
    assert L.moe_dequant_q4(FAKE, FAKE, FAKE, 2, 32, 128, None, None) == q.MOEQ4_ERR_NULL
    assert L.moe_dequant_q4(FAKE, FAKE, FAKE, 2, 32, 128, FAKE + 2, None) == q.MOEQ4_ERR_ALIGN


def test_layer_path_follows_row_count():
    # decode shapes: 8 of 256 experts, H=2048, I=512, shared expert
    E, k, H, I = 256, 8, 2048, 512
    assert q.moe_layer_ffn_path(1, E, k, H, I, True) == q.MOEQ4_PATH_DECODE
    for T in (2, 3, 5, 8):
        assert q.moe_layer_ffn_path(T, E, k, H, I, True) == q.MOEQ4_PATH_FEW_ROWS
    for T in (0, 9, 64, 512, 4096):
        assert q.moe_layer_ffn_path(T, E, k, H, I, True) == q.MOEQ4_PATH_PREFILL
    # past the decode kernels' limits (H > 8192) one row takes the few-row path;
    # past the few-row staging limit (T*(k+1)*I > 49152) rows take the routed path
    assert q.moe_layer_ffn_path(1, 16, 2, 16384, 128, False) == q.MOEQ4_PATH_FEW_ROWS
    assert q.moe_layer_ffn_path(8, 256, 8, 2048, 1024, True) == q.MOEQ4_PATH_PREFILL
    assert q.lib().moe_layer_ffn_path(-1, E, k, H, I, 1) == q.MOEQ4_ERR_SHAPE
    assert q.lib().moe_layer_ffn_path(4, E, 300, H, I, 1) < 0
    # the workspace is that of the path taken
    assert q.moe_layer_ffn_workspace_bytes(1, H, I, E, k, 0, True) == q.moe_decode_workspace_bytes(E, k, H, I, True)
    assert q.moe_layer_ffn_workspace_bytes(5, H, I, E, k, 0, True) == \
        q.moe_small_batch_workspace_bytes(5, E, k, H, I, True)
    assert q.moe_layer_ffn_workspace_bytes(64, H, I, E, k, 0, True) == \
        q.moe_prefill_ffn_chunked_workspace_bytes(64, 64, H, I, E, k, 0, True)


def test_layer_call_rejects_on_host():
    L = q.lib()
    args = [FAKE, FAKE, 4, 2048, 512, 256, 8] + [FAKE] * 6 + [None] * 6 + [0, None, None, FAKE, FAKE, 1 << 30, None]
    bad = list(args)
    bad[13] = FAKE                                   # one shared pointer of six
    assert L.moe_layer_ffn_q4(*bad) == q.MOEQ4_ERR_NULL
    bad = list(args)
    bad[19] = 24                                     # block_rows
    assert L.moe_layer_ffn_q4(*bad) == q.MOEQ4_ERR_SHAPE
    bad = list(args)
    bad[24] = 16                                     # workspace too small
    assert L.moe_layer_ffn_q4(*bad) == q.MOEQ4_ERR_WORKSPACE
    bad = list(args)
    bad[1] = FAKE + 8                                # misaligned X
    assert L.moe_layer_ffn_q4(*bad) == q.MOEQ4_ERR_ALIGN
