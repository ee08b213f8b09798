"""Python binding of libmoeq4 (MoE routing + group-wise affine 4-bit grouped GEMM, gfx950).

Argument marshalling only: every step runs in the HIP kernels of the shared
library.  Functions take torch tensors (device memory) or raw integer device
addresses and pass their pointers, with the caller's current HIP stream,
straight to the C ABI declared in include/moeq4.h.  There is no fallback: if
the library has not been built, importing the binding raises.
"""
from __future__ import annotations

import ctypes
import os

# The HIP runtime that torch loads must be the only one in the process: torch
# hands out its streams and device pointers, and a second copy of
# libamdhip64 would not know them.  Loading torch first makes libmoeq4's
# dependency on libamdhip64.so.7 bind to torch's copy.
import torch  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
# The in-tree build, unless MOEQ4_LIB names another build of the same library
# (an installed copy, or a build of other sources to compare against).
LIB_PATH = os.environ.get("MOEQ4_LIB") or os.path.join(_PKG, "_lib", "libmoeq4.so")

MOEQ4_OK = 0
MOEQ4_ERR_NULL = -1
MOEQ4_ERR_SHAPE = -2
MOEQ4_ERR_ALIGN = -3
MOEQ4_ERR_WORKSPACE = -4
MOEQ4_ERR_UNSUPPORTED = -5
MOEQ4_ERR_HIP = -6
MOEQ4_MAX_EXPERTS = 1024
MOEQ4_MAX_TOPK = 64
MOEQ4_SMALL_MAX_T = 8
MOEQ4_ROUTE_IN_LAUNCH_MAX = 4096
MOEQ4_DECODE_SCRATCH_BYTES = 256 * 1024
MOEQ4_PATH_DECODE = 1
MOEQ4_PATH_FEW_ROWS = 2
MOEQ4_PATH_PREFILL = 3

_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/moeq4.h
SIGNATURES = {
    "moe_strerror": (ctypes.c_char_p, [_i]),
    "moe_last_error_detail": (ctypes.c_char_p, []),
    "moe_default_block_rows": (_i, [_i, _i, _i]),
    "moe_max_blocks": (_i, [_i, _i, _i, _i]),
    "moe_route_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "moe_route": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_topk_softmax": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp]),
    "moe_prepack_q4": (_i, [_vp, _vp, _vp, _i, _i, _i, _vp, _vp, _vp, _vp]),
    "moe_grouped_gemm_q4": (_i, [_vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i,
                                 _vp, _vp]),
    "moe_route_grouped_gemm_q4": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _i] + [_vp] * 8 + [_i, _vp, _vp,
                                                                                          _sz, _vp]),
    "moe_expert_ffn_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "moe_expert_ffn_q4": (_i, [_vp, _i, _i, _i, _i, _i] + [_vp] * 12 + [_vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _sz,
                                                                       _vp]),
    "moe_decode_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "moe_decode_ffn_q4": (_i, [_vp, _vp, _i, _i, _i, _i] + [_vp] * 12 + [_vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_prefill_ffn_chunked_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "moe_prefill_ffn_chunked_q4": (_i, [_vp, _vp, _i, _i, _i, _i, _i] + [_vp] * 12 + [_i, _i, _vp, _vp, _vp, _vp,
                                                                                      _sz, _vp]),
    "moe_small_batch_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "moe_small_batch_ffn_q4": (_i, [_vp, _vp, _i, _i, _i, _i, _i] + [_vp] * 12 + [_vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_calibrate_mfma": (_i, [_i, _i, _vp, _vp]),
    "moe_dequant_q4": (_i, [_vp, _vp, _vp, _i, _i, _i, _vp, _vp]),
    "moe_decode_ffn_q4_noalloc": (_i, [_vp, _vp, _i, _i, _i, _i] + [_vp] * 12 + [_vp, _vp, _vp, _vp]),
    "moe_layer_ffn_path": (_i, [_i, _i, _i, _i, _i, _i]),
    "moe_layer_ffn_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "moe_layer_ffn_q4": (_i, [_vp, _vp, _i, _i, _i, _i, _i] + [_vp] * 12 + [_i, _vp, _vp, _vp, _vp, _sz, _vp]),
}


class MoeQ4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        detail = lib().moe_last_error_detail().decode() if status == MOEQ4_ERR_HIP else ""
        super().__init__(f"{fn}: {strerror(status)} (status {status}) {detail}".rstrip())
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libmoeq4 is not built ({LIB_PATH} missing); run `python -m quantized_grouped_gemm_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = None


def lib():
    """The loaded libmoeq4 (loaded on first use; raises ImportError if it is not built)."""
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def strerror(status: int) -> str:
    return lib().moe_strerror(int(status)).decode()


def _p(x):
    """Device address of a torch tensor, an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ok(fn, status):
    if status != MOEQ4_OK:
        raise MoeQ4Error(fn, status)


def moe_default_block_rows(T: int, E: int, k: int) -> int:
    r = lib().moe_default_block_rows(T, E, k)
    _ok("moe_default_block_rows", min(r, 0))
    return r


def moe_max_blocks(T: int, E: int, k: int, block_rows: int = 0) -> int:
    r = lib().moe_max_blocks(T, E, k, block_rows)
    _ok("moe_max_blocks", min(r, 0))
    return r


def moe_route_workspace_bytes(T: int, E: int, k: int, block_rows: int = 0) -> int:
    return int(lib().moe_route_workspace_bytes(T, E, k, block_rows))


def moe_route(logits, T, E, k, block_rows, topk_ids, topk_w, counts, offsets, perm, inv_perm,
              blocks, num_blocks, workspace, ws_bytes, stream=None):
    _ok("moe_route", lib().moe_route(
        _p(logits), T, E, k, block_rows, _p(topk_ids), _p(topk_w), _p(counts), _p(offsets),
        _p(perm), _p(inv_perm), _p(blocks), _p(num_blocks), _p(workspace), int(ws_bytes),
        _stream(stream)))


def moe_topk_softmax(logits, T, E, k, topk_ids, topk_w, stream=None):
    _ok("moe_topk_softmax", lib().moe_topk_softmax(_p(logits), T, E, k, _p(topk_ids), _p(topk_w),
                                                   _stream(stream)))


def moe_prepack_q4(codes, scales, biases, E, N, K, codes_t, scales_t, biases_t, stream=None):
    _ok("moe_prepack_q4", lib().moe_prepack_q4(
        _p(codes), _p(scales), _p(biases), E, N, K, _p(codes_t), _p(scales_t), _p(biases_t),
        _stream(stream)))


def moe_grouped_gemm_q4(X, T, K, N, E, k, codes_t, scales_t, biases_t, perm, blocks, num_blocks,
                        max_blocks, block_rows, Y, stream=None):
    _ok("moe_grouped_gemm_q4", lib().moe_grouped_gemm_q4(
        _p(X), T, K, N, E, k, _p(codes_t), _p(scales_t), _p(biases_t), _p(perm), _p(blocks),
        _p(num_blocks), max_blocks, block_rows, _p(Y), _stream(stream)))


def moe_route_grouped_gemm_q4(logits, X, T, K, N, E, k, codes_t, scales_t, biases_t, block_rows, topk_ids,
                              topk_w, counts, offsets, perm, inv_perm, blocks, num_blocks, max_blocks, Y,
                              workspace, ws_bytes, stream=None):
    _ok("moe_route_grouped_gemm_q4", lib().moe_route_grouped_gemm_q4(
        _p(logits), _p(X), T, K, N, E, k, _p(codes_t), _p(scales_t), _p(biases_t), block_rows, _p(topk_ids),
        _p(topk_w), _p(counts), _p(offsets), _p(perm), _p(inv_perm), _p(blocks), _p(num_blocks), max_blocks,
        _p(Y), _p(workspace), int(ws_bytes), _stream(stream)))


def moe_expert_ffn_workspace_bytes(T: int, H: int, I: int, E: int, k: int, shared: bool) -> int:
    return int(lib().moe_expert_ffn_workspace_bytes(T, H, I, E, k, int(bool(shared))))


def moe_expert_ffn_q4(X, T, H, I, E, k, gu_codes_t, gu_scales_t, gu_biases_t, dn_codes_t, dn_scales_t,
                      dn_biases_t, sh_gu_codes_t, sh_gu_scales_t, sh_gu_biases_t, sh_dn_codes_t, sh_dn_scales_t,
                      sh_dn_biases_t, topk_w, perm, blocks, num_blocks, max_blocks, block_rows, out, workspace,
                      ws_bytes, stream=None):
    _ok("moe_expert_ffn_q4", lib().moe_expert_ffn_q4(
        _p(X), T, H, I, E, k, _p(gu_codes_t), _p(gu_scales_t), _p(gu_biases_t), _p(dn_codes_t), _p(dn_scales_t),
        _p(dn_biases_t), _p(sh_gu_codes_t), _p(sh_gu_scales_t), _p(sh_gu_biases_t), _p(sh_dn_codes_t),
        _p(sh_dn_scales_t), _p(sh_dn_biases_t), _p(topk_w), _p(perm), _p(blocks), _p(num_blocks), max_blocks,
        block_rows, _p(out), _p(workspace), int(ws_bytes), _stream(stream)))


def moe_decode_workspace_bytes(E: int, k: int, H: int, I: int, shared: bool) -> int:
    return int(lib().moe_decode_workspace_bytes(E, k, H, I, int(bool(shared))))


def moe_decode_ffn_q4(logits, x, E, k, H, I, gu_codes_t, gu_scales_t, gu_biases_t, dn_codes_t,
                      dn_scales_t, dn_biases_t, sh_gu_codes_t, sh_gu_scales_t, sh_gu_biases_t,
                      sh_dn_codes_t, sh_dn_scales_t, sh_dn_biases_t, topk_ids, topk_w, out, workspace,
                      ws_bytes, stream=None):
    _ok("moe_decode_ffn_q4", lib().moe_decode_ffn_q4(
        _p(logits), _p(x), E, k, H, I, _p(gu_codes_t), _p(gu_scales_t), _p(gu_biases_t), _p(dn_codes_t),
        _p(dn_scales_t), _p(dn_biases_t), _p(sh_gu_codes_t), _p(sh_gu_scales_t), _p(sh_gu_biases_t),
        _p(sh_dn_codes_t), _p(sh_dn_scales_t), _p(sh_dn_biases_t), _p(topk_ids), _p(topk_w), _p(out),
        _p(workspace), int(ws_bytes), _stream(stream)))


def moe_decode_ffn_q4_noalloc(logits, x, E, k, H, I, gu_codes_t, gu_scales_t, gu_biases_t, dn_codes_t,
                              dn_scales_t, dn_biases_t, sh_gu_codes_t, sh_gu_scales_t, sh_gu_biases_t,
                              sh_dn_codes_t, sh_dn_scales_t, sh_dn_biases_t, topk_ids, topk_w, out, stream=None):
    _ok("moe_decode_ffn_q4_noalloc", lib().moe_decode_ffn_q4_noalloc(
        _p(logits), _p(x), E, k, H, I, _p(gu_codes_t), _p(gu_scales_t), _p(gu_biases_t), _p(dn_codes_t),
        _p(dn_scales_t), _p(dn_biases_t), _p(sh_gu_codes_t), _p(sh_gu_scales_t), _p(sh_gu_biases_t),
        _p(sh_dn_codes_t), _p(sh_dn_scales_t), _p(sh_dn_biases_t), _p(topk_ids), _p(topk_w), _p(out),
        _stream(stream)))


def moe_prefill_ffn_chunked_workspace_bytes(T: int, chunk_tokens: int, H: int, I: int, E: int, k: int,
                                            block_rows: int, shared: bool) -> int:
    return int(lib().moe_prefill_ffn_chunked_workspace_bytes(T, chunk_tokens, H, I, E, k, block_rows,
                                                             int(bool(shared))))


def moe_prefill_ffn_chunked_q4(logits, X, T, H, I, E, k, gu_codes_t, gu_scales_t, gu_biases_t, dn_codes_t,
                               dn_scales_t, dn_biases_t, sh_gu_codes_t, sh_gu_scales_t, sh_gu_biases_t,
                               sh_dn_codes_t, sh_dn_scales_t, sh_dn_biases_t, chunk_tokens, block_rows, topk_ids,
                               topk_w, out, workspace, ws_bytes, stream=None):
    _ok("moe_prefill_ffn_chunked_q4", lib().moe_prefill_ffn_chunked_q4(
        _p(logits), _p(X), T, H, I, E, k, _p(gu_codes_t), _p(gu_scales_t), _p(gu_biases_t), _p(dn_codes_t),
        _p(dn_scales_t), _p(dn_biases_t), _p(sh_gu_codes_t), _p(sh_gu_scales_t), _p(sh_gu_biases_t),
        _p(sh_dn_codes_t), _p(sh_dn_scales_t), _p(sh_dn_biases_t), int(chunk_tokens), int(block_rows),
        _p(topk_ids), _p(topk_w), _p(out), _p(workspace), int(ws_bytes), _stream(stream)))


def moe_small_batch_workspace_bytes(T: int, E: int, k: int, H: int, I: int, shared: bool) -> int:
    return int(lib().moe_small_batch_workspace_bytes(T, E, k, H, I, int(bool(shared))))


def moe_small_batch_ffn_q4(logits, x, T, E, k, H, I, gu_codes_t, gu_scales_t, gu_biases_t, dn_codes_t,
                           dn_scales_t, dn_biases_t, sh_gu_codes_t, sh_gu_scales_t, sh_gu_biases_t,
                           sh_dn_codes_t, sh_dn_scales_t, sh_dn_biases_t, topk_ids, topk_w, out, workspace,
                           ws_bytes, stream=None):
    _ok("moe_small_batch_ffn_q4", lib().moe_small_batch_ffn_q4(
        _p(logits), _p(x), T, E, k, H, I, _p(gu_codes_t), _p(gu_scales_t), _p(gu_biases_t), _p(dn_codes_t),
        _p(dn_scales_t), _p(dn_biases_t), _p(sh_gu_codes_t), _p(sh_gu_scales_t), _p(sh_gu_biases_t),
        _p(sh_dn_codes_t), _p(sh_dn_scales_t), _p(sh_dn_biases_t), _p(topk_ids), _p(topk_w), _p(out),
        _p(workspace), int(ws_bytes), _stream(stream)))


def moe_dequant_q4(codes_t, scales_t, biases_t, E, N, K, out, stream=None):
    _ok("moe_dequant_q4", lib().moe_dequant_q4(_p(codes_t), _p(scales_t), _p(biases_t), E, N, K, _p(out),
                                               _stream(stream)))


def dequant(packed, E: int, N: int, K: int, out=None, stream=None):
    """Every weight rebuilt as bf16 into a [E, N, K] int16 (bf16 bits) device tensor."""
    ct, st, bt = packed
    if out is None:
        out = torch.empty((E, N, K), dtype=torch.int16, device=ct.device)
    moe_dequant_q4(ct, st, bt, E, N, K, out, stream)
    return out


def moe_calibrate_mfma(workgroups, iters, out, stream=None):
    _ok("moe_calibrate_mfma", lib().moe_calibrate_mfma(int(workgroups), int(iters), _p(out), _stream(stream)))


# ---------------------------------------------------------------- plumbing --
# Device buffers come from torch (memory and streams only).

def alloc_route(T: int, E: int, k: int, block_rows: int = 0, device="cuda"):
    """Output and workspace tensors for moe_route / moe_grouped_gemm_q4."""
    bm = block_rows or moe_default_block_rows(T, E, k)
    mb = moe_max_blocks(T, E, k, bm)
    ws = moe_route_workspace_bytes(T, E, k, bm)
    i32 = dict(dtype=torch.int32, device=device)
    A = T * k
    return dict(
        block_rows=bm, max_blocks=mb,
        topk_ids=torch.empty(max(A, 1), **i32), topk_w=torch.empty(max(A, 1), dtype=torch.float32, device=device),
        counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
        perm=torch.empty(max(A, 1), **i32), inv_perm=torch.empty(max(A, 1), **i32),
        blocks=torch.empty(max(mb, 1) * 4, **i32), num_blocks=torch.empty(4, **i32),
        workspace=torch.empty(max(ws, 1), dtype=torch.uint8, device=device), ws_bytes=ws,
    )


def route(logits, k: int, block_rows: int = 0, bufs=None, stream=None):
    """Runs moe_route on a [T, E] float32 device tensor; returns the buffer dict."""
    T, E = logits.shape
    b = bufs or alloc_route(T, E, k, block_rows, device=logits.device)
    moe_route(logits, T, E, k, b["block_rows"], b["topk_ids"], b["topk_w"], b["counts"], b["offsets"],
              b["perm"], b["inv_perm"], b["blocks"], b["num_blocks"], b["workspace"], b["ws_bytes"],
              stream)
    return b


def topk_softmax(logits, k: int, bufs, stream=None):
    """moe_topk_softmax of [T, E] float32 logits into bufs["topk_ids"] / bufs["topk_w"] (alloc_route)."""
    T, E = logits.shape
    moe_topk_softmax(logits, T, E, k, bufs["topk_ids"], bufs["topk_w"], stream)
    return bufs


def prepack(codes, scales, biases, stream=None):
    """Tiled copies (moe_prepack_q4) of [E, N, K/2] codes and [E, N, K/64] scales/biases."""
    E, N, K2 = codes.shape
    out = (torch.empty_like(codes), torch.empty_like(scales), torch.empty_like(biases))
    moe_prepack_q4(codes, scales, biases, E, N, 2 * K2, *out, stream)
    return out


def grouped_gemm_q4(X, k, packed, rt, Y=None, stream=None):
    """Y [T*k, N] bf16 bit patterns (int16 storage) in sorted order for routing tables ``rt``;
    ``packed`` = (codes_t, scales_t, biases_t) from prepack()."""
    codes_t, scales_t, biases_t = packed
    T, K = X.shape
    E, N, _ = codes_t.shape
    if Y is None:
        Y = torch.empty((max(T * k, 1), N), dtype=torch.int16, device=X.device)
    moe_grouped_gemm_q4(X, T, K, N, E, k, codes_t, scales_t, biases_t, rt["perm"], rt["blocks"],
                        rt["num_blocks"], rt["max_blocks"], rt["block_rows"], Y, stream)
    return Y


def route_grouped_gemm_q4(logits, X, k, packed, rt, Y=None, stream=None):
    """moe_route_grouped_gemm_q4: routing of [T, E] logits into the tables of ``rt`` (alloc_route) and
    Y [T*k, N] bf16 bit patterns in sorted order, in one call; returns Y."""
    codes_t, scales_t, biases_t = packed
    T, K = X.shape
    E, N, _ = codes_t.shape
    if Y is None:
        Y = torch.empty((max(T * k, 1), N), dtype=torch.int16, device=X.device)
    moe_route_grouped_gemm_q4(logits, X, T, K, N, E, k, codes_t, scales_t, biases_t, rt["block_rows"],
                              rt["topk_ids"], rt["topk_w"], rt["counts"], rt["offsets"], rt["perm"],
                              rt["inv_perm"], rt["blocks"], rt["num_blocks"], rt["max_blocks"], Y,
                              rt["workspace"], rt["ws_bytes"], stream)
    return Y


def alloc_decode(E: int, k: int, H: int, I: int, shared: bool = True, device="cuda"):
    """Output and workspace tensors for moe_decode_ffn_q4."""
    ws = moe_decode_workspace_bytes(E, k, H, I, shared)
    if ws == 0:
        raise MoeQ4Error("moe_decode_workspace_bytes", MOEQ4_ERR_SHAPE)
    return dict(
        out=torch.empty(H, dtype=torch.int16, device=device),
        topk_ids=torch.empty(k, dtype=torch.int32, device=device),
        topk_w=torch.empty(k, dtype=torch.float32, device=device),
        workspace=torch.empty(ws, dtype=torch.uint8, device=device), ws_bytes=ws)


def decode_ffn(logits, x, k: int, gu, dn, sh_gu=None, sh_dn=None, bufs=None, stream=None):
    """One batch-1 decode step (moe_decode_ffn_q4).  ``logits`` float32 [E],
    ``x`` bf16 bits [H]; ``gu`` / ``dn`` = prepack() tuples of the [E, 2I, H] and
    [E, H, I] matrices; ``sh_gu`` / ``sh_dn`` the shared expert's ([1, ...]) or
    None.  Returns the buffer dict (``out`` holds bf16 bits [H])."""
    E = logits.shape[-1]
    H = x.shape[-1]
    I = gu[0].shape[1] // 2
    shared = sh_gu is not None
    b = bufs or alloc_decode(E, k, H, I, shared, device=x.device)
    sg = sh_gu if shared else (None, None, None)
    sd = sh_dn if shared else (None, None, None)
    moe_decode_ffn_q4(logits, x, E, k, H, I, *gu, *dn, *sg, *sd, b["topk_ids"], b["topk_w"], b["out"],
                      b["workspace"], b["ws_bytes"], stream)
    return b


def alloc_chunked(T: int, chunk_tokens: int, H: int, I: int, E: int, k: int, block_rows: int = 0,
                  shared: bool = True, device="cuda"):
    """Output and workspace tensors for moe_prefill_ffn_chunked_q4."""
    ws = moe_prefill_ffn_chunked_workspace_bytes(T, chunk_tokens, H, I, E, k, block_rows, shared)
    if ws == 0:
        raise MoeQ4Error("moe_prefill_ffn_chunked_workspace_bytes", MOEQ4_ERR_SHAPE)
    return dict(
        out=torch.empty(max(T, 1), H, dtype=torch.int16, device=device),
        topk_ids=torch.empty(max(T, 1), k, dtype=torch.int32, device=device),
        topk_w=torch.empty(max(T, 1), k, dtype=torch.float32, device=device),
        workspace=torch.empty(ws, dtype=torch.uint8, device=device), ws_bytes=ws,
        chunk_tokens=chunk_tokens, block_rows=block_rows)


def prefill_ffn_chunked(logits, X, k: int, gu, dn, sh_gu=None, sh_dn=None, chunk_tokens: int = 1024,
                        block_rows: int = 0, bufs=None, stream=None):
    """The routed FFN (+ shared expert) of T tokens in chunks of ``chunk_tokens``
    (moe_prefill_ffn_chunked_q4).  ``logits`` float32 [T, E], ``X`` bf16 bits
    [T, H]; weights as expert_ffn.  Returns the buffer dict (``out`` bf16 bits
    [T, H], ``topk_ids`` / ``topk_w`` [T, k])."""
    T, E = logits.shape
    H = X.shape[-1]
    I = gu[0].shape[1] // 2
    shared = sh_gu is not None
    b = bufs or alloc_chunked(T, chunk_tokens, H, I, E, k, block_rows, shared, device=X.device)
    sg = sh_gu if shared else (None, None, None)
    sd = sh_dn if shared else (None, None, None)
    moe_prefill_ffn_chunked_q4(logits, X, T, H, I, E, k, *gu, *dn, *sg, *sd, b["chunk_tokens"], b["block_rows"],
                               b["topk_ids"], b["topk_w"], b["out"], b["workspace"], b["ws_bytes"], stream)
    return b


def alloc_small(T: int, E: int, k: int, H: int, I: int, shared: bool = True, device="cuda"):
    """Output and workspace tensors for moe_small_batch_ffn_q4."""
    ws = moe_small_batch_workspace_bytes(T, E, k, H, I, shared)
    if ws == 0:
        raise MoeQ4Error("moe_small_batch_workspace_bytes", MOEQ4_ERR_SHAPE)
    return dict(
        out=torch.empty(T, H, dtype=torch.int16, device=device),
        topk_ids=torch.empty(T, k, dtype=torch.int32, device=device),
        topk_w=torch.empty(T, k, dtype=torch.float32, device=device),
        workspace=torch.empty(ws, dtype=torch.uint8, device=device), ws_bytes=ws)


def small_batch_ffn(logits, x, k: int, gu, dn, sh_gu=None, sh_dn=None, bufs=None, stream=None):
    """The layer for a few tokens (moe_small_batch_ffn_q4).  ``logits`` float32
    [T, E], ``x`` bf16 bits [T, H], 1 <= T <= 8; weights as decode_ffn.  Returns
    the buffer dict (``out`` holds bf16 bits [T, H])."""
    T, E = logits.shape
    H = x.shape[-1]
    I = gu[0].shape[1] // 2
    shared = sh_gu is not None
    b = bufs or alloc_small(T, E, k, H, I, shared, device=x.device)
    sg = sh_gu if shared else (None, None, None)
    sd = sh_dn if shared else (None, None, None)
    moe_small_batch_ffn_q4(logits, x, T, E, k, H, I, *gu, *dn, *sg, *sd, b["topk_ids"], b["topk_w"], b["out"],
                           b["workspace"], b["ws_bytes"], stream)
    return b


def alloc_ffn(T: int, H: int, I: int, E: int, k: int, shared: bool = True, device="cuda"):
    """Output and workspace tensors for moe_expert_ffn_q4."""
    ws = moe_expert_ffn_workspace_bytes(T, H, I, E, k, shared)
    return dict(out=torch.empty((max(T, 1), H), dtype=torch.int16, device=device),
                workspace=torch.empty(max(ws, 1), dtype=torch.uint8, device=device), ws_bytes=ws)


def expert_ffn(X, k: int, rt, gu, dn, sh_gu=None, sh_dn=None, bufs=None, stream=None):
    """The expert FFNs of a batch (moe_expert_ffn_q4).  ``X`` bf16 bits [T, H];
    ``rt`` the routing buffers of route(); ``gu`` / ``dn`` = prepack() tuples of
    the [E, 2I, H] and [E, H, I] matrices; ``sh_gu`` / ``sh_dn`` the shared
    expert's or None.  Returns the buffer dict (``out`` holds bf16 bits [T, H])."""
    T, H = X.shape
    E, I2, _ = gu[0].shape
    I = I2 // 2
    shared = sh_gu is not None
    b = bufs or alloc_ffn(T, H, I, E, k, shared, device=X.device)
    sg = sh_gu if shared else (None, None, None)
    sd = sh_dn if shared else (None, None, None)
    moe_expert_ffn_q4(X, T, H, I, E, k, *gu, *dn, *sg, *sd, rt["topk_w"], rt["perm"], rt["blocks"],
                      rt["num_blocks"], rt["max_blocks"], rt["block_rows"], b["out"], b["workspace"],
                      b["ws_bytes"], stream)
    return b


def moe_layer_ffn_path(T: int, E: int, k: int, H: int, I: int, shared: bool) -> int:
    r = lib().moe_layer_ffn_path(T, E, k, H, I, int(bool(shared)))
    _ok("moe_layer_ffn_path", min(r, 0))
    return r


def moe_layer_ffn_workspace_bytes(T: int, H: int, I: int, E: int, k: int, block_rows: int, shared: bool) -> int:
    return int(lib().moe_layer_ffn_workspace_bytes(T, H, I, E, k, block_rows, int(bool(shared))))


def moe_layer_ffn_q4(logits, X, T, H, I, E, k, gu_codes_t, gu_scales_t, gu_biases_t, dn_codes_t, dn_scales_t,
                     dn_biases_t, sh_gu_codes_t, sh_gu_scales_t, sh_gu_biases_t, sh_dn_codes_t, sh_dn_scales_t,
                     sh_dn_biases_t, block_rows, topk_ids, topk_w, out, workspace, ws_bytes, stream=None):
    _ok("moe_layer_ffn_q4", lib().moe_layer_ffn_q4(
        _p(logits), _p(X), T, H, I, E, k, _p(gu_codes_t), _p(gu_scales_t), _p(gu_biases_t), _p(dn_codes_t),
        _p(dn_scales_t), _p(dn_biases_t), _p(sh_gu_codes_t), _p(sh_gu_scales_t), _p(sh_gu_biases_t),
        _p(sh_dn_codes_t), _p(sh_dn_scales_t), _p(sh_dn_biases_t), int(block_rows), _p(topk_ids), _p(topk_w),
        _p(out), _p(workspace), int(ws_bytes), _stream(stream)))


def alloc_layer(T: int, H: int, I: int, E: int, k: int, block_rows: int = 0, shared: bool = True, device="cuda"):
    """Output and workspace tensors for moe_layer_ffn_q4."""
    ws = moe_layer_ffn_workspace_bytes(T, H, I, E, k, block_rows, shared)
    if ws == 0 and T > 0:
        raise MoeQ4Error("moe_layer_ffn_workspace_bytes", MOEQ4_ERR_SHAPE)
    return dict(
        out=torch.empty((max(T, 1), H), dtype=torch.int16, device=device),
        topk_ids=torch.empty((max(T, 1), k), dtype=torch.int32, device=device),
        topk_w=torch.empty((max(T, 1), k), dtype=torch.float32, device=device),
        workspace=torch.empty(max(ws, 1), dtype=torch.uint8, device=device), ws_bytes=ws,
        block_rows=block_rows, path=moe_layer_ffn_path(T, E, k, H, I, shared))


def layer_ffn(logits, X, k: int, gu, dn, sh_gu=None, sh_dn=None, block_rows: int = 0, bufs=None, stream=None):
    """The MoE layer from logits to output (moe_layer_ffn_q4), its path chosen
    from T.  ``logits`` float32 [T, E], ``X`` bf16 bits [T, H]; weights as
    expert_ffn.  Returns the buffer dict (``out`` bf16 bits [T, H], ``path``)."""
    T, E = logits.shape
    H = X.shape[-1]
    I = gu[0].shape[1] // 2
    shared = sh_gu is not None
    b = bufs or alloc_layer(T, H, I, E, k, block_rows, shared, device=X.device)
    sg = sh_gu if shared else (None, None, None)
    sd = sh_dn if shared else (None, None, None)
    moe_layer_ffn_q4(logits, X, T, H, I, E, k, *gu, *dn, *sg, *sd, b["block_rows"], b["topk_ids"], b["topk_w"],
                     b["out"], b["workspace"], b["ws_bytes"], stream)
    return b
