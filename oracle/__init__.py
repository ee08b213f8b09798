"""CPU oracle for the MoE routing + Q4 grouped-GEMM path (ctypes over moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the HIP library
and its Python binding never do.  It shares no code with the HIP path.

Follows Perplexity Engineering, "Optimizing on-device inference for Apple
Silicon" (2026), sections "Qwen creates three workload shapes", "Keep expert
routing on the GPU", "Dequantize weights during matrix multiplication" and
"Reduce intermediate and state traffic".  The readings of what the pages leave
open are listed at the top of moe_oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "_build", "libmoe_oracle.so")
_lib = None

_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_vp = ctypes.c_void_p
_int = ctypes.c_int


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc (-O2, OpenMP) into oracle/_build/."""
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        L.oracle_bf16_round.restype = ctypes.c_uint16
        L.oracle_bf16_round.argtypes = [ctypes.c_double]
        L.oracle_dequant_one.restype = ctypes.c_double
        L.oracle_dequant_one.argtypes = [ctypes.c_uint16, ctypes.c_uint16, _int]
        L.oracle_dequant_q4.argtypes = [_u8p, _u16p, _u16p, _int, _int, _f64p]
        L.oracle_topk_softmax.argtypes = [_vp, _int, _int, _int, _vp, _vp]
        L.oracle_route.argtypes = [_vp, _int, _int, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp]
        L.oracle_grouped_gemm_q4.argtypes = [_u16p, _int, _int, _int, _int, _int, _u8p, _u16p,
                                             _u16p, _i32p, _i32p, _f64p]
        L.oracle_expert_rows_q4.argtypes = [_u16p, _int, _int, _u8p, _u16p, _u16p, _i32p, _i32p,
                                            _int, _f64p]
        L.oracle_expert_ffn_q4.argtypes = [_u16p, _int, _int, _int, _int, _int,
                                           _u8p, _u16p, _u16p, _u8p, _u16p, _u16p,
                                           _vp, _vp, _vp, _vp, _vp, _vp,
                                           _i32p, _f64p, _i32p, _int, _f64p]
        L.oracle_expert_ffn_grouped_q4.argtypes = [_u16p, _int, _int, _int, _int, _int,
                                                   _u8p, _u16p, _u16p, _u8p, _u16p, _u16p,
                                                   _vp, _vp, _vp, _vp, _vp, _vp,
                                                   _i32p, _f64p, _f64p]
        L.oracle_num_threads.restype = _int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what} failed with status {rc}")


def num_threads() -> int:
    return lib().oracle_num_threads()


def bf16_round(x: float) -> int:
    """bf16 bit pattern nearest to the real x (ties to even)."""
    return int(lib().oracle_bf16_round(float(x)))


def dequant_one(scale_bits: int, bias_bits: int, code: int) -> float:
    return float(lib().oracle_dequant_one(scale_bits, bias_bits, code))


def dequant_q4(codes, scales, biases) -> np.ndarray:
    """Rebuilt [N, K] matrix (float64 holding bf16 values)."""
    codes = np.ascontiguousarray(codes, np.uint8)
    N, K2 = codes.shape
    W = np.empty((N, 2 * K2), np.float64)
    _check(lib().oracle_dequant_q4(codes, np.ascontiguousarray(scales, np.uint16),
                                   np.ascontiguousarray(biases, np.uint16), N, 2 * K2, W),
           "oracle_dequant_q4")
    return W


def topk_softmax(logits: np.ndarray, k: int):
    logits = np.ascontiguousarray(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    _check(lib().oracle_topk_softmax(_ptr(logits), T, E, k, _ptr(ids), _ptr(w)),
           "oracle_topk_softmax")
    return ids, w


def max_blocks_bound(A: int, E: int, block_rows: int) -> int:
    m = min(E, A)
    return (A + m * (block_rows - 1)) // block_rows


def route(ids: np.ndarray, E: int, block_rows: int) -> dict:
    ids = np.ascontiguousarray(ids, np.int32)
    T, k = ids.shape
    A = T * k
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(A, np.int32)
    inv_perm = np.empty(A, np.int32)
    blocks = np.zeros((max(1, max_blocks_bound(A, E, block_rows)), 4), np.int32)
    nb = np.zeros(1, np.int32)
    _check(lib().oracle_route(_ptr(ids), T, E, k, block_rows, _ptr(counts), _ptr(offsets),
                              _ptr(perm), _ptr(inv_perm), _ptr(blocks), _ptr(nb)), "oracle_route")
    n = int(nb[0])
    return dict(counts=counts, offsets=offsets, perm=perm, inv_perm=inv_perm,
                blocks=blocks[:n].copy(), num_blocks=n)


def grouped_gemm_q4(X, k, Wq, S, B, perm, offsets) -> np.ndarray:
    """Y [A, N] float64 in sorted (expert-grouped) order."""
    X = np.ascontiguousarray(X, np.uint16)
    T, K = X.shape
    E, N, _ = Wq.shape
    A = int(offsets[-1])
    Y = np.empty((A, N), np.float64)
    _check(lib().oracle_grouped_gemm_q4(X, T, K, N, E, k, np.ascontiguousarray(Wq, np.uint8),
                                        np.ascontiguousarray(S, np.uint16),
                                        np.ascontiguousarray(B, np.uint16),
                                        np.ascontiguousarray(perm, np.int32),
                                        np.ascontiguousarray(offsets, np.int32), Y),
           "oracle_grouped_gemm_q4")
    return Y


def expert_rows_q4(X, Wq, S, B, tokens, experts) -> np.ndarray:
    """Y [len(tokens), N]: row r = X[tokens[r]] times rebuilt W[experts[r]]^T."""
    X = np.ascontiguousarray(X, np.uint16)
    T, K = X.shape
    E, N, _ = Wq.shape
    tokens = np.ascontiguousarray(tokens, np.int32)
    experts = np.ascontiguousarray(experts, np.int32)
    Y = np.empty((len(tokens), N), np.float64)
    _check(lib().oracle_expert_rows_q4(X, K, N, np.ascontiguousarray(Wq, np.uint8),
                                       np.ascontiguousarray(S, np.uint16),
                                       np.ascontiguousarray(B, np.uint16), tokens, experts,
                                       len(tokens), Y), "oracle_expert_rows_q4")
    return Y


def expert_ffn_q4(X, ids, w, gu_q, gu_s, gu_b, dn_q, dn_s, dn_b, sh=None, tokens=None) -> np.ndarray:
    """out [len(tokens), H] float64 (all tokens when ``tokens`` is None).
    ``sh`` = (sh_gu_q, sh_gu_s, sh_gu_b, sh_dn_q, sh_dn_s, sh_dn_b) or None."""
    X = np.ascontiguousarray(X, np.uint16)
    T, H = X.shape
    E, I2, _ = gu_q.shape
    I = I2 // 2
    k = ids.shape[1]
    if tokens is None:
        tokens = np.arange(T, dtype=np.int32)
    tokens = np.ascontiguousarray(tokens, np.int32)
    out = np.empty((len(tokens), H), np.float64)
    shp = [None] * 6 if sh is None else [np.ascontiguousarray(a) for a in sh]
    _check(lib().oracle_expert_ffn_q4(
        X, T, H, I, E, k,
        np.ascontiguousarray(gu_q, np.uint8), np.ascontiguousarray(gu_s, np.uint16),
        np.ascontiguousarray(gu_b, np.uint16), np.ascontiguousarray(dn_q, np.uint8),
        np.ascontiguousarray(dn_s, np.uint16), np.ascontiguousarray(dn_b, np.uint16),
        *[_ptr(a) for a in shp],
        np.ascontiguousarray(ids, np.int32), np.ascontiguousarray(w, np.float64), tokens,
        len(tokens), out), "oracle_expert_ffn_q4")
    return out


def expert_ffn_grouped_q4(X, ids, w, gu_q, gu_s, gu_b, dn_q, dn_s, dn_b, sh=None) -> np.ndarray:
    """out [T, H] float64 for every token, expert by expert: each expert's
    matrices are rebuilt once and applied to all rows routed to it.  Bit for
    bit the same values as expert_ffn_q4 (same term order), in a fraction of
    its time at full size."""
    X = np.ascontiguousarray(X, np.uint16)
    T, H = X.shape
    E, I2, _ = gu_q.shape
    I = I2 // 2
    k = ids.shape[1]
    out = np.empty((T, H), np.float64)
    shp = [None] * 6 if sh is None else [np.ascontiguousarray(a) for a in sh]
    _check(lib().oracle_expert_ffn_grouped_q4(
        X, T, H, I, E, k,
        np.ascontiguousarray(gu_q, np.uint8), np.ascontiguousarray(gu_s, np.uint16),
        np.ascontiguousarray(gu_b, np.uint16), np.ascontiguousarray(dn_q, np.uint8),
        np.ascontiguousarray(dn_s, np.uint16), np.ascontiguousarray(dn_b, np.uint16),
        *[_ptr(a) for a in shp],
        np.ascontiguousarray(ids, np.int32), np.ascontiguousarray(w, np.float64), out),
        "oracle_expert_ffn_grouped_q4")
    return out
