"""Seeded synthetic inputs for the MoE routing + Q4 grouped-GEMM path.

This module draws random inputs and nothing else: it holds none of the
method's arithmetic (no top-k, no routing, no dequantisation, no matmul).
Both the CPU oracle (``oracle/``) and the HIP library receive the arrays it
returns, so the two sides always see identical bytes.

Every array comes from numpy's PCG64 ``default_rng([config_id, stream, step])``.
Streams: 0 logits, 1 activations, 2 codes, 3 scales, 4 bias noise,
5 shared-expert weights, 6 skew bias table.

Storage formats (the inputs the path consumes):

* logits: float32 ``[T, E]``.
* activations ``X``: bf16 bit patterns (uint16) ``[T, K]``.
* a group-wise affine 4-bit matrix ``[N, K]`` is three arrays:
  ``codes`` uint8 ``[N, K/2]`` (two 4-bit codes per byte, the lower K index in
  the low nibble), ``scales`` and ``biases`` bf16 bit patterns ``[N, K/64]``.
  Codes uniform on 0..15, packed two per byte, are exactly uniform bytes, so
  the generator draws bytes directly and never packs anything.

The five named workloads mirror the shapes of the expert layers in the pages
(Perplexity, "Optimizing on-device inference for Apple Silicon": section
"Qwen creates three workload shapes": 8 of 256 experts plus one shared expert;
section "Dequantize weights during matrix multiplication": 64 weights per group
with a bf16 scale and bias).  The hidden/intermediate sizes are not on the
pages; they are the ones of the workloads below.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

GROUP = 64

# stream ids
S_LOGITS, S_ACTS, S_CODES, S_SCALES, S_BIAS, S_SHARED, S_SKEW = range(7)


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    T: int
    E: int
    k: int
    K: int            # input dim of the single projection, or hidden size H for the FFN
    N: int            # output dim of the single projection, or intermediate size I for the FFN
    ffn: bool = False  # gate+up [2N x K] -> SwiGLU -> down [K x N], plus a shared expert
    skew_alpha: float = 0.0   # logits += alpha * ln p_e, p_e ~ (e+1)^-zipf_s
    zipf_s: float = 1.1
    steps: int = 1


WORKLOADS = {
    1: Workload(1, "tiny T=64 E=16 k=2 K=256 N=128", T=64, E=16, k=2, K=256, N=128),
    2: Workload(2, "prefill chunk T=512 E=256 k=8 K=2048 N=512", T=512, E=256, k=8, K=2048, N=512),
    3: Workload(3, "expert FFN + shared T=4096 E=256 k=8 H=2048 I=512", T=4096, E=256, k=8,
                K=2048, N=512, ffn=True),
    4: Workload(4, "skewed routing T=16384 E=256 k=8 K=2048 N=512 zipf 1.1", T=16384, E=256, k=8,
                K=2048, N=512, skew_alpha=0.94),
    5: Workload(5, "batch-1 decode T=1 E=256 k=8 H=2048 I=512 + shared", T=1, E=256, k=8,
                K=2048, N=512, ffn=True, steps=1000),
}


def rng(cid: int, stream: int, step: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(cid), int(stream), int(step)])


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def gen_logits(cid: int, T: int, E: int, step: int = 0, skew_alpha: float = 0.0,
               zipf_s: float = 1.1) -> np.ndarray:
    """Router logits ~ N(0,1), optionally plus a per-expert Zipf bias alpha*ln p_e."""
    x = rng(cid, S_LOGITS, step).standard_normal((T, E), dtype=np.float32)
    if skew_alpha:
        p = (np.arange(1, E + 1, dtype=np.float64)) ** (-zipf_s)
        p /= p.sum()
        x = (x + (skew_alpha * np.log(p)).astype(np.float32)[None, :]).astype(np.float32)
    return np.ascontiguousarray(x)


def gen_acts(cid: int, T: int, K: int, step: int = 0) -> np.ndarray:
    """Activations bf16(N(0,1)) as uint16 bit patterns [T, K]."""
    return to_bf16_bits(rng(cid, S_ACTS, step).standard_normal((T, K), dtype=np.float32))


def gen_q4(cid: int, nmat: int, N: int, K: int, step: int = 0,
           shared: bool = False, scale_sigma: float = 0.02, bias_sigma: float = 0.002):
    """``nmat`` group-wise affine 4-bit matrices of shape [N, K].

    codes uniform 0..15 (uniform bytes), scale = bf16(|N(0, scale_sigma)|),
    bias = bf16(-8*scale + N(0, bias_sigma)) with the bf16-rounded scale.
    Returns (codes uint8 [nmat,N,K/2], scales uint16 [nmat,N,K/64], biases uint16 [nmat,N,K/64]).
    """
    assert K % GROUP == 0
    if shared:
        r_codes = rng(cid, S_SHARED, 3 * step + 0)
        r_scale = rng(cid, S_SHARED, 3 * step + 1)
        r_bias = rng(cid, S_SHARED, 3 * step + 2)
    else:
        r_codes, r_scale, r_bias = rng(cid, S_CODES, step), rng(cid, S_SCALES, step), rng(cid, S_BIAS, step)
    codes = r_codes.integers(0, 256, size=(nmat, N, K // 2), dtype=np.uint8)
    g = (nmat, N, K // GROUP)
    s_bits = to_bf16_bits(np.abs(r_scale.standard_normal(g, dtype=np.float32) * np.float32(scale_sigma)))
    s = bf16_bits_to_f32(s_bits)
    b = (-8.0 * s + r_bias.standard_normal(g, dtype=np.float32) * np.float32(bias_sigma)).astype(np.float32)
    return codes, s_bits, to_bf16_bits(b)


@dataclasses.dataclass
class Problem:
    """One set of inputs.  Single projection: Wq/S/B are [E, N, K/2] / [E, N, K/64].
    FFN: gu_* are [E, 2N, K...] (gate rows 0..N-1, up rows N..2N-1), dn_* are [E, K, N...],
    sh_* the same for the one shared expert (leading dim 1)."""
    w: Workload
    logits: np.ndarray
    X: np.ndarray
    Wq: Optional[np.ndarray] = None
    S: Optional[np.ndarray] = None
    B: Optional[np.ndarray] = None
    gu_q: Optional[np.ndarray] = None
    gu_s: Optional[np.ndarray] = None
    gu_b: Optional[np.ndarray] = None
    dn_q: Optional[np.ndarray] = None
    dn_s: Optional[np.ndarray] = None
    dn_b: Optional[np.ndarray] = None
    sh_gu_q: Optional[np.ndarray] = None
    sh_gu_s: Optional[np.ndarray] = None
    sh_gu_b: Optional[np.ndarray] = None
    sh_dn_q: Optional[np.ndarray] = None
    sh_dn_s: Optional[np.ndarray] = None
    sh_dn_b: Optional[np.ndarray] = None


def make_problem(w: Workload, step: int = 0, weights: bool = True, shared: bool = True) -> Problem:
    """All inputs of workload ``w``.  Logits and activations depend on ``step``
    (fresh per decode step); weights do not."""
    logits = gen_logits(w.cid, w.T, w.E, step, w.skew_alpha, w.zipf_s)
    X = gen_acts(w.cid, w.T, w.K, step)
    p = Problem(w, logits, X)
    if not weights:
        return p
    if not w.ffn:
        p.Wq, p.S, p.B = gen_q4(w.cid, w.E, w.N, w.K, step=0)
    else:
        p.gu_q, p.gu_s, p.gu_b = gen_q4(w.cid, w.E, 2 * w.N, w.K, step=0)
        p.dn_q, p.dn_s, p.dn_b = gen_q4(w.cid, w.E, w.K, w.N, step=1)
        if shared:
            p.sh_gu_q, p.sh_gu_s, p.sh_gu_b = gen_q4(w.cid, 1, 2 * w.N, w.K, step=0, shared=True)
            p.sh_dn_q, p.sh_dn_s, p.sh_dn_b = gen_q4(w.cid, 1, w.K, w.N, step=1, shared=True)
    return p


def custom(cid: int, T: int, E: int, k: int, K: int, N: int, ffn: bool = False,
           skew_alpha: float = 0.0) -> Workload:
    """An ad-hoc shape (parity sweeps over ragged tails, tiny cases, ...)."""
    return Workload(cid, f"custom T={T} E={E} k={k} K={K} N={N}", T=T, E=E, k=k, K=K, N=N,
                    ffn=ffn, skew_alpha=skew_alpha)
