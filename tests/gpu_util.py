"""Helpers for the GPU parity tests: host <-> device copies and one call of
each library entry point through the binding (test infrastructure)."""
from __future__ import annotations

import numpy as np
import torch

import quantized_grouped_gemm_amd as q


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor, dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def gpu_route(logits: np.ndarray, k: int, block_rows: int):
    """moe_route on the GPU; returns host copies of every output."""
    T, E = logits.shape
    d = dev(np.ascontiguousarray(logits, np.float32)) if T > 0 else torch.empty((0, E), device="cuda")
    b = q.alloc_route(T, E, k, block_rows)
    # poison the outputs so that unwritten entries are visible
    for key in ("topk_ids", "perm", "inv_perm", "blocks", "counts", "offsets", "num_blocks"):
        b[key].fill_(-7)
    q.moe_route(d if T > 0 else None, T, E, k, b["block_rows"], b["topk_ids"], b["topk_w"], b["counts"],
                b["offsets"], b["perm"], b["inv_perm"], b["blocks"], b["num_blocks"], b["workspace"],
                b["ws_bytes"])
    torch.cuda.synchronize()
    A = T * k
    nb = int(host(b["num_blocks"])[0])
    out = dict(
        ids=host(b["topk_ids"])[:A].reshape(T, k), w=host(b["topk_w"])[:A].reshape(T, k),
        counts=host(b["counts"]), offsets=host(b["offsets"]), perm=host(b["perm"])[:A],
        inv_perm=host(b["inv_perm"])[:A], num_blocks=nb,
        blocks=host(b["blocks"]).reshape(-1, 4)[:nb], dev=b, block_rows=b["block_rows"],
        max_blocks=b["max_blocks"])
    return out


NAN_BF16 = 0x7FC0  # quiet NaN: an output the kernels never write stays NaN and fails every comparison


def nan_filled(shape, device="cuda") -> torch.Tensor:
    """int16 tensor (bf16 bit patterns) filled with NaN."""
    return torch.full(shape, NAN_BF16, dtype=torch.int16, device=device)


def gpu_gemm(X: np.ndarray, k: int, Wq, S, B, rt_dev: dict, reps: int = 1) -> np.ndarray:
    """moe_prepack_q4 + moe_grouped_gemm_q4 with routing tables already on the
    device; Y as bf16 bits [T*k, N], poisoned with NaN before the call."""
    Xd = dev(X)
    packed = q.prepack(dev(Wq), dev(S), dev(B))
    T = X.shape[0]
    Y = nan_filled((max(T * k, 1), Wq.shape[1]))
    for _ in range(reps):
        Y = q.grouped_gemm_q4(Xd, k, packed, rt_dev, Y=Y)
    torch.cuda.synchronize()
    return host(Y, np.uint16)


def _nibble_order(b8: np.ndarray) -> np.ndarray:
    """8 row-major bytes (16 codes) -> the tiled word order: per 32-bit word, codes
    c0..c7 stored as nibbles c0,c2,c4,c6,c1,c3,c5,c7."""
    out = np.zeros(8, np.uint8)
    for w in range(2):
        codes = []
        for byte in b8[4 * w: 4 * w + 4]:
            codes += [int(byte) & 15, int(byte) >> 4]
        nib = [codes[i] for i in (0, 2, 4, 6, 1, 3, 5, 7)]
        for j in range(4):
            out[4 * w + j] = nib[2 * j] | (nib[2 * j + 1] << 4)
    return out


def tiled_layout(codes: np.ndarray, scales: np.ndarray, biases: np.ndarray):
    """The tiled layout of moe_prepack_q4, as documented in moeq4.h, built on the host."""
    E, N, K2 = codes.shape
    K = 2 * K2
    G, NT = K // 64, N // 16
    C = (G + 1) // 2
    ct = np.zeros(E * N * K2, np.uint8)
    st = np.zeros(E * N * G, np.uint16)
    bt = np.zeros(E * N * G, np.uint16)
    for e in range(E):
        for t in range(NT):
            for c in range(C):
                full = 2 * c + 1 < G
                base = e * N * K2 + c * NT * 1024 + t * (1024 if full else 512)
                for q_ in range(4):
                    for r in range(16):
                        l = 16 * q_ + r
                        row = codes[e, 16 * t + r]
                        first = _nibble_order(row[c * 64 + q_ * 8: c * 64 + q_ * 8 + 8])
                        if full:
                            ct[base + 16 * l: base + 16 * l + 8] = first
                            ct[base + 16 * l + 8: base + 16 * l + 16] = _nibble_order(
                                row[c * 64 + 32 + q_ * 8: c * 64 + 40 + q_ * 8])
                        else:
                            ct[base + 8 * l: base + 8 * l + 8] = first
                for r in range(16):
                    for g in ((2 * c, 2 * c + 1) if full else (2 * c,)):
                        dst = e * N * G + 32 * c * NT + (32 * t + 2 * r + (g - 2 * c) if full else 16 * t + r)
                        st[dst] = scales[e, 16 * t + r, g]
                        bt[dst] = biases[e, 16 * t + r, g]
    return ct.reshape(codes.shape), st.reshape(scales.shape), bt.reshape(biases.shape)
