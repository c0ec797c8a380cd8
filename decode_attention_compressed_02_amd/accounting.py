"""Memory, traffic and FLOP models of the SWAN decode step.

Formulas follow the SWAN page (memory analysis section and appendix A.2) and
the per-token KV-size formula of "Reuse, Evict, or Limit Earlier Context"
(section 3.4).  The HBM-traffic model is this library's own: the bytes the
decode kernels must move at minimum for the layouts they read.
"""
from __future__ import annotations

import math


def sparse_vector_bytes(k: int, value_bytes: int = 2, index_bytes: int = 1, offset_bytes: int = 2) -> int:
    """Bytes of one pruned vector: k (index, value) pairs plus the constant
    2-byte CSR offset (SWAN page, memory-savings paragraphs): 3k + 2 with fp16 values and
    8-bit indices, 2k + 2 with 8-bit float values."""
    return k * (value_bytes + index_bytes) + offset_bytes


def dense_vector_bytes(d_h: int = 128, value_bytes: int = 2) -> int:
    """A dense fp16 vector: d_h * 2 bytes (256 at d_h = 128)."""
    return d_h * value_bytes


def compression_ratio(k: int, d_h: int = 128, value_bytes: int = 2) -> float:
    """Sparse-to-dense size ratio (3k + 2) / 256 at fp16, d_h = 128."""
    return sparse_vector_bytes(k, value_bytes) / dense_vector_bytes(d_h)


def memory_break_even_k(d_h: int = 128, value_bytes: int = 2) -> int:
    """Largest k whose sparse vector is still smaller than the dense one."""
    k = 0
    while sparse_vector_bytes(k + 1, value_bytes) < dense_vector_bytes(d_h):
        k += 1
    return k


def kv_bytes_per_token(layers: int, H_kv: int, d_head: int, elem_bytes: int) -> int:
    """Dense K+V bytes per token over all layers: 2 * L * H_kv * d_head * b."""
    return 2 * layers * H_kv * d_head * elem_bytes


def flops_standard(L: int, d_h: int = 128) -> float:
    """Dense decode attention of one head: 2 L d_h for scores plus 2 L d_h
    for the output (softmax is lower order)."""
    return 4.0 * L * d_h


def flops_swan(L: int, b: int, k: int, d_h: int = 128, k_v: int | None = None) -> float:
    """SWAN decode of one head (appendix A.2): 4 d_h^2 for projecting q and k,
    2 (L - b) k + 2 b d_h for scores, 2 (L - b) k_v + 2 b d_h for the output."""
    k_v = k if k_v is None else k_v
    return 4.0 * d_h * d_h + 2.0 * (L - b) * k + 2.0 * b * d_h + 2.0 * (L - b) * k_v + 2.0 * b * d_h


def break_even_length(b: int, k: int, d_h: int = 128) -> float:
    """Context length beyond which SWAN needs fewer FLOPs than dense decode:
    C_swan < C_std  <=>  L > b + d_h^2 / (d_h - k)  (for k < d_h)."""
    if k >= d_h:
        return math.inf
    return b + d_h * d_h / (d_h - k)


# ---------------------------------------------------------------------------
# per-step traffic and work of this library's decode kernels
# ---------------------------------------------------------------------------

def split_kernel_bytes(n_per_seq, H_kv: int, N_h: int, R_fill_per_seq, k: int, d_h: int = 128,
                       value_bytes: int = 2, k_v: int = 0) -> int:
    """Algorithmic HBM bytes of one launch of the split (streaming) kernel:
    every sparse row read once (k key and k_v value entries, k_v = k unless
    given, each a one-byte index and a value of value_bytes -- 6k bytes per
    token per kv-head with fp16 values, 4k with fp8), every buffered token
    read once (K and V fp16, 4 d_h bytes), and the fp32 rotated queries read
    once.  Partials (a few percent) are not counted."""
    sparse = sum(int(n) for n in n_per_seq) * H_kv * (k + (k_v or k)) * (1 + value_bytes)
    dense = sum(int(r) for r in R_fill_per_seq) * H_kv * 4 * d_h
    q_in = len(list(n_per_seq)) * N_h * d_h * 4
    return sparse + dense + q_in


def decode_bytes(n_per_seq, H_kv: int, N_h: int, R_fill_per_seq, k: int, d_h: int = 128,
                 value_bytes: int = 2, k_v: int = 0) -> int:
    """Algorithmic bytes of the whole decode (split + reduce): the split
    kernel's bytes plus the fp32 outputs written once."""
    B = len(list(n_per_seq))
    return split_kernel_bytes(n_per_seq, H_kv, N_h, R_fill_per_seq, k, d_h, value_bytes, k_v) + B * N_h * d_h * 4


def decode_flops(n_per_seq, H_kv: int, N_h: int, R_fill_per_seq, k: int, d_h: int = 128, k_v: int = 0) -> float:
    """Multiply-add FLOPs (2 per MAC) of scores and outputs over all heads."""
    g = N_h // H_kv
    tot = 0.0
    for n, r in zip(n_per_seq, R_fill_per_seq):
        tot += H_kv * g * (2.0 * n * (k + (k_v or k)) + 4.0 * r * d_h)
    return tot
