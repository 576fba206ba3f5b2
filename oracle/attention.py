"""Oracle: exact softmax attention in float64 on dequantized values (test
infrastructure only).

For query row i of head h and key row j of KV head h // (Hq/Hkv):

    x_ij = softmax_scale * (q_i . k_j)
    p_ij = exp(x_ij - max_j x_ij) / sum_j exp(x_ij - max_j x_ij)
    o_i  = sum_j p_ij v_j

with keys j <= i only when causal, and j < L_b in decode. ``q``, ``k``, ``v`` are
the dequantized values ``s_block * code`` (the [Ascend-INT8] page, section 1 of
its INT8-operator optimisations: INT8 x INT8 products accumulated in INT32 and
converted once at the output, which reaches exactly this dot product of the
dequantized rows; and its section 3: decode attention computed on an INT8 KV
cache). ``softmax_scale`` is the exact float32 the kernels receive (1/sqrt(D) in
the pages' listings, [FA-INT8/INT4] INT8 layer and [Edge-FA] third layer).
The pages' own blocked loops do not compute softmax attention (they sum
per-block exponentials without rescaling them to a common maximum); this
oracle follows the definition instead.
"""
from __future__ import annotations

import numpy as np


def _attend(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, softmax_scale: float,
            causal_rows: np.ndarray | None) -> np.ndarray:
    """Softmax attention of the given query rows over all rows of k/v (float64).
    ``causal_rows`` holds each query's own position when causal, else None."""
    x = float(softmax_scale) * (q_rows @ k.T)
    if causal_rows is not None:
        j = np.arange(k.shape[0])[None, :]
        x = np.where(j <= causal_rows[:, None], x, -np.inf)
    m = x.max(axis=1, keepdims=True)
    p = np.exp(x - m)
    return (p @ v) / p.sum(axis=1, keepdims=True)


def attention_rows(q_hat, k_hat, v_hat, softmax_scale: float, causal: bool,
                   b: int, h: int, rows) -> np.ndarray:
    """Output rows ``rows`` of query head ``h`` in batch ``b``; inputs BNSD float64,
    K/V with Hkv heads (query head h reads KV head h // (Hq // Hkv))."""
    Hq, Hkv = q_hat.shape[1], k_hat.shape[1]
    kvh = h // (Hq // Hkv)
    rows = np.asarray(rows, dtype=np.int64)
    q_rows = np.asarray(q_hat[b, h], dtype=np.float64)[rows]
    return _attend(q_rows, np.asarray(k_hat[b, kvh], np.float64),
                   np.asarray(v_hat[b, kvh], np.float64), softmax_scale,
                   rows if causal else None)


def attention(q_hat, k_hat, v_hat, softmax_scale: float, causal: bool = False) -> np.ndarray:
    """Full output [B, Hq, Sq, D] in float64. Causal requires Sq == Sk."""
    B, Hq, Sq, D = q_hat.shape
    Hkv, Sk = k_hat.shape[1], k_hat.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if causal and Sq != Sk:
        raise ValueError("causal attention needs Sq == Sk")
    out = np.empty((B, Hq, Sq, v_hat.shape[3]), dtype=np.float64)
    rows = np.arange(Sq)
    for b in range(B):
        for h in range(Hq):
            out[b, h] = attention_rows(q_hat, k_hat, v_hat, softmax_scale, causal, b, h, rows)
    return out


def decode(q, k_hat, v_hat, lens, softmax_scale: float) -> np.ndarray:
    """One query token per sequence against its first ``lens[b]`` cache rows.

    q: [B, Hq, 1, D] (the unquantized query, e.g. fp16, used exactly);
    k_hat, v_hat: [B, Hkv, S_max, D] dequantized cache (float64);
    returns [B, Hq, 1, D] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, _, D = q.shape
    Hkv = k_hat.shape[1]
    out = np.empty((B, Hq, 1, v_hat.shape[3]), dtype=np.float64)
    for b in range(B):
        L = int(lens[b])
        for h in range(Hq):
            kvh = h // (Hq // Hkv)
            out[b, h] = _attend(q[b, h], np.asarray(k_hat[b, kvh, :L], np.float64),
                                np.asarray(v_hat[b, kvh, :L], np.float64), softmax_scale, None)
    return out
