"""fp64 oracle of the GQA-path decode of GQLA (one group: 16 query heads over that group's cache).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's CPU baseline use it.

GQLA summary, section "Arquitetura", item 2: the latent is expanded into g groups of keys and
values and decode runs standard grouped-query attention; the cache holds the per-group keys and
values plus the shared RoPE key.  Readings (the pages give neither): d_h = 128; a cache row is
[k (128) | RoPE key (64) | v (128)].  For every (sequence b, query token i, head h) with the visible
rows j (all L_b, or L_b - s_q + 1 + i when causal):
    s_j = scale * q[b,i,h,0:192] . row_j[0:192],  O = softmax(s) . row_j[192:320],  LSE = ln sum exp(s_j)
evaluated with :func:`oracle.attention` (the pinned fp64 definition) on the gathered rows.

The section's central claim -- the GQA path and the absorbed MQA path are algebraically equivalent
over the same weights -- is the pin: with k_j = W_UK^T c_j and v_j = W_UV c_j from a latent c_j and
the group's up-projections, this path equals absorb -> latent attention -> un-absorb (tests).
`mistake` plants an error for the pin tests.
"""
from __future__ import annotations

import numpy as np

D_H = 128
D_KEY = D_H + 64
ROW = D_KEY + D_H

V_FROM_KEY = 1      # values taken from the key dims 0..127
KEY_WITHOUT_ROPE = 2  # the shared RoPE key left out of the score


def _f64(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gqa_decode(q_bits, cache_bits, block_table, seqlens, scale: float, causal: bool, mistake: int = 0,
               oracle=None, exact_inputs: bool = False):
    """fp64 O [b, s_q, h, 128] and LSE [b, s_q, h]; q bf16 [b, s_q, h, 192], cache bf16 [pages, 64, 320]
    (with exact_inputs, q and cache are fp64 values instead of bf16 bit patterns).
    A sequence with L_b outside [0, 64 * table width] or a page outside the pool gets NaN."""
    if oracle is None:
        from . import default
        oracle = default()
    conv = (lambda x: np.asarray(x, dtype=np.float64)) if exact_inputs else _f64
    q = conv(q_bits)
    cache = np.asarray(cache_bits)   # bf16 bits (converted row by row below)
    bt = np.asarray(block_table, dtype=np.int64)
    sl = np.asarray(seqlens, dtype=np.int64)
    b, s_q, h, _ = q.shape
    num_pages, page = cache.shape[:2]
    o = np.zeros((b, s_q, h, D_H))
    lse = np.full((b, s_q, h), -np.inf)
    for bi in range(b):
        L = int(sl[bi])
        if L < 0 or L > page * bt.shape[1]:
            o[bi], lse[bi] = np.nan, np.nan
            continue
        pos = np.arange(L)
        pages = bt[bi, pos // page]
        if ((pages < 0) | (pages >= num_pages)).any():
            o[bi], lse[bi] = np.nan, np.nan
            continue
        rows = conv(cache[pages, pos % page])
        for i in range(s_q):
            n = min(max(L - s_q + 1 + i, 0), L) if causal else L
            k = rows[:n, :D_KEY].copy()
            v = rows[:n, :D_H] if mistake == V_FROM_KEY else rows[:n, D_KEY:ROW]
            qi = q[bi, i].copy()
            if mistake == KEY_WITHOUT_ROPE:
                k[:, D_H:] = 0.0
            o[bi, i], lse[bi, i] = oracle.attention(qi, k, v, scale)
    return o, lse
