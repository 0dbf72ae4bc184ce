"""fp64 oracle of the absorption steps either side of the decode path, and of the decompressed
multi-head attention they must reproduce.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's CPU baseline use it.

Absorbed-MQA form (GQLA summary, section "Arquitetura", item 1): the key and value up-projections
are absorbed into the query and output projections, so every head attends the shared latent cache
directly.  With latent c_j (512), RoPE key r_j (64) and per-head weights W_UK[h] (512 x 128),
W_UV[h] (128 x 512) -- the per-head no-RoPE width 128 is a reading, the pages give only 512 and 64:
  decompressed: k_j = W_UK[h]^T c_j, v_j = W_UV[h] c_j,
                s_j = scale (q_nope . k_j + q_rope . r_j),  o = sum_j softmax(s)_j v_j
  absorbed:     q = [W_UK[h] q_nope ; q_rope],  O_lat = attention of q over [c_j ; r_j] with values c_j,
                o = W_UV[h] O_lat
and the two are equal because q_nope . (W_UK^T c) = (W_UK q_nope) . c and W_UV is linear.
`mistake` plants an error for the pin tests.
"""
from __future__ import annotations

import numpy as np

HEAD_SHIFT = 1   # head h uses the weights of head h + 1
NO_ROPE = 2      # the RoPE part of the query is dropped


def _f64(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def absorb_q(q_nope, q_rope, w_uk, mistake: int = 0) -> np.ndarray:
    """fp64 [..., h, 576] from fp64 q_nope [..., h, 128], q_rope [..., h, 64], w_uk [h, 512, 128]."""
    q_nope = np.asarray(q_nope, dtype=np.float64)
    w = np.asarray(w_uk, dtype=np.float64)
    if mistake == HEAD_SHIFT:
        w = np.roll(w, -1, axis=0)
    lat = np.einsum("hnk,...hk->...hn", w, q_nope)
    rope = np.zeros_like(np.asarray(q_rope, dtype=np.float64)) if mistake == NO_ROPE else np.asarray(q_rope, np.float64)
    return np.concatenate([lat, rope], axis=-1)


def unabsorb_o(o_latent, w_uv, mistake: int = 0) -> np.ndarray:
    """fp64 [..., h, 128] from fp64 o_latent [..., h, 512] and w_uv [h, 128, 512]."""
    w = np.asarray(w_uv, dtype=np.float64)
    if mistake == HEAD_SHIFT:
        w = np.roll(w, -1, axis=0)
    return np.einsum("hdn,...hn->...hd", w, np.asarray(o_latent, dtype=np.float64))


def decompressed_attention(q_nope, q_rope, c, r, w_uk, w_uv, scale: float):
    """Per-head attention with decompressed keys and values, fp64.

    q_nope [h, 128], q_rope [h, 64], c [n, 512], r [n, 64]; returns o [h, 128] and LSE [h]."""
    q_nope = np.asarray(q_nope, np.float64)
    q_rope = np.asarray(q_rope, np.float64)
    c = np.asarray(c, np.float64)
    r = np.asarray(r, np.float64)
    w_uk = np.asarray(w_uk, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    h = q_nope.shape[0]
    o = np.empty((h, w_uv.shape[1]))
    lse = np.empty(h)
    for hh in range(h):
        k = c @ w_uk[hh]                    # [n, 128]: k_j = W_UK^T c_j
        v = c @ w_uv[hh].T                  # [n, 128]: v_j = W_UV c_j
        s = scale * (k @ q_nope[hh] + r @ q_rope[hh])
        m = s.max()
        e = np.exp(s - m)
        o[hh] = (e @ v) / e.sum()
        lse[hh] = m + np.log(e.sum())
    return o, lse
