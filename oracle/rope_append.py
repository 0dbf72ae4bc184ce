"""fp64 oracle of the paged cache append with rotary embedding of the RoPE parts.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's CPU baseline use it;
the library never calls it.

What it computes (the step that feeds the decode path).  The cache row of the absorbed form is
the 512-d latent followed by one 64-d RoPE key shared by all heads (GQLA summary, section
"Arquitetura": the cache stores the latent and one shared RoPE key).  For sequence b and new
token i of a decode step, pos = L_b - s_q + i; the row at page block_table[b][pos // 64], slot
pos % 64 receives the latent unchanged and the RoPE key rotated by pos, and the 64-d RoPE part
of every head of the token's query is rotated by pos.

Reading (the pages name the RoPE key but give no formula): the rotary embedding in its original
pairwise form -- dims (2p, 2p+1) turn by the angle pos * base**(-2p/64), p = 0..31.

Everything is evaluated in fp64 on the exact bf16 input values; outputs are fp64 (the GPU rounds
them once to bf16).  `mistake` plants one of several plausible errors, for the pin tests.
"""
from __future__ import annotations

import numpy as np

D_V = 512
ROPE_DIM = 64
PAGE = 64

# planted mistakes (0 = none)
HALF_SPLIT = 1     # pairs (p, p + 32) instead of (2p, 2p + 1)
SIN_SIGN = 2       # rotation by -angle
EXPONENT = 3       # base ** (-p / 64) instead of base ** (-2p / 64)
POS_OFF_BY_ONE = 4 # pos = L - s_q + i + 1


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def rope_rotate(x, pos, base: float, mistake: int = 0) -> np.ndarray:
    """Rotate the 64-d parts x[..., 64] (fp64) by positions `pos` (broadcast to x[..., 0])."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    p = np.arange(d // 2, dtype=np.float64)
    theta = base ** (-(p if mistake == EXPONENT else 2.0 * p) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    if mistake == SIN_SIGN:
        ang = -ang
    c, s = np.cos(ang), np.sin(ang)
    if mistake == HALF_SPLIT:
        xe, xo = x[..., : d // 2], x[..., d // 2:]
    else:
        xe, xo = x[..., 0::2], x[..., 1::2]
    re = xe * c - xo * s
    im = xe * s + xo * c
    out = np.empty_like(x)
    if mistake == HALF_SPLIT:
        out[..., : d // 2], out[..., d // 2:] = re, im
    else:
        out[..., 0::2], out[..., 1::2] = re, im
    return out


def append_rope(kv_latent_bits, k_rope_bits, q_bits, block_table, seqlens, num_pages: int, base: float,
                mistake: int = 0):
    """The append step for all new tokens.

    kv_latent_bits uint16 [b, s_q, 512], k_rope_bits uint16 [b, s_q, 64], q_bits uint16 [b, s_q, h, 576],
    block_table int32 [b, stride], seqlens int32 [b].
    Returns (rows, q_rope): rows maps (page, slot) -> (latent bits uint16 [512], rotated key fp64 [64]) for
    every token with a valid slot; q_rope fp64 [b, s_q, h, 64] is the rotated query RoPE part (NaN for a
    token without a valid slot: negative pos, L_b beyond the table, or a page outside [0, num_pages)).
    """
    lat = np.asarray(kv_latent_bits, dtype=np.uint16)
    kr = bf16_bits_to_f64(k_rope_bits)
    qr = bf16_bits_to_f64(np.asarray(q_bits, dtype=np.uint16)[..., D_V:])
    bt = np.asarray(block_table, dtype=np.int64)
    sl = np.asarray(seqlens, dtype=np.int64)
    b, s_q = lat.shape[:2]
    rows = {}
    q_rope = np.full(qr.shape, np.nan)
    for bi in range(b):
        for i in range(s_q):
            pos = int(sl[bi]) - s_q + i + (1 if mistake == POS_OFF_BY_ONE else 0)
            if pos < 0 or sl[bi] > PAGE * bt.shape[1] or pos // PAGE >= bt.shape[1]:
                continue
            page = int(bt[bi, pos // PAGE])
            if page < 0 or page >= num_pages:
                continue
            rows[(page, pos % PAGE)] = (lat[bi, i].copy(), rope_rotate(kr[bi, i], pos, base, mistake))
            q_rope[bi, i] = rope_rotate(qr[bi, i], np.full(qr.shape[2], pos), base, mistake)
    return rows, q_rope
