"""Pins of the oracle's second output, sum_j p_j |v_j| per element (the tests' error scale for
weights rounded before the weighted sum): brute force on a small case, the triangle inequality
against |O|, and equality with O when every value is nonnegative."""
from __future__ import annotations

import math

import numpy as np

import oracle
from mla_decode_attention_amd.inputs import bf16_bits_to_f32, make_case


def _case():
    return make_case("value_scale", batch=2, s_q=2, heads=16, seqlen=[9, 70], seed=81, causal=True,
                     outlier_frac=0.2, outlier_scale=8.0)


def test_value_scale_brute_force():
    c = _case()
    o, lse, a = oracle.mla_decode(c.q, c.cache, c.block_table, c.seqlens, c.softmax_scale, c.causal,
                                  with_scale=True)
    q = bf16_bits_to_f32(c.q).astype(np.float64)
    kv = bf16_bits_to_f32(c.cache).astype(np.float64)
    for b, i, h in [(0, 0, 3), (0, 1, 15), (1, 0, 0), (1, 1, 7)]:
        L = int(c.seqlens[b])
        n = L - c.s_q + 1 + i
        keys = [kv[c.block_table[b, j // 64], j % 64] for j in range(n)]
        s = [c.softmax_scale * math.fsum(q[b, i, h, d] * k[d] for d in range(576)) for k in keys]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        l = math.fsum(e)
        for d in (0, 1, 255, 511):
            want = math.fsum(e[j] * abs(keys[j][d]) for j in range(n)) / l
            assert abs(a[b, i, h, d] - want) <= 1e-12 * max(1.0, want)


def test_value_scale_bounds_and_equality():
    c = _case()
    o, lse, a = oracle.mla_decode(c.q, c.cache, c.block_table, c.seqlens, c.softmax_scale, c.causal,
                                  with_scale=True)
    assert (a >= np.abs(o) * (1 - 1e-12)).all()
    # nonnegative values (sign bits cleared): the weighted sum of |v| is the weighted sum of v
    pos = c.cache & np.uint16(0x7FFF)
    o2, _, a2 = oracle.mla_decode(c.q, pos, c.block_table, c.seqlens, c.softmax_scale, c.causal, with_scale=True)
    np.testing.assert_array_equal(o2, a2)
