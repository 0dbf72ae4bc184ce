"""Pins of the GQA-path oracle (oracle/gqa.py), CPU only.

The GQLA page's claim is the pin: over a cache expanded from a latent with the group's
up-projections (k_j = W_UK^T c_j, v_j = W_UV c_j, shared RoPE key r_j), the GQA path equals the
absorbed MQA path (absorb the query, attend the latent cache, un-absorb) in fp64.  Planted mistakes
(values from the key dims, RoPE key left out) must break it; causal rows follow the decode rule.
"""
import numpy as np
import pytest

import oracle
from oracle import absorb as AB
from oracle import gqa as G


def _expanded_case(L=(90, 33), s_q=2, seed=21):
    rng = np.random.default_rng(seed)
    b, h = len(L), 16
    pages = [(n + 63) // 64 for n in L]
    pool = sum(pages)
    lat = rng.standard_normal((pool, 64, 512))
    rope = rng.standard_normal((pool, 64, 64))
    w_uk = rng.standard_normal((512, 128)) / 16            # the group's W_UK (shared by its 16 heads)
    w_uv = rng.standard_normal((128, 512)) / 16
    gq = np.concatenate([lat @ w_uk, rope, lat @ w_uv.T], axis=-1)       # [pool, 64, 320], exact
    bt = np.full((b, max(pages)), -1, dtype=np.int32)
    perm = rng.permutation(pool)
    off = 0
    for i, p in enumerate(pages):
        bt[i, :p] = perm[off:off + p]
        off += p
    q_nope = rng.standard_normal((b, s_q, h, 128))
    q_rope = rng.standard_normal((b, s_q, h, 64))
    return dict(lat=lat, rope=rope, w_uk=w_uk, w_uv=w_uv, gq=gq, bt=bt, sl=np.array(L, dtype=np.int32),
                q_nope=q_nope, q_rope=q_rope, scale=1 / np.sqrt(192))


def _gqa_f64(d, causal, mistake=0):
    q = np.concatenate([d["q_nope"], d["q_rope"]], axis=-1)
    return G.gqa_decode(q, d["gq"], d["bt"], d["sl"], d["scale"], causal, mistake, exact_inputs=True)


def _absorbed(d, causal):
    b, s_q, h, _ = d["q_nope"].shape
    o = np.zeros((b, s_q, h, 128))
    lse = np.zeros((b, s_q, h))
    w_uk = np.broadcast_to(d["w_uk"], (h, 512, 128))
    w_uv = np.broadcast_to(d["w_uv"], (h, 128, 512))
    for bi in range(b):
        L = int(d["sl"][bi])
        pos = np.arange(L)
        pg = d["bt"][bi, pos // 64]
        c, r = d["lat"][pg, pos % 64], d["rope"][pg, pos % 64]
        for i in range(s_q):
            n = min(max(L - s_q + 1 + i, 0), L) if causal else L
            q = AB.absorb_q(d["q_nope"][bi, i], d["q_rope"][bi, i], w_uk)
            ol, lse[bi, i] = oracle.attention(q, np.concatenate([c[:n], r[:n]], axis=1), c[:n], d["scale"])
            o[bi, i] = AB.unabsorb_o(ol, w_uv)
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_path_equals_absorbed_path(causal):
    d = _expanded_case()
    o, l = _gqa_f64(d, causal)
    ro, rl = _absorbed(d, causal)
    np.testing.assert_allclose(o, ro, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(l, rl, rtol=1e-12)


@pytest.mark.parametrize("mistake", [G.V_FROM_KEY, G.KEY_WITHOUT_ROPE])
def test_planted_mistake_breaks_equivalence(mistake):
    d = _expanded_case()
    o, _ = _gqa_f64(d, False, mistake)
    ro, _ = _absorbed(d, False)
    assert not np.allclose(o, ro, rtol=1e-6, atol=1e-8)


def test_causal_token0_sees_one_key_less():
    d = _expanded_case(L=(70,), s_q=2)
    o, l = _gqa_f64(d, True)
    d1 = dict(d)
    d1["sl"] = np.array([69], dtype=np.int32)
    d1["q_nope"], d1["q_rope"] = d["q_nope"][:, :1], d["q_rope"][:, :1]
    o1, l1 = _gqa_f64(d1, False)
    np.testing.assert_allclose(o[:, 0], o1[:, 0], rtol=1e-13, atol=1e-14)
