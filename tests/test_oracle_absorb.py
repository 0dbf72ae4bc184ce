"""Pins of the absorption oracle (oracle/absorb.py), CPU only.

The absorbed chain -- absorb the query, attend the latent cache with the (pinned) attention oracle,
un-absorb the output -- must equal decompressed per-head attention in fp64; a weight that selects
the first 128 latent dims must copy q_nope; planted mistakes must fail.
"""
import numpy as np
import pytest

import oracle
from oracle import absorb as AB


def _setup(h=4, n=37, seed=3):
    rng = np.random.default_rng(seed)
    return dict(q_nope=rng.standard_normal((h, 128)), q_rope=rng.standard_normal((h, 64)),
                c=rng.standard_normal((n, 512)), r=rng.standard_normal((n, 64)),
                w_uk=rng.standard_normal((h, 512, 128)) / 16, w_uv=rng.standard_normal((h, 128, 512)) / 16,
                scale=0.0721)


def _chain(d, mistake=0):
    q = AB.absorb_q(d["q_nope"], d["q_rope"], d["w_uk"], mistake)          # [h, 576]
    keys = np.concatenate([d["c"], d["r"]], axis=1)                          # [n, 576]
    o_lat, lse = oracle.attention(q, keys, d["c"], d["scale"])
    return AB.unabsorb_o(o_lat, d["w_uv"], mistake), lse


def test_absorbed_chain_equals_decompressed_attention():
    d = _setup()
    o, lse = _chain(d)
    ro, rl = AB.decompressed_attention(d["q_nope"], d["q_rope"], d["c"], d["r"], d["w_uk"], d["w_uv"], d["scale"])
    np.testing.assert_allclose(o, ro, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=1e-12)


def test_selector_weight_copies_q_nope():
    d = _setup(h=2)
    w = np.zeros((2, 512, 128))
    w[:, :128, :] = np.eye(128)
    q = AB.absorb_q(d["q_nope"], d["q_rope"], w)
    np.testing.assert_array_equal(q[:, :128], d["q_nope"])
    np.testing.assert_array_equal(q[:, 128:512], 0.0)
    np.testing.assert_array_equal(q[:, 512:], d["q_rope"])


@pytest.mark.parametrize("mistake", [AB.HEAD_SHIFT, AB.NO_ROPE])
def test_planted_mistake_breaks_the_equivalence(mistake):
    d = _setup()
    o, lse = _chain(d, mistake)
    ro, rl = AB.decompressed_attention(d["q_nope"], d["q_rope"], d["c"], d["r"], d["w_uk"], d["w_uv"], d["scale"])
    assert not np.allclose(o, ro, rtol=1e-6, atol=1e-8)
