"""Pins of the append + rotary-embedding oracle (oracle/rope_append.py), CPU only.

The pages give no rotary formula (the reading is the original pairwise form), so the rotation is
pinned by what any rotary embedding must satisfy -- identity at position 0, a rotation of each
(2p, 2p+1) pair and of nothing else, counterclockwise at 1 rad per position in pair 0, relative
positions (q(m).k(n) depends on m - n only), composition -- plus the geometric frequency schedule
of the reading, and the cache placement is pinned by a hand-worked example.  Every planted
mistake must fail at least one pin.
"""
import math

import numpy as np
import pytest

from oracle import rope_append as RA

BASE = 10000.0


def _rng():
    return np.random.default_rng(7)


def pin_identity_at_zero(m):
    x = _rng().standard_normal((5, 64))
    return np.array_equal(RA.rope_rotate(x, np.zeros(5), BASE, m), x)


def pin_pairs_keep_their_norm(m):
    x = _rng().standard_normal((6, 64))
    y = RA.rope_rotate(x, np.array([1, 7, 100, 4095, 65535, 123456]), BASE, m)
    n0 = x[:, 0::2] ** 2 + x[:, 1::2] ** 2
    n1 = y[:, 0::2] ** 2 + y[:, 1::2] ** 2
    return np.allclose(n0, n1, rtol=1e-12, atol=0)


def pin_only_its_own_pair_moves(m):
    ok = True
    for p in (0, 5, 31):
        x = np.zeros(64)
        x[2 * p], x[2 * p + 1] = 0.6, -0.8
        y = RA.rope_rotate(x, 333, BASE, m)
        rest = np.delete(y, [2 * p, 2 * p + 1])
        ok &= np.all(rest == 0.0) and abs(math.hypot(y[2 * p], y[2 * p + 1]) - 1.0) < 1e-14
    return bool(ok)


def pin_pair0_turns_one_radian_counterclockwise(m):
    x = np.zeros(64)
    x[0] = 1.0
    y = RA.rope_rotate(x, 1, BASE, m)
    return abs(math.atan2(y[1], y[0]) - 1.0) < 1e-15


def pin_relative_positions(m):
    r = _rng()
    q, k = r.standard_normal(64), r.standard_normal(64)
    ok = True
    for a, b in ((5, 2), (1000, 999), (70000, 12345)):
        lhs = RA.rope_rotate(q, a, BASE, m) @ RA.rope_rotate(k, b, BASE, m)
        rhs = RA.rope_rotate(q, a - b, BASE, m) @ k
        ok &= abs(lhs - rhs) <= 1e-9 * (abs(lhs) + 1)
    return bool(ok)


def pin_composition(m):
    x = _rng().standard_normal(64)
    return np.allclose(RA.rope_rotate(RA.rope_rotate(x, 300, BASE, m), 77, BASE, m),
                       RA.rope_rotate(x, 377, BASE, m), rtol=1e-10, atol=1e-12)


def pin_geometric_schedule(m):
    # angle per position of pair p, measured on a unit vector; the reading's schedule has a
    # constant ratio base^(-2/64) between neighbouring pairs
    angles = []
    for p in range(32):
        x = np.zeros(64)
        x[2 * p] = 1.0
        y = RA.rope_rotate(x, 1, BASE, m)
        angles.append(math.atan2(y[2 * p + 1], y[2 * p]))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratios = np.array(angles[1:]) / np.array(angles[:-1])
    return bool(np.allclose(ratios, BASE ** (-2.0 / 64), rtol=1e-12))


def _placement_case():
    # two sequences, two new tokens each: L = 70 (tokens at 68, 69 -> table entry 1 = page 0,
    # slots 4, 5) and L = 2 (tokens at 0, 1 -> table entry 0 = page 1, slots 0, 1)
    lat = np.arange(2 * 2 * 512, dtype=np.uint16).reshape(2, 2, 512)
    kr = np.full((2, 2, 64), 0x3f80, dtype=np.uint16)        # 1.0
    q = np.full((2, 2, 3, 576), 0x3f80, dtype=np.uint16)
    bt = np.array([[2, 0], [1, -1]], dtype=np.int32)
    sl = np.array([70, 2], dtype=np.int32)
    return lat, kr, q, bt, sl


def pin_cache_placement(m):
    lat, kr, q, bt, sl = _placement_case()
    rows, qr = RA.append_rope(lat, kr, q, bt, sl, num_pages=3, base=BASE, mistake=m)
    if sorted(rows) != [(0, 4), (0, 5), (1, 0), (1, 1)]:
        return False
    if not np.array_equal(rows[(0, 5)][0], lat[0, 1]) or not np.array_equal(rows[(1, 0)][0], lat[1, 0]):
        return False
    # the key of the token at position 0 is not rotated
    return bool(np.all(rows[(1, 0)][1] == 1.0)) and bool(np.all(qr[1, 0] == 1.0))


def pin_invalid_tokens_write_nothing(m):
    lat, kr, q, bt, sl = _placement_case()
    sl = np.array([1, 2], dtype=np.int32)          # sequence 0: token 0 would sit at position -1
    bt = np.array([[2, 0], [5, -1]], dtype=np.int32)  # sequence 1: page 5 is outside the pool
    rows, qr = RA.append_rope(lat, kr, q, bt, sl, num_pages=3, base=BASE, mistake=m)
    return sorted(rows) == [(2, 0)] and np.isnan(qr[0, 0]).all() and np.isnan(qr[1]).all() and \
        not np.isnan(qr[0, 1]).any()


PINS = [pin_identity_at_zero, pin_pairs_keep_their_norm, pin_only_its_own_pair_moves,
        pin_pair0_turns_one_radian_counterclockwise, pin_relative_positions, pin_composition,
        pin_geometric_schedule, pin_cache_placement, pin_invalid_tokens_write_nothing]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    assert pin(0)


@pytest.mark.parametrize("mistake", [RA.HALF_SPLIT, RA.SIN_SIGN, RA.EXPONENT, RA.POS_OFF_BY_ONE])
def test_planted_mistake_fails_a_pin(mistake):
    failed = [p.__name__ for p in PINS if not p(mistake)]
    assert failed, f"planted mistake {mistake} passes every pin"
