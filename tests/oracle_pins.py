"""Pins for the fp64 oracle: checks against facts that do not come from the oracle itself.

Each ``pin_*`` takes an :class:`oracle.Oracle` handle and raises AssertionError
when the oracle disagrees with
  * a pure-Python brute-force evaluation of the definition (math.fsum/math.exp)
    on tiny inputs, with its own page-table walk;
  * closed forms: one visible key gives O = v_0 exactly and LSE = scale q.k_0;
    a zero query gives O = mean(V) and LSE = ln n; identical keys give mean(V);
    one dominant key gives its own value;
  * invariants: probabilities sum to one; a KV split merged by LSE equals the
    unsplit result; relabelling the pool pages changes nothing;
  * the ETAP transposed ordering (FlashMLA-ETAP summary, "Mecanismo Central");
  * a statistical closed form: for N(0, I) keys, exponential tilting gives
    O -> scale * q[:512] and LSE -> ln L + scale^2 |q|^2 / 2.
The same functions run against deliberately wrong oracle builds to show that
each plausible mistake is caught by at least one pin.
"""
from __future__ import annotations

import math

import numpy as np

import oracle as oracle_mod
from mla_decode_attention_amd.inputs import BF16_QNAN, bf16_bits_to_f32, f32_to_bf16_bits, make_case

SCALE = 1.0 / math.sqrt(192.0)


def brute_attention(q, k, v, scale):
    """Definition of softmax attention in pure Python, one row at a time."""
    outs, lses = [], []
    for qi in q:
        s = [scale * math.fsum(float(a) * float(b) for a, b in zip(qi, kj)) for kj in k]
        if not s:
            outs.append([0.0] * len(v[0]) if len(v) else [])
            lses.append(-math.inf)
            continue
        m = max(s)
        e = [math.exp(x - m) for x in s]
        l = math.fsum(e)
        outs.append([math.fsum(e[j] * float(v[j][d]) for j in range(len(k))) / l for d in range(len(v[0]))])
        lses.append(m + math.log(l))
    return np.array(outs), np.array(lses)


def brute_mla(q_bits, cache_bits, table, seqlens, scale, causal, d_v=512):
    """Pure-Python paged decode: walks the block table itself, decodes bf16 by bit shift."""
    b_, s_q, h, _ = q_bits.shape
    page_size = cache_bits.shape[1]
    qf = bf16_bits_to_f32(q_bits).astype(np.float64)
    cf = bf16_bits_to_f32(cache_bits).astype(np.float64)
    o = np.zeros((b_, s_q, h, d_v))
    lse = np.zeros((b_, s_q, h))
    for b in range(b_):
        L = int(seqlens[b])
        for i in range(s_q):
            n = min(max(L - s_q + 1 + i, 0), L) if causal else L
            keys = [cf[int(table[b][j // page_size]), j % page_size] for j in range(n)]
            vals = [kk[:d_v] for kk in keys]
            for hh in range(h):
                if n == 0:
                    o[b, i, hh] = 0.0
                    lse[b, i, hh] = -math.inf
                    continue
                ob, lb = brute_attention([qf[b, i, hh]], keys, vals, scale)
                o[b, i, hh] = ob[0]
                lse[b, i, hh] = lb[0]
    return o, lse


def _tiny_paged_case(rng, page_size=4, batch=2, s_q=2, heads=2, lens=(5, 3), d_k=576, pool=7):
    """Hand-built paged case with a small page size, shuffled table and NaN in unused slots."""
    qf = rng.standard_normal((batch, s_q, heads, d_k)).astype(np.float32)
    cf = rng.standard_normal((pool, page_size, d_k)).astype(np.float32)
    q_bits, cache_bits = f32_to_bf16_bits(qf), f32_to_bf16_bits(cf)
    perm = rng.permutation(pool)
    pages = [(L + page_size - 1) // page_size for L in lens]
    table = np.full((batch, max(pages) + 1), -1, dtype=np.int32)
    off = 0
    owned = np.zeros(pool, dtype=bool)
    for b, npg in enumerate(pages):
        table[b, :npg] = perm[off:off + npg]
        owned[perm[off:off + npg]] = True
        off += npg
        tail = lens[b] % page_size
        if tail:
            cache_bits[table[b, npg - 1], tail:] = BF16_QNAN
    cache_bits[~owned] = BF16_QNAN
    return q_bits, cache_bits, table, np.array(lens, dtype=np.int32)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    same_inf = (np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b)))
    with np.errstate(invalid="ignore"):
        diff = np.where(same_inf, 0.0, np.abs(a - b))
    assert np.all(np.isfinite(diff)) and diff.max(initial=0.0) <= tol, (what, float(np.nanmax(diff, initial=0.0)))


# ---------------------------------------------------------------------------------------------

def pin_brute_force_dense(orc):
    rng = np.random.default_rng(11)
    q, k, v = rng.standard_normal((3, 8)), rng.standard_normal((7, 8)), rng.standard_normal((7, 5))
    o, lse = orc.attention(q, k, v, 0.37)
    bo, bl = brute_attention(q.tolist(), k.tolist(), v.tolist(), 0.37)
    _close(o, bo, 1e-12, "dense O vs brute force")
    _close(lse, bl, 1e-12, "dense LSE vs brute force")


def pin_brute_force_paged(orc):
    rng = np.random.default_rng(12)
    q_bits, cache_bits, table, lens = _tiny_paged_case(rng)
    for causal in (False, True):
        o, lse = orc.mla_decode(q_bits, cache_bits, table, lens, SCALE, causal)
        bo, bl = brute_mla(q_bits, cache_bits, table, lens, SCALE, causal)
        _close(o, bo, 1e-12, f"paged O vs brute force (causal={causal})")
        _close(lse, bl, 1e-12, f"paged LSE vs brute force (causal={causal})")


def pin_brute_force_page64(orc):
    case = make_case("pin64", batch=2, s_q=1, heads=2, seqlen=[70, 3], seed=13, pool_pages=4)
    o, lse = orc.mla_decode(case.q, case.cache, case.block_table, case.seqlens, SCALE, False)
    bo, bl = brute_mla(case.q, case.cache, case.block_table, case.seqlens, SCALE, False)
    _close(o, bo, 1e-12, "page-64 O vs brute force")
    _close(lse, bl, 1e-12, "page-64 LSE vs brute force")


def pin_transposed_identity(orc):
    rng = np.random.default_rng(14)
    q = rng.standard_normal((16, 576))
    k = rng.standard_normal((100, 576))
    v = k[:, :512]
    o, lse = orc.attention(q, k, v, SCALE)
    ot, lt = oracle_mod.transposed_attention(q, k, v, SCALE)
    _close(o, ot, 1e-13, "O vs (V^T P^T)^T")
    _close(lse, lt, 1e-12, "LSE vs transposed form")


def pin_single_key(orc):
    case = make_case("pin1", batch=1, s_q=1, heads=3, seqlen=1, seed=15)
    o, lse = orc.mla_decode(case.q, case.cache, case.block_table, case.seqlens, SCALE, False)
    key = bf16_bits_to_f32(case.cache[case.block_table[0, 0], 0]).astype(np.float64)
    qf = bf16_bits_to_f32(case.q[0, 0]).astype(np.float64)
    for hh in range(3):
        assert np.array_equal(o[0, 0, hh], key[:512]), "one key must return its value exactly"
        want = SCALE * math.fsum(float(a) * float(b) for a, b in zip(qf[hh], key))
        assert abs(lse[0, 0, hh] - want) <= 1e-12, ("one-key LSE", lse[0, 0, hh], want)


def pin_zero_query(orc):
    case = make_case("pin0", batch=2, s_q=1, heads=2, seqlen=[37, 130], seed=16, zero_q=True)
    o, lse = orc.mla_decode(case.q, case.cache, case.block_table, case.seqlens, SCALE, False)
    cf = bf16_bits_to_f32(case.cache).astype(np.float64)
    for b in range(2):
        L = int(case.seqlens[b])
        vals = np.stack([cf[case.block_table[b, j // 64], j % 64, :512] for j in range(L)])
        mean = np.array([math.fsum(vals[:, d]) / L for d in range(512)])
        for hh in range(2):
            _close(o[b, 0, hh], mean, 1e-13, "zero query gives mean(V)")
            assert abs(lse[b, 0, hh] - math.log(L)) <= 1e-13, ("zero query LSE = ln n", lse[b, 0, hh], math.log(L))


def pin_identical_keys(orc):
    rng = np.random.default_rng(17)
    kk = rng.standard_normal(64)
    k = np.tile(kk, (9, 1))
    v = rng.standard_normal((9, 6))
    q = rng.standard_normal((2, 64))
    o, _ = orc.attention(q, k, v, 0.5)
    mean = np.array([math.fsum(v[:, d]) / 9 for d in range(6)])
    for r in range(2):
        _close(o[r], mean, 1e-13, "identical keys give mean(V)")


def pin_probabilities_sum_to_one(orc):
    rng = np.random.default_rng(18)
    q, k, v = rng.standard_normal((4, 32)), rng.standard_normal((50, 32)) * 3, rng.standard_normal((50, 8))
    _, _, p = orc.attention(q, k, v, 0.8, return_probs=True)
    assert (p >= 0).all()
    for r in range(4):
        assert abs(math.fsum(p[r]) - 1.0) <= 1e-14, ("P row sum", math.fsum(p[r]))


def pin_dominant_key(orc):
    """A key whose score exceeds the rest by ~1000 takes all the weight; exp must not overflow."""
    rng = np.random.default_rng(19)
    q = rng.standard_normal((1, 16))
    k = rng.standard_normal((5, 16))
    k[3] = q[0] * (1000.0 / float(q[0] @ q[0]))
    v = rng.standard_normal((5, 4))
    o, lse = orc.attention(q, k, v, 1.0)
    assert np.all(np.isfinite(o)) and np.isfinite(lse).all(), "overflow in softmax"
    _close(o[0], v[3], 1e-12, "dominant key returns its value")
    s_max = math.fsum(float(a) * float(b) for a, b in zip(q[0], k[3]))
    assert abs(lse[0] - s_max) <= 1e-9, ("dominant key LSE", lse[0], s_max)


def pin_split_invariance(orc):
    rng = np.random.default_rng(20)
    n_k = 40
    q = rng.standard_normal((3, 576))
    k = rng.standard_normal((n_k, 576))
    v = k[:, :512].copy()
    o_full, lse_full = orc.attention(q, k, v, SCALE)
    cuts = [[0, n_k], [0, 1, 2, 3, n_k], [0, 0, 17, 17, n_k], sorted([0, n_k] + list(rng.integers(0, n_k, 6)))]
    cuts.append(list(range(n_k + 1)))               # every key its own part
    for bounds in cuts:
        parts_o, parts_l = [], []
        for a, b in zip(bounds[:-1], bounds[1:]):
            po, pl = orc.attention(q, k[a:b], v[a:b], SCALE)
            parts_o.append(po)
            parts_l.append(pl)
        mo, ml = oracle_mod.merge_by_lse(parts_o, parts_l)
        _close(mo, o_full, 1e-13, f"split {bounds[:6]}... merged O")
        _close(ml, lse_full, 1e-12, f"split {bounds[:6]}... merged LSE")


def pin_page_relabelling(orc):
    case = make_case("pinperm", batch=3, s_q=2, heads=2, seqlen=[150, 64, 1], seed=21, pool_pages=9,
                     causal=True)
    o1, l1 = orc.mla_decode(case.q, case.cache, case.block_table, case.seqlens, SCALE, True)
    rng = np.random.default_rng(22)
    relabel = rng.permutation(case.num_pages)          # pool page p moves to relabel[p]
    cache2 = np.full_like(case.cache, BF16_QNAN)
    cache2[relabel] = case.cache
    table2 = np.where(case.block_table >= 0, relabel[np.maximum(case.block_table, 0)], -1).astype(np.int32)
    o2, l2 = orc.mla_decode(case.q, cache2, table2, case.seqlens, SCALE, True)
    _close(o1, o2, 1e-13, "page relabelling changes O")
    _close(l1, l2, 1e-13, "page relabelling changes LSE")


def pin_causal_rows(orc):
    case = make_case("pincausal", batch=2, s_q=2, heads=2, seqlen=[77, 1], seed=23, causal=True)
    o, lse = orc.mla_decode(case.q, case.cache, case.block_table, case.seqlens, SCALE, True)
    cf = bf16_bits_to_f32(case.cache).astype(np.float64)
    qf = bf16_bits_to_f32(case.q).astype(np.float64)
    L = 77
    keys = np.stack([cf[case.block_table[0, j // 64], j % 64] for j in range(L)])
    for i in range(2):
        n = L - 2 + 1 + i
        ro, rl = orc.attention(qf[0, i], keys[:n], keys[:n, :512], SCALE)
        _close(o[0, i], ro, 1e-13, f"causal token {i} sees {n} keys")
        _close(lse[0, i], rl, 1e-12, f"causal token {i} LSE")
    # L = 1: the first query token sees nothing, the second sees the one key
    assert np.all(o[1, 0] == 0.0) and np.all(np.isneginf(lse[1, 0])), "empty row must be O=0, LSE=-inf"
    key = cf[case.block_table[1, 0], 0]
    assert np.array_equal(o[1, 1], np.broadcast_to(key[:512], (2, 512)))


def pin_empty_sequence(orc):
    case = make_case("pinempty", batch=2, s_q=1, heads=2, seqlen=[0, 5], seed=24)
    o, lse = orc.mla_decode(case.q, case.cache, case.block_table, case.seqlens, SCALE, False)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(o[1])) and np.all(np.isfinite(lse[1]))


def pin_statistical_closed_form(orc):
    """Exponential tilting of N(0, I) keys: O -> scale q[:512], LSE -> ln L + scale^2 |q|^2 / 2."""
    L = 16384
    case = make_case("pinstat", batch=1, s_q=1, heads=4, seqlen=L, seed=25)
    qf = bf16_bits_to_f32(case.q).astype(np.float64)
    # shrink q so that scale^2 |q|^2 = 1 (keeps the estimator's noise at sqrt(e / L) ~ 0.013)
    shrink = 1.0 / (SCALE * np.linalg.norm(qf[0, 0], axis=-1, keepdims=True))
    q_bits = f32_to_bf16_bits((qf[0, 0] * shrink).astype(np.float32))[None, None]
    o, lse = orc.mla_decode(q_bits, case.cache, case.block_table, case.seqlens, SCALE, False)
    qs = bf16_bits_to_f32(q_bits[0, 0]).astype(np.float64)
    for hh in range(4):
        dev = o[0, 0, hh] - SCALE * qs[hh, :512]
        rms = float(np.sqrt(np.mean(dev * dev)))
        assert rms < 0.035, ("tilted mean of V", hh, rms)
        want = math.log(L) + 0.5 * SCALE * SCALE * float(qs[hh] @ qs[hh])
        assert abs(lse[0, 0, hh] - want) < 0.06, ("tilted LSE", hh, lse[0, 0, hh], want)


ALL_PINS = [pin_brute_force_dense, pin_brute_force_paged, pin_brute_force_page64, pin_transposed_identity,
            pin_single_key, pin_zero_query, pin_identical_keys, pin_probabilities_sum_to_one, pin_dominant_key,
            pin_split_invariance, pin_page_relabelling, pin_causal_rows, pin_empty_sequence,
            pin_statistical_closed_form]
