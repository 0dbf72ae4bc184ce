"""GPU parity of the cache-append + rotary step (mla_cache_append_rope) against the fp64 oracle.

Bar: the latent copy and every cache row and query dim the step must not touch are bit-exact; each
rotated dim is the correctly rounded bf16 of the oracle's fp64 rotation (the kernel evaluates the
rotation in fp64 and rounds once, so |gpu - exact| <= half a bf16 ulp, up to fp64 noise); tokens
without a valid slot write nothing and get NaN query dims.
"""
import numpy as np
import pytest

from gpu_helpers import log
from mla_decode_attention_amd.inputs import make_append_inputs, make_case
from oracle import rope_append as RA

pytestmark = pytest.mark.gpu


def _f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _correctly_rounded(gpu_bits, exact):
    g = _f64(gpu_bits)
    e = np.floor(np.log2(np.maximum(np.abs(exact), 2.0 ** -126)))
    half_ulp = 0.5 * 2.0 ** (e - 7)
    return np.abs(g - exact) <= half_ulp * (1 + 1e-9)


def _run(case, lat_bits, rope_bits, dev, base=10000.0, bt=None):
    import torch

    import mla_decode_attention_amd as mla
    bt = case.block_table if bt is None else bt
    t = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    q = t(case.q)
    cache = t(case.cache)
    mla.cache_append_rope(t(lat_bits), t(rope_bits), q, cache, torch.from_numpy(bt).to(dev),
                          torch.from_numpy(case.seqlens).to(dev), base)
    torch.cuda.synchronize()
    return (q.view(torch.int16).cpu().numpy().view(np.uint16), cache.view(torch.int16).cpu().numpy().view(np.uint16))


def _check(case, lat_bits, rope_bits, q_gpu, cache_gpu, base=10000.0, bt=None):
    bt = case.block_table if bt is None else bt
    rows, q_rope = RA.append_rope(lat_bits, rope_bits, case.q, bt, case.seqlens, case.cache.shape[0], base)
    # cache: the written rows, and nothing else
    expect_changed = np.zeros(case.cache.shape[:2], dtype=bool)
    for (page, slot), (lat, key) in rows.items():
        expect_changed[page, slot] = True
        assert np.array_equal(cache_gpu[page, slot, :512], lat), f"latent of row {(page, slot)}"
        ok = _correctly_rounded(cache_gpu[page, slot, 512:], key)
        assert ok.all(), f"RoPE key of row {(page, slot)}: {np.flatnonzero(~ok)[:4]}"
    same = (cache_gpu == case.cache).all(axis=2)
    assert np.all(same | expect_changed), "a cache row outside the new tokens' slots changed"
    # query: latent dims untouched, RoPE dims rotated (NaN for tokens without a slot)
    assert np.array_equal(q_gpu[..., :512], case.q[..., :512]), "query latent dims changed"
    bad = np.isnan(q_rope)
    assert np.array_equal((q_gpu[..., 512:] & 0x7FFF) > 0x7F80, bad), "NaN pattern of the query RoPE dims"
    ok = _correctly_rounded(q_gpu[..., 512:][~bad], q_rope[~bad])
    assert ok.all(), f"{(~ok).sum()} query RoPE dims not correctly rounded"
    return len(rows), int(bad.any(axis=(-1, -2)).sum())   # tokens without a slot


@pytest.mark.parametrize("batch,s_q,heads,lens", [
    (16, 1, 16, (1, 4096)),
    (8, 2, 128, (2, 9000)),
    (4, 2, 16, [65536, 65535, 64, 3]),
])
def test_append_rope_matches_oracle(dev, batch, s_q, heads, lens):
    case = make_case(f"append_b{batch}_sq{s_q}_h{heads}", batch=batch, s_q=s_q, heads=heads, seqlen=lens,
                     seed=41, poison=False)
    lat, rope = make_append_inputs(case, seed=42)
    log(f"append {case.name}: lens {case.seqlens.tolist()[:6]}")
    q_gpu, cache_gpu = _run(case, lat, rope, dev)
    n_rows, n_bad = _check(case, lat, rope, q_gpu, cache_gpu)
    assert n_rows == batch * s_q and n_bad == 0


def test_append_invalid_tokens_write_nothing(dev):
    # L = 1 with two new tokens (token 0 at position -1), a page outside the pool, a length past
    # the table: no cache row for those tokens, NaN query RoPE dims
    case = make_case("append_bad", batch=4, s_q=2, heads=16, seqlen=[1, 300, 500, 70], seed=43, poison=False,
                     table_slack=1)
    lat, rope = make_append_inputs(case, seed=44)
    bt = case.block_table.copy()
    bt[1, (300 - 2) // 64] = case.cache.shape[0]          # sequence 1: bad page for its new tokens
    sl = case.seqlens.copy()
    sl[2] = 64 * bt.shape[1] + 1                            # sequence 2: longer than its table
    case.seqlens = sl
    q_gpu, cache_gpu = _run(case, lat, rope, dev, bt=bt)
    n_rows, n_bad = _check(case, lat, rope, q_gpu, cache_gpu, bt=bt)
    assert n_rows == 3 and n_bad == 5
