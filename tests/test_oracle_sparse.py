"""Pins of the sparse (top-k) decode oracle, CPU only.

The sparse step is the attention definition over a gathered key set, so it is pinned against the
dense decode oracle (all positions listed in order), against invariances (order of the list, -1
slots), and against closed forms (one row listed k times: O = v, LSE = s + ln k), plus the error
rules (an index past L_b or a row on a page outside the pool gives NaN; no index gives O = 0,
LSE = -inf).
"""
import math

import numpy as np

import oracle
from mla_decode_attention_amd.inputs import make_case, make_sparse_indices


def _case(lens=(37, 130, 64), s_q=2, seed=5):
    return make_case("sparse_pin", batch=len(lens), s_q=s_q, heads=16, seqlen=list(lens), seed=seed)


def test_all_positions_in_order_equal_dense_decode():
    c = _case()
    topk = int(c.seqlens.max())
    ind = np.full((c.batch, c.s_q, topk), -1, dtype=np.int32)
    for b in range(c.batch):
        ind[b, :, : c.seqlens[b]] = np.arange(c.seqlens[b])
    o, l = oracle.sparse_decode(c.q, c.cache, c.block_table, c.seqlens, ind, c.softmax_scale)
    ro, rl = oracle.mla_decode(c.q, c.cache, c.block_table, c.seqlens, c.softmax_scale, False)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, rl, rtol=1e-14)


def test_order_and_unused_slots_do_not_matter():
    c = _case(seed=6)
    ind = make_sparse_indices(c, 48, seed=7)
    o1, l1 = oracle.sparse_decode(c.q, c.cache, c.block_table, c.seqlens, ind, c.softmax_scale)
    rng = np.random.default_rng(8)
    wide = np.full((c.batch, c.s_q, 80), -1, dtype=np.int32)
    for b in range(c.batch):
        for i in range(c.s_q):
            slots = rng.choice(80, size=48, replace=False)
            wide[b, i, slots] = rng.permutation(ind[b, i])
    o2, l2 = oracle.sparse_decode(c.q, c.cache, c.block_table, c.seqlens, wide, c.softmax_scale)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=1e-14)


def test_one_row_listed_k_times():
    c = _case(lens=(200,), s_q=1, seed=9)
    k, pos = 5, 123
    ind = np.full((1, 1, 8), -1, dtype=np.int32)
    ind[0, 0, :k] = pos
    o, l = oracle.sparse_decode(c.q, c.cache, c.block_table, c.seqlens, ind, c.softmax_scale)
    page = c.block_table[0, pos // 64]
    row = (c.cache[page, pos % 64].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q = (c.q[0, 0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(o[0, 0], np.broadcast_to(row[:512], (16, 512)))
    s = c.softmax_scale * (q @ row)
    np.testing.assert_allclose(l[0, 0], s + math.log(k), rtol=1e-14)


def test_error_rules():
    c = _case(lens=(100, 100, 100), s_q=1, seed=10)
    ind = make_sparse_indices(c, 16, seed=11)
    ind[0, 0, 3] = 100                     # past L_0
    bt = c.block_table.copy()
    bt[1, :] = c.num_pages                 # every page of sequence 1 outside the pool
    ind[2, 0, :] = -1                      # no index at all
    o, l = oracle.sparse_decode(c.q, c.cache, bt, c.seqlens, ind, c.softmax_scale)
    assert np.isnan(o[0]).all() and np.isnan(l[0]).all()
    assert np.isnan(o[1]).all() and np.isnan(l[1]).all()
    assert (o[2] == 0).all() and np.isneginf(l[2]).all()
