"""GPU parity where the plain workload tests leave gaps: work items longer than one 64-entry
block-table window, every split of the keys the plan can be told to make, and every row of the
two full-size workloads (with a zero query on the headline: LSE = ln L exactly, since every key
then weighs the same)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from mla_decode_attention_amd import workloads
from mla_decode_attention_amd.inputs import bf16_bits_to_f32, make_case

from gpu_helpers import log, parity, to_device

pytestmark = pytest.mark.gpu

ONE_ITEM = 1 << 30   # chunk larger than any sequence: one work item per sequence


def _decode_with_chunk(case, tensors, chunk, dev):
    """plan (mla_decode_plan_chunked) + fwd; returns float64 O, LSE and the raw bf16 / fp32 bits."""
    import torch

    import mla_decode_attention_amd as mla
    q, cache, bt, sl = tensors
    ws = torch.empty(mla.workspace_size(case.batch, case.s_q, case.heads), dtype=torch.uint8, device=dev)
    out = torch.empty((case.batch, case.s_q, case.heads, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((case.batch, case.s_q, case.heads), dtype=torch.float32, device=dev)
    mla.plan(sl, case.s_q, case.heads, ws, chunk_pages=chunk)
    mla.fwd(q, cache, bt, sl, case.softmax_scale, case.causal, ws, out, lse)
    torch.cuda.synchronize()
    ob = out.view(torch.int16).cpu().numpy().view(np.uint16)
    lb = lse.cpu().numpy()
    return bf16_bits_to_f32(ob).astype(np.float64), lb.astype(np.float64), ob, lb


def _items(case, tensors, chunk, dev):
    """(sequence, first page, end page) of the plan's work items."""
    import torch

    import mla_decode_attention_amd as mla
    sl = tensors[3]
    ws = torch.zeros(mla.workspace_size(case.batch, case.s_q, case.heads), dtype=torch.uint8, device=dev)
    mla.plan(sl, case.s_q, case.heads, ws, chunk_pages=chunk)
    torch.cuda.synchronize()
    w = ws.cpu().numpy()
    n_items = int(w[:64].view(np.int32)[4])
    a256 = lambda x: (x + 255) & ~255
    off = a256(a256(a256(64) + 4 * case.batch) + 4 * (case.batch + 1))
    return w[off:off + 16 * n_items].view(np.int32).reshape(-1, 4)[:, :3]


# (heads, s_q, causal): the 16-row kernel, the 32-row and 64-row forms of the wide kernel, and a
# head count whose last 32-row block is half empty
LONG_ITEM_CONFIGS = [(16, 1, False), (16, 2, True), (128, 1, False), (48, 2, True)]


@pytest.mark.parametrize("chunk", [ONE_ITEM, 100])
@pytest.mark.parametrize("heads,s_q,causal", LONG_ITEM_CONFIGS)
def test_items_longer_than_a_block_table_window(dev, heads, s_q, causal, chunk):
    """Items of up to 141 pages (one per sequence) or 100 pages starting off a window boundary: the
    kernels refill their 64-entry block-table window inside an item.  The pool holds four times the
    owned pages, the spare ones NaN, so a wrong page id shows as NaN instead of valid data."""
    lens = [9000, 300, 5000, 64 * 70 + 3]
    need = sum((L + 63) // 64 for L in lens)
    case = make_case(f"long_items_h{heads}_sq{s_q}", batch=len(lens), s_q=s_q, heads=heads, seqlen=lens, seed=71,
                     causal=causal, pool_pages=4 * need, table_slack=5)
    t = to_device(case, dev)
    items = _items(case, t, chunk, dev)
    longest = int((items[:, 2] - items[:, 1]).max())
    log(f"case {case.name} chunk={chunk}: {len(items)} items, longest {longest} pages")
    assert longest > 64
    o, l, _, _ = _decode_with_chunk(case, t, chunk, dev)
    ro, rl, rs = oracle.mla_decode(case.q, case.cache, case.block_table, case.seqlens, case.softmax_scale,
                                   case.causal, with_scale=True)
    parity(o, l, ro, rl, f"{case.name} chunk={chunk}", scale=rs)


@pytest.mark.parametrize("heads,s_q,causal", [(16, 1, False), (32, 1, False), (128, 1, False), (64, 2, True)])
def test_split_invariance_under_forced_chunks(dev, heads, s_q, causal):
    """The same inputs planned with 1-page items, 3-page items, the automatic split and one item per
    sequence: every result meets the bar against the oracle, and each plan gives the same bits on
    a rerun."""
    lens = [2000, 1500, 700, 1]
    case = make_case(f"split_inv_h{heads}_sq{s_q}", batch=len(lens), s_q=s_q, heads=heads, seqlen=lens, seed=72,
                     causal=causal, pool_pages=sum((L + 63) // 64 for L in lens) + 16)
    t = to_device(case, dev)
    ro, rl, rs = oracle.mla_decode(case.q, case.cache, case.block_table, case.seqlens, case.softmax_scale,
                                   case.causal, with_scale=True)
    for chunk in (1, 3, 0, ONE_ITEM):
        items = _items(case, t, chunk, dev)
        sizes = items[:, 2] - items[:, 1]
        if chunk in (1, 3):
            assert sizes.max() <= chunk, (chunk, sizes.tolist())
        elif chunk == ONE_ITEM:
            assert len(items) == sum(L > 0 for L in lens)
        o, l, ob, lb = _decode_with_chunk(case, t, chunk, dev)
        parity(o, l, ro, rl, f"{case.name} chunk={chunk} ({len(items)} items)", scale=rs)
        _, _, ob2, lb2 = _decode_with_chunk(case, t, chunk, dev)
        assert np.array_equal(ob, ob2) and np.array_equal(lb.view(np.int32), lb2.view(np.int32)), chunk


@pytest.fixture(scope="module")
def headline():
    log("generating the headline workload (1.2 GB of cache)")
    return workloads.build(workloads.HEADLINE)


def test_headline_every_row(dev, headline):
    """All 256 query rows of the headline workload, in the benchmark's launch configuration."""
    case = headline
    t = to_device(case, dev)
    o, l, _, _ = _decode_with_chunk(case, t, 0, dev)
    ro, rl, rs = oracle.mla_decode(case.q, case.cache, case.block_table, case.seqlens, case.softmax_scale,
                                   case.causal, with_scale=True)
    parity(o, l, ro, rl, f"{case.name} (all {case.rows} rows)", scale=rs)


def test_headline_zero_query(dev, headline):
    """q = 0 on the headline shape: every key weighs 1, so l counts the 65536 keys exactly and
    LSE = ln 65536 for every row (a tile dropped or read twice moves it by 1/65536); O is the mean
    of the value rows."""
    import torch
    case = headline
    q, cache, bt, sl = to_device(case, dev)
    q.zero_()
    o, l, _, _ = _decode_with_chunk(case, (q, cache, bt, sl), 0, dev)
    np.testing.assert_allclose(l, np.log(65536.0), rtol=1e-6)
    zq = np.zeros_like(case.q)
    ro, rl, rs = oracle.mla_decode(zq, case.cache, case.block_table, case.seqlens, case.softmax_scale, case.causal,
                                   with_scale=True)
    parity(o, l, ro, rl, f"{case.name} q=0", scale=rs)
    del q, cache, bt, sl
    torch.cuda.empty_cache()


def test_allheads_256_rows(dev):
    """256 of the 1024 query rows of the all-heads workload (all 128 heads of two sequences)."""
    case = workloads.build("allheads_b8_h128_L32768")
    t = to_device(case, dev)
    o, l, _, _ = _decode_with_chunk(case, t, 0, dev)
    rows = np.arange(3 * 128, 5 * 128)   # sequences 3 and 4, every head
    ro, rl, rs = oracle.mla_decode(case.q, case.cache, case.block_table, case.seqlens, case.softmax_scale,
                                   case.causal, rows=rows, with_scale=True)
    parity(o.reshape(case.rows, -1)[rows], l.reshape(-1)[rows], ro, rl, f"{case.name} (rows {rows[0]}..{rows[-1]})",
           scale=rs)
