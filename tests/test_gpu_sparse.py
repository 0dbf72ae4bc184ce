"""GPU parity of the sparse (top-k) decode path (mla_sparse_decode_*) against the fp64 oracle.

Same bar as the dense decode (O max-abs 1e-2 / RMSE 2e-3 normalised as in gpu_helpers, LSE relative
1e-4), element by element over every row; index lists cover ragged top-k (not a multiple of the
16-token tile, longer than the sequence), unused -1 slots, positions listed twice and 64K contexts;
error rules are checked element by element too.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import log, parity, to_device
from mla_decode_attention_amd.inputs import bf16_bits_to_f32, make_case, make_sparse_indices

pytestmark = pytest.mark.gpu


def _run(case, ind, dev, bt=None):
    import torch

    import mla_decode_attention_amd as mla
    q, cache, bt_d, sl = to_device(case, dev)
    if bt is not None:
        bt_d = torch.from_numpy(bt).to(dev)
    out, lse = mla.sparse_decode(q, cache, bt_d, sl, torch.from_numpy(ind).to(dev), case.softmax_scale)
    torch.cuda.synchronize()
    o = bf16_bits_to_f32(out.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return o, lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("batch,s_q,lens,topk,pad,dup", [
    (4, 1, (1, 5000), 2048, 0.0, False),
    (3, 2, [100, 2000, 70000], 64, 0.1, True),
    (5, 1, [10, 17, 33, 300, 4096], 17, 0.3, False),
    (2, 2, [65536, 40000], 4096, 0.0, False),
    (16, 1, (8192, 16384), 1, 0.0, False),
])
def test_sparse_decode_matches_oracle(dev, batch, s_q, lens, topk, pad, dup):
    case = make_case(f"sparse_b{batch}_sq{s_q}_k{topk}", batch=batch, s_q=s_q, heads=16, seqlen=lens, seed=51)
    ind = make_sparse_indices(case, topk, seed=52, pad_frac=pad, duplicates=dup)
    log(f"sparse {case.name}: lens {case.seqlens.tolist()[:6]} topk {topk}")
    o, l = _run(case, ind, dev)
    ro, rl = oracle.sparse_decode(case.q, case.cache, case.block_table, case.seqlens, ind, case.softmax_scale)
    parity(o, l, ro, rl, case.name)


def test_sparse_all_positions_match_dense_decode(dev):
    from gpu_helpers import run_gpu
    case = make_case("sparse_vs_dense", batch=3, s_q=1, heads=16, seqlen=[300, 1000, 64], seed=53)
    topk = int(case.seqlens.max())
    ind = np.full((case.batch, 1, topk), -1, dtype=np.int32)
    for b in range(case.batch):
        ind[b, 0, : case.seqlens[b]] = np.random.default_rng(b).permutation(case.seqlens[b])
    o, l = _run(case, ind, dev)
    od, ld = run_gpu(case, dev)
    ro, rl = oracle.mla_decode(case.q, case.cache, case.block_table, case.seqlens, case.softmax_scale, False)
    parity(o, l, ro, rl, "sparse, every position")
    parity(od, ld, ro, rl, "dense")


def test_sparse_error_rules(dev):
    case = make_case("sparse_bad", batch=4, s_q=2, heads=16, seqlen=[500, 500, 500, 500], seed=54)
    ind = make_sparse_indices(case, 40, seed=55)
    ind[0, 1, 7] = 500                       # token (0, 1): index past L_0
    bt = case.block_table.copy()
    bt[1, :] = case.num_pages                # sequence 1: every page outside the pool
    ind[2, 0, :] = -1                        # token (2, 0): no index
    o, l = _run(case, ind, dev, bt=bt)
    ro, rl = oracle.sparse_decode(case.q, case.cache, bt, case.seqlens, ind, case.softmax_scale)
    nan_tok = np.isnan(rl).all(axis=-1)
    assert nan_tok.tolist() == [[False, True], [True, True], [False, False], [False, False]]
    assert np.array_equal(np.isnan(l), np.isnan(rl)) and np.isnan(o[nan_tok]).all()
    assert (o[2, 0] == 0).all() and np.isneginf(l[2, 0]).all()
    ok = ~nan_tok
    parity(o[ok], l[ok], ro[ok], rl[ok], "valid tokens next to bad ones")
