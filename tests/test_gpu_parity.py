"""GPU parity: the HIP path through the C ABI against the fp64 oracle, element by element."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from mla_decode_attention_amd import workloads
from mla_decode_attention_amd.inputs import make_case

from gpu_helpers import log, parity, run_gpu, to_device

pytestmark = pytest.mark.gpu


def full_parity(case, dev, what=None):
    what = what or case.name
    log(f"case {what}: b={case.batch} s_q={case.s_q} h={case.heads} L={case.seqlens.tolist()[:6]} "
        f"causal={case.causal} pages={case.num_pages}")
    o, l = run_gpu(case, dev)
    ro, rl, rs = oracle.mla_decode(case.q, case.cache, case.block_table, case.seqlens, case.softmax_scale,
                                   case.causal, with_scale=True)
    return parity(o, l, ro, rl, what, scale=rs)


@pytest.mark.parametrize("name", ["tiny_b1_h16_L256", "paged_b16_h16_L4096", "mtp_b16_h16_sq2_L8K-16K"])
def test_workload_full(dev, name):
    full_parity(workloads.build(name), dev)


RAGGED = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 129, 1000, 4097]


@pytest.mark.parametrize("heads,s_q,causal", [(16, 1, False), (16, 2, True), (16, 2, False), (32, 1, False),
                                             (32, 2, True), (64, 1, False), (64, 2, True), (128, 1, False),
                                             (128, 2, True), (48, 1, False), (48, 2, True), (80, 1, False),
                                             (80, 2, True), (96, 1, False), (96, 2, True), (112, 1, False),
                                             (112, 2, True)])
def test_ragged_lengths_all_row_configs(dev, heads, s_q, causal):
    lens = RAGGED if heads <= 32 else RAGGED[:10] + [700]
    case = make_case(f"ragged_h{heads}_sq{s_q}", batch=len(lens), s_q=s_q, heads=heads, seqlen=lens, seed=31,
                     causal=causal, pool_pages=sum((L + 63) // 64 for L in lens) + 5, table_slack=3)
    full_parity(case, dev)


def _sweep_params(n=16, seed=4242):
    """Seeded shapes for the sweep: head count, query tokens, causal flag, batch, a length mix
    (wide random, page multiples +-1, tiny) and the softmax scale (including 0 and a negative)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        heads = int(rng.choice([16, 32, 64, 128]))
        s_q = int(rng.integers(1, 3))
        causal = bool(rng.integers(0, 2))
        batch = int(rng.integers(1, 5 if heads >= 64 else 13))
        kind = int(rng.integers(0, 3))
        top = 3000 if heads >= 64 else 6000
        if kind == 0:
            lens = rng.integers(0, top, size=batch)
        elif kind == 1:
            lens = np.clip(64 * rng.integers(0, top // 64, size=batch) + rng.integers(-1, 2, size=batch), 0, None)
        else:
            lens = rng.integers(0, 130, size=batch)
        scale = float(rng.choice([1.0 / np.sqrt(192.0), 0.02, 0.25, -0.08, 0.0]))
        out.append(pytest.param(heads, s_q, causal, [int(x) for x in lens], scale, 5000 + i, id=f"sweep{i}"))
    return out


@pytest.mark.parametrize("heads,s_q,causal,lens,scale,seed", _sweep_params())
def test_seeded_shape_sweep(dev, heads, s_q, causal, lens, scale, seed):
    case = make_case(f"sweep_h{heads}_sq{s_q}", batch=len(lens), s_q=s_q, heads=heads, seqlen=lens, seed=seed,
                     causal=causal, softmax_scale=scale, pool_pages=sum((L + 63) // 64 for L in lens) + 3,
                     table_slack=2)
    full_parity(case, dev, f"{case.name} scale={scale:.4g}")


@pytest.mark.parametrize("heads", [16, 64, 128])
def test_empty_and_single_key_sequences(dev, heads):
    """Empty sequences (no work item), one and two keys (a causal first token that sees nothing or
    one key), in the 32-row, 128-row and 256-row forms."""
    case = make_case(f"empty_mix_h{heads}", batch=5, s_q=2, heads=heads, seqlen=[0, 1, 2, 0, 70], seed=32,
                     causal=True)
    full_parity(case, dev)


def test_zero_query_gives_mean_value(dev):
    case = make_case("zero_q", batch=2, s_q=1, heads=16, seqlen=[300, 4000], seed=33, zero_q=True)
    o, l = run_gpu(case, dev)
    np.testing.assert_allclose(l, np.log(case.seqlens.astype(np.float64))[:, None, None].repeat(16, 2),
                               rtol=1e-6)
    full_parity(case, dev)


def test_outlier_rows_softmax_max_tracking(dev):
    case = make_case("outliers", batch=4, s_q=2, heads=32, seqlen=(3000, 9000), seed=34, causal=True,
                     outlier_frac=0.01, outlier_scale=8.0)
    full_parity(case, dev)


@pytest.mark.parametrize("heads,s_q", [(16, 1), (16, 2), (128, 1)])
def test_deterministic_for_a_plan(dev, heads, s_q):
    """The same inputs and plan give bit-identical O and LSE on a rerun, in every kernel form."""
    import torch

    import mla_decode_attention_amd as mla
    causal = s_q == 2
    case = make_case(f"det_h{heads}_sq{s_q}", batch=3, s_q=s_q, heads=heads, seqlen=[5000, 130, 2048], seed=35,
                     causal=causal)
    q, cache, bt, sl = to_device(case, dev)
    out1, lse1 = mla.decode(q, cache, bt, sl, case.softmax_scale, causal)
    out2, lse2 = out1.clone(), lse1.clone()
    out1.zero_()
    mla.fwd(q, cache, bt, sl, case.softmax_scale, causal, *_workspace_for(mla, case, sl, dev), out1, lse1)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16)) and torch.equal(lse1, lse2)


def _workspace_for(mla, case, sl, dev):
    import torch
    ws = torch.empty(mla.workspace_size(case.batch, case.s_q, case.heads), dtype=torch.uint8, device=dev)
    mla.plan(sl, case.s_q, case.heads, ws)
    return (ws,)


@pytest.mark.parametrize("heads,s_q", [(16, 1), (16, 2), (128, 1), (48, 2)])
def test_bad_page_and_mismatched_plan_give_nan_not_fault(dev, heads, s_q):
    """A page id outside the pool poisons only its sequence (NaN O and LSE), in the 16-row kernel
    and in the paired kernel's 32-row and 64-row forms; a plan made for other lengths or another
    head count poisons the whole batch.  No case reads outside the cache."""
    import torch

    import mla_decode_attention_amd as mla
    causal = s_q == 2
    case = make_case(f"badpage_h{heads}_sq{s_q}", batch=3, s_q=s_q, heads=heads, seqlen=[200, 300, 100], seed=36,
                     causal=causal)
    q, cache, bt, sl = to_device(case, dev)
    bt_bad = bt.clone()
    bt_bad[1, 2] = case.num_pages + 7          # out of the pool
    out, lse = mla.decode(q, cache, bt_bad, sl, case.softmax_scale, causal)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    assert np.isnan(o[1]).all() and np.isnan(l[1]).all()
    ro, rl = oracle.mla_decode(case.q, case.cache, case.block_table, case.seqlens, case.softmax_scale, causal)
    parity(o[[0, 2]], l[[0, 2]], ro[[0, 2]], rl[[0, 2]], f"sequences beside a bad page (h{heads} s_q{s_q})")
    # plan made for other seqlens
    ws = torch.empty(mla.workspace_size(3, s_q, heads), dtype=torch.uint8, device=dev)
    mla.plan(sl + 1, s_q, heads, ws)
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    mla.fwd(q, cache, bt, sl, case.softmax_scale, causal, ws, out2, lse2)
    torch.cuda.synchronize()
    assert torch.isnan(lse2).all()
    # plan made for another head count: the whole batch is NaN
    other = 32 if heads != 32 else 64
    nbytes = max(mla.workspace_size(3, s_q, other), mla.workspace_size(3, s_q, heads))
    ws3 = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    mla.plan(sl, s_q, other, ws3)
    mla.fwd(q, cache, bt, sl, case.softmax_scale, causal, ws3, out2, lse2)
    torch.cuda.synchronize()
    assert torch.isnan(lse2).all() and torch.isnan(out2.float()).all()


def test_workspace_too_small_is_reported(dev):
    import torch

    import mla_decode_attention_amd as mla
    case = make_case("ws", batch=2, s_q=1, heads=16, seqlen=[64, 64], seed=37)
    q, cache, bt, sl = to_device(case, dev)
    need = mla.workspace_size(2, 1, 16)
    ws = torch.empty(need - 256, dtype=torch.uint8, device=dev)
    with pytest.raises(mla.MlaDecodeError) as e:
        mla.plan(sl, 1, 16, ws)
    assert e.value.status == -3


def _long_batch_lens(batch, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 300, batch)
    lens[::7] = 0
    lens[3::11] = rng.integers(1000, 3000, len(lens[3::11]))
    return [int(x) for x in lens]


def _plan_lens(kind):
    rng = np.random.default_rng(47)
    return {
        "mixed": lambda: [0, 1, 64, 65, 5000, 65536, 12345, 3],
        "batch_beyond_slots": lambda: _long_batch_lens(300, 41),
        "all_empty": lambda: [0] * 9,
        "one_huge": lambda: [0, 1, 262144, 5],
        "many_tiny": lambda: [int(x) for x in rng.integers(1, 65, 200)],
        "uneven_like_mtp": lambda: [int(x) for x in rng.integers(8192, 16385, 16)],
        "batch_near_slots": lambda: [int(x) for x in rng.integers(0, 5000, 120)],
        # the plan reads only the lengths: page counts near 2^25 (INT_MAX tokens) must not overflow
        "near_int_max": lambda: [2 ** 31 - 1, 2 ** 31 - 64, 5, 0],
        # the headline's lengths: a plan large enough for the XCD weighting of the items
        "headline_like": lambda: [65536] * 16,
        # more sequences than the plan kernel keeps in registers (4 per thread of 1024)
        "beyond_register_cache": lambda: [int(x) for x in rng.integers(0, 300, 5000)],
    }[kind]()


@pytest.mark.parametrize("lens_kind", ["mixed", "batch_beyond_slots", "all_empty", "one_huge", "many_tiny",
                                       "uneven_like_mtp", "batch_near_slots", "near_int_max", "headline_like",
                                       "beyond_register_cache"])
def test_plan_covers_every_page_once(dev, lens_kind):
    """Read the plan back: items tile each sequence's pages exactly once, in balanced chunks of the
    smallest size that fits one wave of split workgroups (one item per sequence once the batch
    reaches the number of workgroup slots)."""
    import torch

    import mla_decode_attention_amd as mla
    lens = _plan_lens(lens_kind)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    for s_q, heads in [(1, 16), (2, 16), (1, 128), (2, 128)]:
        ws = torch.zeros(mla.workspace_size(len(lens), s_q, heads), dtype=torch.uint8, device=dev)
        mla.plan(sl, s_q, heads, ws)
        torch.cuda.synchronize()
        w = ws.cpu().numpy()
        hdr = w[:64].view(np.int32)
        assert hdr[0] == 0x4D4C4131 and hdr[1] == len(lens) and hdr[2] == s_q and hdr[3] == heads
        n_items, cap, rows = int(hdr[4]), int(hdr[5]), int(hdr[6])
        assert rows == s_q * heads and n_items <= cap

        def a256(x):
            return (x + 255) & ~255
        off = a256(64)
        off_len = off
        off = a256(off + 4 * len(lens))
        off_bs = off
        off = a256(off + 4 * (len(lens) + 1))
        off_items = off
        assert w[off_len:off_len + 4 * len(lens)].view(np.int32).tolist() == lens
        bs = w[off_bs:off_bs + 4 * (len(lens) + 1)].view(np.int32)
        items = w[off_items:off_items + 16 * n_items].view(np.int32).reshape(-1, 4)
        assert bs[0] == 0 and bs[-1] == n_items and np.all(np.diff(bs) >= 0)
        sizes = []
        for b, L in enumerate(lens):
            its = items[bs[b]:bs[b + 1]]
            pages = (L + 63) // 64
            assert (its[:, 0] == b).all()
            assert its[:, 3].tolist() == list(range(len(its)))
            # the item ranges tile [0, pages) in order, each non-empty
            if pages == 0:
                assert len(its) == 0, (b, L)
            else:
                assert its[0, 1] == 0 and its[-1, 2] == pages, (b, L)
                assert (its[1:, 1] == its[:-1, 2]).all() and (its[:, 2] > its[:, 1]).all(), (b, L)
            sizes += (its[:, 2] - its[:, 1]).tolist()
            sz = its[:, 2] - its[:, 1]
            # the split points, exactly: floor(s pg / n), or with 16 : 15 weights for even : odd items
            n = len(its)
            if n:
                weighted = sum((x + 63) // 64 for x in lens) >= 8192 and pages >= 8 * n
                ev0 = 1 if bs[b] % 2 == 0 else 0

                def point(k):
                    if not weighted:
                        return k * pages // n
                    e, en = (k + ev0) // 2, (n + ev0) // 2
                    return pages * (16 * e + 15 * (k - e)) // (16 * en + 15 * (n - en))
                assert its[:, 1].tolist() == [point(k) for k in range(n)], (b, L)
                assert its[:, 2].tolist() == [point(k + 1) for k in range(n)], (b, L)
            if len(its) > 1 and pages >= 8 * len(its) and sum((x + 63) // 64 for x in lens) >= 8192:
                # weighted (large plans): even-index items are not smaller
                idx = np.arange(bs[b], bs[b + 1])
                assert sz[idx % 2 == 0].min() >= sz[idx % 2 == 1].max() - 1, (b, L, sz.tolist())
        # the chunk is the smallest page count whose per-sequence split counts fit the
        # cap - batch workgroup slots (one wave of split workgroups)
        slots = cap - len(lens)
        pages = [(L + 63) // 64 for L in lens]
        if slots > len(lens):
            lo, hi = 1, max(pages) + 1   # smallest c with sum ceil(p / c) <= slots (bisection: it is monotone)
            while lo < hi:
                mid = (lo + hi) // 2
                if sum(-(-p // mid) for p in pages) <= slots:
                    hi = mid
                else:
                    lo = mid + 1
            chunk = lo
            # items of 8 pages or more are weighted 16:15 between even and odd XCDs (item x runs on
            # XCD x % 8), so an even-XCD item may exceed the even-split chunk by up to 1/15.5
            assert n_items <= slots and max(sizes, default=0) <= chunk + chunk // 15 + 1
        else:   # every sequence is one item
            chunk = max(pages)
            assert n_items == sum(p > 0 for p in pages)
        log(f"plan s_q={s_q} h={heads}: {n_items} items (capacity {cap}), chunk {chunk}, "
            f"sizes {min(sizes, default=0)}..{max(sizes, default=0)}")


@pytest.mark.parametrize("heads,s_q,batch", [(16, 1, 300), (16, 2, 300), (128, 1, 140)])
def test_batch_beyond_workgroup_slots(dev, heads, s_q, batch):
    """More sequences than resident split workgroups: the plan makes one item per sequence and the
    extra workgroups run as later waves; every row still matches the oracle."""
    lens = _long_batch_lens(batch, 42 + heads + s_q)
    case = make_case(f"batch{batch}_h{heads}_sq{s_q}", batch=batch, s_q=s_q, heads=heads, seqlen=lens, seed=43,
                     causal=s_q == 2)
    full_parity(case, dev)
