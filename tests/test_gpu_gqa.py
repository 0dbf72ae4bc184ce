"""GPU parity of the GQA path of GQLA (mla_gqa_decode_*) against the fp64 oracle, and the GQLA
equivalence on the GPU: over a cache expanded from a latent with a group's up-projections, the GQA
kernel and the absorbed chain (absorb -> latent decode -> un-absorb) both reproduce the same fp64
attention.

Bars: the decode bar (gpu_helpers) for parity; for the equivalence, whose GPU paths round the
expanded cache / the absorbed query and the outputs to bf16, max-abs <= 2e-2 max|o| and
RMSE <= 4e-3 rms(o) against the fp64 result on the unrounded weights.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import log, parity, to_device
from mla_decode_attention_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits, make_case
from oracle import absorb as AB
from oracle import gqa as G

pytestmark = pytest.mark.gpu

RAGGED = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 129, 1000, 4097]


def _gqa_case(name, batch, s_q, lens, seed, causal, **kw):
    return make_case(name, batch=batch, s_q=s_q, heads=16, seqlen=lens, seed=seed, causal=causal,
                     row_dims=G.ROW, q_dims=G.D_KEY, **kw)


def _run(case, dev, bt=None):
    import torch

    import mla_decode_attention_amd as mla
    q, cache, bt_d, sl = to_device(case, dev)
    if bt is not None:
        bt_d = torch.from_numpy(bt).to(dev)
    out, lse = mla.gqa_decode(q, cache, bt_d, sl, case.softmax_scale, case.causal)
    torch.cuda.synchronize()
    o = bf16_bits_to_f32(out.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return o, lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("batch,s_q,lens,causal", [
    (16, 2, (8192, 16384), True),
    (len(RAGGED), 1, RAGGED, False),
    (len(RAGGED), 2, RAGGED, True),
    (5, 2, [0, 1, 2, 0, 70], True),
])
def test_gqa_matches_oracle(dev, batch, s_q, lens, causal):
    case = _gqa_case(f"gqa_b{batch}_sq{s_q}", batch, s_q, lens, seed=71, causal=causal)
    log(f"gqa {case.name}: lens {case.seqlens.tolist()[:6]} causal={causal}")
    o, l = _run(case, dev)
    ro, rl = G.gqa_decode(case.q, case.cache, case.block_table, case.seqlens, case.softmax_scale, causal)
    parity(o, l, ro, rl, case.name)


@pytest.mark.parametrize("s_q", [1, 2])
def test_gqa_items_longer_than_a_block_table_window(dev, s_q):
    """More sequences than resident split workgroups (512 with one query token, 256 with two), so
    the plan makes every sequence one work item and the long ones span up to 141 pages: the kernel
    refills its 64-entry block-table window inside an item, with two tiles in flight per wave.  The
    pool holds four times the owned pages, the spare ones NaN, so a wrong page id shows."""
    rng = np.random.default_rng(77 + s_q)
    lens = [int(x) for x in rng.integers(0, 100, 520)]
    lens[5], lens[100], lens[300], lens[511] = 9000, 5000, 64 * 70 + 3, 64 * 65
    need = sum((L + 63) // 64 for L in lens)
    case = _gqa_case(f"gqa_long_items_sq{s_q}", len(lens), s_q, lens, seed=78, causal=s_q == 2,
                     pool_pages=4 * need, table_slack=5)
    log(f"gqa {case.name}: {len(lens)} sequences, longest {max(lens)} tokens, pool {4 * need} pages")
    o, l = _run(case, dev)
    ro, rl = G.gqa_decode(case.q, case.cache, case.block_table, case.seqlens, case.softmax_scale, case.causal)
    parity(o, l, ro, rl, case.name)


def test_gqa_bad_page_gives_nan(dev):
    case = _gqa_case("gqa_bad", 3, 2, [300, 200, 500], seed=72, causal=True)
    bt = case.block_table.copy()
    bt[1, 1] = case.cache.shape[0]
    o, l = _run(case, dev, bt=bt)
    assert np.isnan(l[1]).all() and np.isnan(o[1]).all()
    ro, rl = G.gqa_decode(case.q, case.cache, case.block_table, case.seqlens, case.softmax_scale, True)
    parity(o[[0, 2]], l[[0, 2]], ro[[0, 2]], rl[[0, 2]], "valid sequences beside a bad one")


def test_gqa_path_and_absorbed_path_agree_on_gpu(dev):
    import torch

    import mla_decode_attention_amd as mla
    rng = np.random.default_rng(73)
    lat_case = make_case("gqla_latent", batch=3, s_q=2, heads=16, seqlen=[900, 64, 2500], seed=74, causal=True,
                         poison=False)
    lat = bf16_bits_to_f32(lat_case.cache[..., :512]).astype(np.float64)
    rope = bf16_bits_to_f32(lat_case.cache[..., 512:]).astype(np.float64)
    w_uk = (rng.standard_normal((512, 128)) / 16).astype(np.float32)
    w_uv = (rng.standard_normal((128, 512)) / 16).astype(np.float32)
    wuk_b, wuv_b = f32_to_bf16_bits(w_uk), f32_to_bf16_bits(w_uv)
    wuk64 = bf16_bits_to_f32(wuk_b).astype(np.float64)
    wuv64 = bf16_bits_to_f32(wuv_b).astype(np.float64)
    # GQA cache: the group's keys and values expanded from the latent, rounded to bf16
    gqa_cache = f32_to_bf16_bits(np.concatenate([lat @ wuk64, rope, lat @ wuv64.T], axis=-1).astype(np.float32))
    q_nope = f32_to_bf16_bits(rng.standard_normal((3, 2, 16, 128)).astype(np.float32))
    q_rope = lat_case.q[..., 512:]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    bt = torch.from_numpy(lat_case.block_table).to(dev)
    sl = torch.from_numpy(lat_case.seqlens).to(dev)
    # GQA path
    og, _ = mla.gqa_decode(t(np.concatenate([q_nope, q_rope], axis=-1)), t(gqa_cache), bt, sl,
                           lat_case.softmax_scale, True)
    # absorbed path: absorb -> latent decode -> un-absorb
    qa = mla.absorb_q(t(q_nope), t(q_rope), t(np.broadcast_to(wuk_b, (16, 512, 128))))
    ol, _ = mla.decode(qa, t(lat_case.cache), bt, sl, lat_case.softmax_scale, True)
    oa = mla.unabsorb_o(ol, t(np.broadcast_to(wuv_b, (16, 128, 512))))
    torch.cuda.synchronize()
    f = lambda x: bf16_bits_to_f32(x.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    og, oa = f(og), f(oa)
    # fp64 reference: the absorbed chain on the exact (unrounded-weight-product) values
    ref = np.zeros_like(og)
    qn = bf16_bits_to_f32(q_nope).astype(np.float64)
    qr = bf16_bits_to_f32(q_rope).astype(np.float64)
    for b in range(3):
        L = int(lat_case.seqlens[b])
        pos = np.arange(L)
        pg = lat_case.block_table[b, pos // 64]
        c, r = lat[pg, pos % 64], rope[pg, pos % 64]
        for i in range(2):
            n = L - 2 + 1 + i
            q = AB.absorb_q(qn[b, i], qr[b, i], np.broadcast_to(wuk64, (16, 512, 128)))
            o_lat, _ = oracle.attention(q, np.concatenate([c[:n], r[:n]], axis=1), c[:n], lat_case.softmax_scale)
            ref[b, i] = AB.unabsorb_o(o_lat, np.broadcast_to(wuv64, (16, 128, 512)))
    for what, o in (("GQA path", og), ("absorbed path", oa)):
        e = o - ref
        mx, rmse = float(np.abs(e).max()), float(np.sqrt(np.mean(e ** 2)))
        log(f"{what}: max-abs {mx:.3e} (max|o| {np.abs(ref).max():.3f}) rmse {rmse:.3e} (rms {np.sqrt(np.mean(ref**2)):.3f})")
        assert mx <= 2e-2 * np.abs(ref).max() and rmse <= 4e-3 * np.sqrt(np.mean(ref ** 2)), what
