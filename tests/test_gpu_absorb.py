"""GPU parity of the absorption steps (mla_absorb_q, mla_unabsorb_o) against the fp64 oracle, and of
the whole absorbed chain against decompressed per-head attention.

Per-element bar, from the arithmetic: bf16 products are exact in fp32, fp32 accumulation over
K <= 512 terms adds at most ~K 2^-24 sum|a w| and the output is rounded once to bf16 (2^-9
relative), so |gpu - exact| <= 2^-8 |exact| + 2^-13 sum_k |a_k w_k| (twice each term).
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import log
from mla_decode_attention_amd.inputs import bf16_bits_to_f32, make_absorb_inputs, make_case
from oracle import absorb as AB

pytestmark = pytest.mark.gpu


def _f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _t(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _within_bar(gpu, exact, absdot):
    return np.abs(gpu - exact) <= 2.0 ** -8 * np.abs(exact) + 2.0 ** -13 * absdot


@pytest.mark.parametrize("batch,s_q,heads", [(16, 1, 16), (8, 2, 128), (3, 2, 32), (1, 1, 64)])
def test_absorb_and_unabsorb_match_oracle(dev, batch, s_q, heads):
    import torch

    import mla_decode_attention_amd as mla
    qn, qr, wuk, wuv = make_absorb_inputs(batch, s_q, heads, seed=61)
    log(f"absorb b={batch} s_q={s_q} h={heads}")
    q = mla.absorb_q(_t(qn, dev), _t(qr, dev), _t(wuk, dev))
    ol = np.random.default_rng(62).standard_normal((batch, s_q, heads, 512)).astype(np.float32)
    from mla_decode_attention_amd.inputs import f32_to_bf16_bits
    ol_bits = f32_to_bf16_bits(ol)
    o = mla.unabsorb_o(_t(ol_bits, dev), _t(wuv, dev))
    torch.cuda.synchronize()
    q_gpu, o_gpu = _f64(_bits(q)), _f64(_bits(o))
    exact_q = AB.absorb_q(_f64(qn), _f64(qr), _f64(wuk))
    absdot_q = np.einsum("hnk,...hk->...hn", np.abs(_f64(wuk)), np.abs(_f64(qn)))
    assert np.array_equal(_bits(q)[..., 512:], qr), "RoPE part must be copied bit for bit"
    ok = _within_bar(q_gpu[..., :512], exact_q[..., :512], absdot_q)
    assert ok.all(), f"absorb: {(~ok).sum()} elements off the bar"
    exact_o = AB.unabsorb_o(_f64(ol_bits), _f64(wuv))
    absdot_o = np.einsum("hdn,...hn->...hd", np.abs(_f64(wuv)), np.abs(_f64(ol_bits)))
    ok = _within_bar(o_gpu, exact_o, absdot_o)
    assert ok.all(), f"unabsorb: {(~ok).sum()} elements off the bar"


def test_absorbed_chain_on_gpu_matches_decompressed_attention(dev):
    """absorb -> decode over the latent cache -> un-absorb, against fp64 decompressed attention.
    Three bf16 roundings sit on the GPU chain (absorbed query, decode output, final output), so the
    bar is the decode bar scaled by the output's magnitude: max-abs <= 2e-2 max|o|, RMSE <= 4e-3 rms(o)."""
    import torch

    import mla_decode_attention_amd as mla
    case = make_case("absorb_chain", batch=4, s_q=1, heads=16, seqlen=[700, 64, 3000, 1], seed=63)
    qn, qr, wuk, wuv = make_absorb_inputs(case.batch, case.s_q, case.heads, seed=64)
    q = mla.absorb_q(_t(qn, dev), _t(qr, dev), _t(wuk, dev))
    from gpu_helpers import to_device
    _, cache, bt, sl = to_device(case, dev)
    out, lse = mla.decode(q, cache, bt, sl, case.softmax_scale, False)
    o = mla.unabsorb_o(out, _t(wuv, dev))
    torch.cuda.synchronize()
    o_gpu = _f64(_bits(o))
    err_max, ref_max, sq_err, sq_ref = 0.0, 0.0, 0.0, 0.0
    for b in range(case.batch):
        L = int(case.seqlens[b])
        pos = np.arange(L)
        rows = _f64(case.cache[case.block_table[b, pos // 64], pos % 64])
        ro, _ = AB.decompressed_attention(_f64(qn[b, 0]), _f64(qr[b, 0]), rows[:, :512], rows[:, 512:],
                                          _f64(wuk), _f64(wuv), case.softmax_scale)
        e = o_gpu[b, 0] - ro
        err_max = max(err_max, float(np.abs(e).max()))
        ref_max = max(ref_max, float(np.abs(ro).max()))
        sq_err += float((e ** 2).sum())
        sq_ref += float((ro ** 2).sum())
    rmse, rms = (sq_err / o_gpu.size) ** 0.5, (sq_ref / o_gpu.size) ** 0.5
    log(f"absorbed chain: max-abs {err_max:.3e} (max |o| {ref_max:.3f}), rmse {rmse:.3e} (rms {rms:.3f})")
    assert err_max <= 2e-2 * ref_max and rmse <= 4e-3 * rms
