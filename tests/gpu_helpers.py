"""Shared helpers for the GPU tests: device upload, one decode through the C ABI, the parity bar."""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

from mla_decode_attention_amd.inputs import DecodeCase, bf16_bits_to_f32

# Tolerances of the decode step against the fp64 oracle: O max-abs <= 1e-2 and RMSE <= 2e-3,
# LSE relative error <= 1e-4.  Errors in O are divided by max(1, scale of O_ref) (max |O_ref| for
# max-abs, rms(O_ref) for RMSE) -- identical to the literal bar whenever |O| <= 1, and the only
# reading that a bf16 output can meet when softmax mass concentrates on x8 outlier rows and |O|
# reaches ~32 (rounding the exact result to bf16 alone then costs 0.0625).  LSE error is divided
# by max(1, |LSE_ref|).
O_MAXABS = 1e-2
O_RMSE = 2e-3
LSE_REL = 1e-4
# Per element, whatever the scale of O: the literal max-abs bar plus what bf16 arithmetic allows
# on top of it -- rounding O to bf16 (at most 2^-8 |O|) and rounding the probabilities to bf16 for
# the value product (at most 2^-8 sum_j p_j |v_j|, the oracle's error scale of each element):
#   |gpu - ref| <= 1e-2 + 2^-8 (|ref| + sum_j p_j |v_j|).
# Without the error scale, 2^-7 |ref| stands in for both terms (exact when the values a row's
# softmax mass sits on share one sign).
O_ELEM_REL = 2.0 ** -8


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def to_device(case: DecodeCase, dev):
    import torch
    q = torch.from_numpy(case.q.view(np.int16)).to(dev).view(torch.bfloat16)
    cache = torch.from_numpy(case.cache.view(np.int16)).to(dev).view(torch.bfloat16)
    bt = torch.from_numpy(case.block_table).to(dev)
    sl = torch.from_numpy(case.seqlens).to(dev)
    return q, cache, bt, sl


def run_gpu(case: DecodeCase, dev, tensors=None):
    """One plan + fwd through the C ABI; returns (O float64 [b,s_q,h,512], LSE float64 [b,s_q,h])."""
    import torch

    import mla_decode_attention_amd as mla
    q, cache, bt, sl = tensors if tensors is not None else to_device(case, dev)
    out, lse = mla.decode(q, cache, bt, sl, case.softmax_scale, case.causal)
    torch.cuda.synchronize()
    o = bf16_bits_to_f32(out.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return o, lse.cpu().numpy().astype(np.float64)


def parity(o, lse, ro, rl, what: str = "", scale=None):
    """Assert the bar; returns the raw and normalised error figures.  scale: the oracle's
    sum_j p_j |v_j| per element (with_scale=True), for the per-element bar."""
    o = np.asarray(o, dtype=np.float64)
    ro = np.asarray(ro, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    rl = np.asarray(rl, dtype=np.float64)
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: -inf LSE rows differ"
    assert np.all(o[empty] == 0.0), f"{what}: rows with no key must be exactly 0"
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse[~empty])), f"{what}: non-finite output"
    err = np.abs(o - ro)
    maxabs = float(err.max(initial=0.0))
    rmse = float(np.sqrt(np.mean(err ** 2))) if err.size else 0.0
    o_scale_max = max(1.0, float(np.abs(ro).max(initial=0.0)))
    o_scale_rms = max(1.0, float(np.sqrt(np.mean(ro ** 2))) if ro.size else 1.0)
    lse_rel = float(np.max(np.abs(lse[~empty] - rl[~empty]) / np.maximum(1.0, np.abs(rl[~empty])), initial=0.0))
    fig = dict(maxabs=maxabs, rmse=rmse, maxabs_norm=maxabs / o_scale_max, rmse_norm=rmse / o_scale_rms,
               lse_rel=lse_rel)
    # rounding-aware per-element bar
    if scale is not None:
        bound = O_MAXABS + O_ELEM_REL * (np.abs(ro) + np.asarray(scale, dtype=np.float64).reshape(ro.shape))
    else:
        bound = O_MAXABS + 2 * O_ELEM_REL * np.abs(ro)
    fig["elem_excess"] = float((err - bound).max(initial=-1.0))   # <= 0: inside the bar
    fig["max_abs_ref"] = o_scale_max
    log(f"parity {what}: O max-abs {maxabs:.3e} (norm {fig['maxabs_norm']:.3e}) rmse {rmse:.3e} "
        f"(norm {fig['rmse_norm']:.3e}); LSE rel {lse_rel:.3e}; per-element slack {-fig['elem_excess']:.3e}")
    record = os.environ.get("MLA_PARITY_RECORD")
    if record:   # raw and normalised figures of every parity check, one JSON line each
        with open(record, "a") as f:
            f.write(json.dumps(dict(case=what, **fig)) + "\n")
    assert fig["elem_excess"] <= 0.0, (what, fig)
    assert fig["maxabs_norm"] <= O_MAXABS, (what, fig)
    assert fig["rmse_norm"] <= O_RMSE, (what, fig)
    assert lse_rel <= LSE_REL, (what, fig)
    return fig
