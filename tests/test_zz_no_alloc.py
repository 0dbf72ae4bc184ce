"""The allocation-free entry point (mla_decode_fwd_noalloc, built-in device workspace) against plan +
fwd with a caller workspace: bit-identical outputs, on two calls in a row (the second smaller), and
the size limit reported as an error with nothing launched."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

from mla_decode_attention_amd.inputs import make_case

from gpu_helpers import log, to_device

pytestmark = pytest.mark.gpu


def _noalloc(mla, case, tensors, out, lse):
    import torch
    q, cache, bt, sl = tensors
    status = mla.lib().mla_decode_fwd_noalloc(
        q.data_ptr(), cache.data_ptr(), bt.data_ptr(), bt.shape[1], sl.data_ptr(), case.batch, case.s_q, case.heads,
        cache.shape[0], cache.shape[1], ctypes.c_float(case.softmax_scale), int(case.causal), out.data_ptr(),
        lse.data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return status


def test_noalloc_matches_plan_and_fwd(dev):
    import torch

    import mla_decode_attention_amd as mla
    big = make_case("noalloc_big", batch=6, s_q=2, heads=128, seqlen=[5000, 1, 0, 777, 4096, 130], seed=61,
                    causal=True, pool_pages=sum((L + 63) // 64 for L in [5000, 1, 0, 777, 4096, 130]) + 9)
    small = make_case("noalloc_small", batch=3, s_q=1, heads=16, seqlen=[300, 65, 2000], seed=62)
    for case in (big, small):   # two calls in a row on one GPU, the second with a smaller input
        log(f"case {case.name}: b={case.batch} s_q={case.s_q} h={case.heads} L={case.seqlens.tolist()}")
        t = to_device(case, dev)
        out = torch.full((case.batch, case.s_q, case.heads, 512), float("nan"), dtype=torch.bfloat16, device=dev)
        lse = torch.full((case.batch, case.s_q, case.heads), float("nan"), dtype=torch.float32, device=dev)
        assert _noalloc(mla, case, t, out, lse) == 0
        ref_out, ref_lse = mla.decode(*t, case.softmax_scale, case.causal)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), case.name
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), case.name


def test_noalloc_rejects_shapes_beyond_its_scratch(dev):
    import torch

    import mla_decode_attention_amd as mla
    # 700 sequences of 128 heads need far more workspace than the built-in 128 MiB
    need = mla.workspace_size(700, 1, 128)
    assert need > (128 << 20)
    case = make_case("noalloc_huge", batch=700, s_q=1, heads=128, seqlen=1, seed=63, poison=False)
    t = to_device(case, dev)
    out = torch.zeros((case.batch, 1, 128, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((case.batch, 1, 128), dtype=torch.float32, device=dev)
    assert _noalloc(mla, case, t, out, lse) == -3
    torch.cuda.synchronize()
    assert not out.view(torch.int16).any() and not lse.view(torch.int32).any()   # nothing was launched
