"""The C ABI from plain C.

A gcc-built client (tests/c_client/decode_from_c.c) runs mla_decode_workspace_size, mla_decode_plan
and mla_decode_fwd through include/mla_decode.h alone, on hipMalloc'd buffers and the default
stream.  Its O and LSE must meet the decode bar against the fp64 oracle and be bit-identical to the
Python binding's result on the same inputs (same plan, same device).
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from gpu_helpers import log, parity, run_gpu
from mla_decode_attention_amd.inputs import bf16_bits_to_f32, make_case

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_client", "decode_from_c")


@pytest.mark.parametrize("heads,s_q,causal", [(16, 1, False), (16, 2, True), (128, 1, False)])
def test_c_client_matches_oracle_and_binding(dev, tmp_path, heads, s_q, causal):
    if not os.path.exists(BIN):
        pytest.fail("tests/c_client/decode_from_c is not built: run __graft_entry__.build()")
    lens = [1, 63, 64, 65, 700, 2049]
    case = make_case(f"c_client_h{heads}_sq{s_q}", batch=len(lens), s_q=s_q, heads=heads, seqlen=lens, seed=51,
                     causal=causal)
    case.q.astype(np.uint16).tofile(tmp_path / "q.bin")
    case.cache.astype(np.uint16).tofile(tmp_path / "cache.bin")
    case.block_table.astype(np.int32).tofile(tmp_path / "bt.bin")
    case.seqlens.astype(np.int32).tofile(tmp_path / "seqlens.bin")
    args = [BIN, str(tmp_path), str(case.batch), str(s_q), str(heads), str(case.cache.shape[0]),
            str(case.block_table.shape[1]), repr(float(case.softmax_scale)), str(int(causal))]
    log(f"c client: {' '.join(args[2:])}")
    res = subprocess.run(args, capture_output=True, text=True, timeout=120)
    log(f"c client exit {res.returncode}: {res.stdout.strip()} {res.stderr.strip()}")
    assert res.returncode == 0, res.stderr
    rows = case.batch * s_q * heads
    o_bits = np.fromfile(tmp_path / "out.bin", dtype=np.uint16).reshape(case.batch, s_q, heads, 512)
    lse = np.fromfile(tmp_path / "lse.bin", dtype=np.float32).reshape(case.batch, s_q, heads)
    assert lse.size == rows
    o = bf16_bits_to_f32(o_bits).astype(np.float64)
    ro, rl = oracle.mla_decode(case.q, case.cache, case.block_table, case.seqlens, case.softmax_scale, case.causal)
    parity(o, lse.astype(np.float64), ro, rl, f"{case.name} (C client)")
    # the binding on the same inputs: identical bits
    bo, bl = run_gpu(case, dev)
    assert np.array_equal(bo, o) and np.array_equal(bl, lse.astype(np.float64), equal_nan=True)
