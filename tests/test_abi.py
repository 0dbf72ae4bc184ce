"""The C ABI without a GPU: the library loads, exports what include/mla_decode.h declares, and every
argument error is reported by status code before any HIP call (CPU only)."""
import ctypes
import math
import os
import re

import pytest

import mla_decode_attention_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mla.LIB_PATH):
        from mla_decode_attention_amd import build
        build.build()
    return mla.lib()


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(mla.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings(L):
    for code, name in mla.STATUS.items():
        assert mla.status_string(code).startswith(name)
    assert "unknown" in mla.status_string(-99)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    assert re.search(r"#define MLA_DECODE_D_K 576\b", text)
    assert re.search(r"#define MLA_DECODE_D_V 512\b", text)
    assert re.search(r"#define MLA_DECODE_PAGE_SIZE 64\b", text)
    assert re.search(r"#define MLA_DECODE_MAX_BATCH \(1 << 20\)", text)
    for code, name in mla.STATUS.items():
        assert re.search(rf"{name}\s*=\s*{code}\b", text), name


P = ctypes.c_void_p
FAKE = 0x10000   # aligned, never dereferenced: every call below fails validation first


def _fwd(L, **kw):
    args = dict(q=FAKE, kv=FAKE, bt=FAKE, bt_stride=4, sl=FAKE, batch=1, s_q=1, heads=16, num_pages=4,
                page_size=64, scale=1 / math.sqrt(192), causal=0, ws=FAKE, ws_bytes=1 << 20, out=FAKE, lse=FAKE)
    args.update(kw)
    return L.mla_decode_fwd(P(args["q"]), P(args["kv"]), P(args["bt"]), args["bt_stride"], P(args["sl"]),
                            args["batch"], args["s_q"], args["heads"], args["num_pages"], args["page_size"],
                            ctypes.c_float(args["scale"]), args["causal"], P(args["ws"]), args["ws_bytes"],
                            P(args["out"]), P(args["lse"]), None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), -1), (dict(kv=0), -1), (dict(bt=0), -1), (dict(sl=0), -1), (dict(ws=0), -1),
    (dict(out=0), -1), (dict(lse=0), -1), (dict(batch=0), -1), (dict(batch=-3), -1), (dict(batch=(1 << 20) + 1), -1),
    (dict(bt_stride=0), -1),
    (dict(num_pages=0), -1), (dict(scale=float("nan")), -1), (dict(scale=float("inf")), -1), (dict(scale=3e38), -1),
    (dict(causal=2), -1), (dict(q=FAKE + 8), -1), (dict(kv=FAKE + 2), -1), (dict(ws=FAKE + 16), -1),
    (dict(heads=8), -2), (dict(heads=24), -2), (dict(heads=256), -2), (dict(s_q=3), -2), (dict(s_q=0), -2),
    (dict(page_size=32), -2),
])
def test_fwd_argument_errors(L, kw, code):
    assert _fwd(L, **kw) == code


def test_plan_argument_errors(L):
    ws = P(FAKE)
    assert L.mla_decode_plan(None, 1, 1, 16, ws, 1 << 20, None) == -1
    assert L.mla_decode_plan(P(FAKE), 0, 1, 16, ws, 1 << 20, None) == -1
    assert L.mla_decode_plan(P(FAKE), (1 << 20) + 1, 1, 16, ws, 1 << 20, None) == -1
    assert L.mla_decode_plan(P(FAKE), 1, 1, 16, None, 1 << 20, None) == -1
    assert L.mla_decode_plan(P(FAKE), 1, 1, 16, P(FAKE + 4), 1 << 20, None) == -1
    assert L.mla_decode_plan(P(FAKE), 1, 3, 16, ws, 1 << 20, None) == -2
    assert L.mla_decode_plan(P(FAKE), 1, 1, 20, ws, 1 << 20, None) == -2


def test_plan_chunked_argument_errors(L):
    ws = P(FAKE)
    assert L.mla_decode_plan_chunked(P(FAKE), 1, 1, 16, -1, ws, 1 << 20, None) == -1   # negative chunk
    assert L.mla_decode_plan_chunked(None, 1, 1, 16, 4, ws, 1 << 20, None) == -1
    assert L.mla_decode_plan_chunked(P(FAKE), 0, 1, 16, 4, ws, 1 << 20, None) == -1
    assert L.mla_decode_plan_chunked(P(FAKE), 1, 1, 16, 4, P(FAKE + 4), 1 << 20, None) == -1
    assert L.mla_decode_plan_chunked(P(FAKE), 1, 3, 16, 4, ws, 1 << 20, None) == -2
    assert L.mla_decode_plan_chunked(P(FAKE), 1, 1, 20, 4, ws, 1 << 20, None) == -2


def test_workspace_size_argument_errors(L):
    n = ctypes.c_size_t(0)
    assert L.mla_decode_workspace_size(1, 1, 16, None) == -1
    assert L.mla_decode_workspace_size(0, 1, 16, ctypes.byref(n)) == -1
    assert L.mla_decode_workspace_size((1 << 20) + 1, 1, 16, ctypes.byref(n)) == -1
    # heads must be a multiple of 16 in 16..128: 48 is supported, 40 and 144 are not
    assert L.mla_decode_workspace_size(1, 2, 40, ctypes.byref(n)) == -2
    assert L.mla_decode_workspace_size(1, 1, 144, ctypes.byref(n)) == -2


def _append(L, **kw):
    args = dict(lat=FAKE, rope=FAKE, q=FAKE, kv=FAKE, bt=FAKE, bt_stride=4, sl=FAKE, batch=1, s_q=1, heads=16,
                num_pages=4, page_size=64, base=10000.0)
    args.update(kw)
    return L.mla_cache_append_rope(P(args["lat"]), P(args["rope"]), P(args["q"]), P(args["kv"]), P(args["bt"]),
                                   args["bt_stride"], P(args["sl"]), args["batch"], args["s_q"], args["heads"],
                                   args["num_pages"], args["page_size"], ctypes.c_float(args["base"]), None)


@pytest.mark.parametrize("kw,code", [
    (dict(lat=0), -1), (dict(rope=0), -1), (dict(q=0), -1), (dict(kv=0), -1), (dict(bt=0), -1), (dict(sl=0), -1),
    (dict(batch=0), -1), (dict(batch=(1 << 20) + 1), -1), (dict(bt_stride=0), -1), (dict(num_pages=0), -1),
    (dict(base=1.0), -1),
    (dict(base=float("nan")), -1), (dict(base=float("inf")), -1), (dict(lat=FAKE + 8), -1), (dict(q=FAKE + 2), -1),
    (dict(heads=8), -2), (dict(s_q=3), -2), (dict(page_size=128), -2),
])
def test_append_argument_errors(L, kw, code):
    assert _append(L, **kw) == code


def _sparse_fwd(L, **kw):
    args = dict(q=FAKE, kv=FAKE, bt=FAKE, bt_stride=4, sl=FAKE, ind=FAKE, batch=1, s_q=1, heads=16, topk=64,
                num_pages=4, page_size=64, scale=0.07, ws=FAKE, ws_bytes=1 << 20, out=FAKE, lse=FAKE)
    args.update(kw)
    return L.mla_sparse_decode_fwd(P(args["q"]), P(args["kv"]), P(args["bt"]), args["bt_stride"], P(args["sl"]),
                                   P(args["ind"]), args["batch"], args["s_q"], args["heads"], args["topk"],
                                   args["num_pages"], args["page_size"], ctypes.c_float(args["scale"]), P(args["ws"]),
                                   args["ws_bytes"], P(args["out"]), P(args["lse"]), None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), -1), (dict(ind=0), -1), (dict(ws=0), -1), (dict(out=0), -1), (dict(batch=0), -1), (dict(topk=0), -1),
    (dict(num_pages=(1 << 25) + 1), -1),
    (dict(bt_stride=0), -1), (dict(num_pages=0), -1), (dict(scale=float("nan")), -1), (dict(ind=FAKE + 2), -1),
    (dict(ws=FAKE + 64), -1), (dict(heads=32), -2), (dict(heads=128), -2), (dict(s_q=3), -2), (dict(page_size=16), -2),
])
def test_sparse_fwd_argument_errors(L, kw, code):
    assert _sparse_fwd(L, **kw) == code


def test_sparse_plan_and_size_argument_errors(L):
    n = ctypes.c_size_t(0)
    assert L.mla_sparse_decode_workspace_size(1, 1, 16, 64, None) == -1
    assert L.mla_sparse_decode_workspace_size(0, 1, 16, 64, ctypes.byref(n)) == -1
    assert L.mla_sparse_decode_workspace_size(1, 1, 16, 0, ctypes.byref(n)) == -1
    assert L.mla_sparse_decode_workspace_size(1, 1, 64, 64, ctypes.byref(n)) == -2
    assert L.mla_sparse_decode_plan(1, 1, 16, 64, None, 1 << 20, None) == -1
    assert L.mla_sparse_decode_plan(1, 1, 16, 64, P(FAKE + 8), 1 << 20, None) == -1
    assert L.mla_sparse_decode_plan(1, 3, 16, 64, P(FAKE), 1 << 20, None) == -2


def test_absorb_argument_errors(L):
    f = P(FAKE)
    assert L.mla_absorb_q(None, f, f, 1, 1, 16, f, None) == -1
    assert L.mla_absorb_q(f, f, f, 0, 1, 16, f, None) == -1
    assert L.mla_absorb_q(P(FAKE + 8), f, f, 1, 1, 16, f, None) == -1
    assert L.mla_absorb_q(f, f, f, 1, 1, 24, f, None) == -2
    assert L.mla_absorb_q(f, f, f, 1, 3, 16, f, None) == -2
    assert L.mla_unabsorb_o(f, None, 1, 1, 16, f, None) == -1
    assert L.mla_unabsorb_o(f, f, 0, 1, 16, f, None) == -1
    assert L.mla_unabsorb_o(f, f, 1, 2, 256, f, None) == -2


def test_gqa_argument_errors(L):
    f = P(FAKE)
    n = ctypes.c_size_t(0)
    args = lambda **kw: {**dict(q=FAKE, kv=FAKE, bt=FAKE, bs=4, sl=FAKE, b=1, s_q=2, h=16, np_=4, ps=64, sc=0.07, c=1,
                                ws=FAKE, wsb=1 << 20, out=FAKE, lse=FAKE), **kw}
    call = lambda a: L.mla_gqa_decode_fwd(P(a["q"]), P(a["kv"]), P(a["bt"]), a["bs"], P(a["sl"]), a["b"], a["s_q"],
                                           a["h"], a["np_"], a["ps"], ctypes.c_float(a["sc"]), a["c"], P(a["ws"]),
                                           a["wsb"], P(a["out"]), P(a["lse"]), None)
    for kw, code in [(dict(q=0), -1), (dict(kv=0), -1), (dict(b=0), -1), (dict(b=(1 << 20) + 1), -1), (dict(c=3), -1),
                     (dict(sc=float("inf")), -1),
                     (dict(q=FAKE + 2), -1), (dict(h=32), -2), (dict(s_q=3), -2), (dict(ps=32), -2)]:
        assert call(args(**kw)) == code, kw
    assert L.mla_gqa_decode_workspace_size(1, 1, 16, None) == -1
    assert L.mla_gqa_decode_workspace_size(1, 1, 128, ctypes.byref(n)) == -2
    assert L.mla_gqa_decode_plan(None, 1, 1, 16, f, 1 << 20, None) == -1
    assert L.mla_gqa_decode_plan(f, 1, 2, 64, f, 1 << 20, None) == -2
    if not __import__("torch").cuda.is_available():
        assert call(args()) == -4


def test_valid_arguments_without_a_gpu_report_no_device(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    n = ctypes.c_size_t(0)
    assert L.mla_decode_workspace_size(16, 1, 16, ctypes.byref(n)) == -4
    assert L.mla_decode_plan(P(FAKE), 1, 1, 16, P(FAKE), 1 << 20, None) == -4
    assert _fwd(L) == -4
    assert _append(L) == -4
    assert _sparse_fwd(L) == -4
    assert L.mla_absorb_q(P(FAKE), P(FAKE), P(FAKE), 1, 1, 16, P(FAKE), None) == -4
    assert L.mla_unabsorb_o(P(FAKE), P(FAKE), 1, 1, 16, P(FAKE), None) == -4
    assert L.mla_sparse_decode_plan(1, 1, 16, 64, P(FAKE), 1 << 20, None) == -4
    with pytest.raises(mla.MlaDecodeError):
        mla.workspace_size(16, 1, 16)
