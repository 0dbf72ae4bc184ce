"""fp64 CPU oracle for MLA decode attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path (the GPU library and its
binding do not import this package).

Functions, each with the passage it follows:
  * :func:`attention` -- standard softmax attention S = Q K^T, P = softmax(S),
    O = P V (FlashMLA-ETAP summary, "Mecanismo Central"), max-subtracted softmax
    (blog page, "数值稳定性增强", without its epsilon), fp64 (summary,
    "Estabilidade Numerica": the accuracy reference is double precision).
    Implemented in C (``mla_oracle.c``).
  * :func:`mla_decode` -- the same definition for every (sequence, query token,
    head) row of an absorbed-MQA decode step over a paged bf16 latent cache
    (GQLA summary, "Arquitetura": all heads attend the shared latent + RoPE key;
    the value is the first 512 dims of the row).  Implemented in C.
  * :func:`transposed_attention` -- the ETAP ordering S^T = K Q^T,
    P^T = softmax(S^T) along the key axis, O = (V^T P^T)^T (summary, "Mecanismo
    Central", item 1), written with numpy fp64 matmuls as the steps.
  * :func:`sparse_decode` -- top-k (sparse) decode: every head of a query token
    attends exactly the cache rows its index list names (GQLA summary, "GQLA
    Esparso": fine-grained sparse attention over the latent cache; the selection
    is an input), i.e. :func:`attention` over a gathered key set.
  * :mod:`oracle.rope_append` -- the cache append with rotary embedding of the
    RoPE parts (the step that feeds the decode path).
  * :func:`merge_by_lse` -- merge of results over disjoint key subsets by their
    log-sum-exp; it is the exact identity softmax over a union of key sets
    obeys, used to pin split invariance.

Readings where the pages are silent are listed in the design notes; the main
ones: LSE is natural log of sum_j exp(scale * q.k_j); a row with no visible key
gives O = 0 and LSE = -inf; s_q = 2 causal rows are bottom-right aligned.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build_oracle

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_LIBS: dict[int, ctypes.CDLL] = {}


def _load(planted_mistake: int = 0) -> ctypes.CDLL:
    lib = _LIBS.get(planted_mistake)
    if lib is not None:
        return lib
    path = build_oracle.lib_path(planted_mistake)
    if planted_mistake != 0 or not os.path.exists(path):
        build_oracle.build(planted_mistake)
    lib = ctypes.CDLL(path)
    lib.oracle_attention_f64.argtypes = [_I64, _I64, _I64, _I64, _P, _P, _P, ctypes.c_double, _P, _P, _P]
    lib.oracle_attention_f64.restype = ctypes.c_int
    lib.oracle_mla_decode.argtypes = [_P, _P, _P, _I64, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                      ctypes.c_double, ctypes.c_int, _P, _I64, _P, _P, ctypes.c_int]
    lib.oracle_mla_decode.restype = ctypes.c_int
    lib.oracle_mla_decode_with_scale.argtypes = [_P, _P, _P, _I64, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                                 ctypes.c_double, ctypes.c_int, _P, _I64, _P, _P, _P, ctypes.c_int]
    lib.oracle_mla_decode_with_scale.restype = ctypes.c_int
    _LIBS[planted_mistake] = lib
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(_P)


class Oracle:
    """Handle on one build of the C oracle (``planted_mistake`` > 0 only in pin tests)."""

    def __init__(self, planted_mistake: int = 0):
        self.planted_mistake = planted_mistake
        self.lib = _load(planted_mistake)

    def attention(self, q, k, v, scale: float, return_probs: bool = False):
        q = np.ascontiguousarray(q, dtype=np.float64)
        k = np.ascontiguousarray(k, dtype=np.float64).reshape(-1, q.shape[1])
        v = np.ascontiguousarray(v, dtype=np.float64)
        v = v.reshape(k.shape[0], -1) if v.size else v.reshape(0, max(1, v.shape[-1]))
        n_q, d_k = q.shape
        n_k, d_v = k.shape[0], v.shape[1]
        o = np.empty((n_q, d_v))
        lse = np.empty(n_q)
        p = np.empty((n_q, n_k)) if return_probs else None
        rc = self.lib.oracle_attention_f64(n_q, n_k, d_k, d_v, _ptr(q), _ptr(k), _ptr(v), float(scale),
                                           _ptr(o), _ptr(lse), _ptr(p))
        if rc != 0:
            raise RuntimeError(f"oracle_attention_f64 failed: {rc}")
        return (o, lse, p) if return_probs else (o, lse)

    def mla_decode(self, q_bits, cache_bits, block_table, seqlens, scale: float, causal: bool,
                   d_v: int = 512, rows=None, threads: int | None = None, with_scale: bool = False):
        """fp64 O and LSE for the given rows (default: all, shaped [b, s_q, h, d_v] and [b, s_q, h]).
        with_scale: also sum_j p_j |v_j| per element (shaped like O), the error scale of rounding the
        weights before the weighted sum."""
        q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
        cache_bits = np.ascontiguousarray(cache_bits, dtype=np.uint16)
        block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        seqlens = np.ascontiguousarray(seqlens, dtype=np.int32)
        b, s_q, h, d_k = q_bits.shape
        num_pages, page_size, d_k2 = cache_bits.shape
        assert d_k2 == d_k and block_table.shape[0] == b and seqlens.shape == (b,)
        sel = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = b * s_q * h if sel is None else sel.shape[0]
        o = np.empty((n_rows, d_v))
        lse = np.empty(n_rows)
        threads = threads or (os.cpu_count() or 1)
        if with_scale:
            o_abs = np.empty((n_rows, d_v))
            rc = self.lib.oracle_mla_decode_with_scale(
                _ptr(q_bits), _ptr(cache_bits), _ptr(block_table), block_table.shape[1], _ptr(seqlens), b, s_q, h,
                num_pages, page_size, d_k, d_v, float(scale), int(bool(causal)), _ptr(sel), n_rows, _ptr(o),
                _ptr(o_abs), _ptr(lse), int(threads))
        else:
            o_abs = None
            rc = self.lib.oracle_mla_decode(_ptr(q_bits), _ptr(cache_bits), _ptr(block_table), block_table.shape[1],
                                            _ptr(seqlens), b, s_q, h, num_pages, page_size, d_k, d_v, float(scale),
                                            int(bool(causal)), _ptr(sel), n_rows, _ptr(o), _ptr(lse), int(threads))
        if rc != 0:
            raise RuntimeError(f"oracle_mla_decode failed: {rc}")
        if sel is None:
            o, lse = o.reshape(b, s_q, h, d_v), lse.reshape(b, s_q, h)
            o_abs = None if o_abs is None else o_abs.reshape(b, s_q, h, d_v)
        return (o, lse, o_abs) if with_scale else (o, lse)


_DEFAULT: Oracle | None = None


def default() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle(0)
    return _DEFAULT


def attention(q, k, v, scale: float, return_probs: bool = False):
    return default().attention(q, k, v, scale, return_probs)


def mla_decode(q_bits, cache_bits, block_table, seqlens, scale, causal, d_v=512, rows=None, threads=None,
               with_scale=False):
    return default().mla_decode(q_bits, cache_bits, block_table, seqlens, scale, causal, d_v, rows, threads,
                                with_scale)


def _bf16_f64(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def sparse_decode(q_bits, cache_bits, block_table, seqlens, indices, scale: float, d_v: int = 512,
                  oracle: Oracle | None = None):
    """fp64 O [b, s_q, h, d_v] and LSE [b, s_q, h] of the sparse decode step.

    indices int [b, s_q, topk]: logical token positions of sequence b (cache row of position j:
    page block_table[b][j // 64], slot j % 64); -1 marks an unused slot; a position listed twice is
    two keys.  Every head of query token (b, i) attends the rows listed for (b, i).  A token with an
    index outside [0, L_b) or whose row lies on a page outside the pool gets NaN; one with no index
    gets O = 0, LSE = -inf.
    """
    orc = oracle or default()
    q_bits = np.asarray(q_bits, dtype=np.uint16)
    cache_bits = np.asarray(cache_bits, dtype=np.uint16)
    bt = np.asarray(block_table, dtype=np.int64)
    sl = np.asarray(seqlens, dtype=np.int64)
    ind = np.asarray(indices, dtype=np.int64)
    b, s_q, h, _ = q_bits.shape
    num_pages, page = cache_bits.shape[:2]
    o = np.zeros((b, s_q, h, d_v))
    lse = np.full((b, s_q, h), -np.inf)
    for bi in range(b):
        for i in range(s_q):
            idx = ind[bi, i]
            idx = idx[idx >= 0]
            if idx.size and (idx.max() >= sl[bi] or sl[bi] > page * bt.shape[1]):
                o[bi, i], lse[bi, i] = np.nan, np.nan
                continue
            pages = bt[bi, idx // page]
            if ((pages < 0) | (pages >= num_pages)).any():
                o[bi, i], lse[bi, i] = np.nan, np.nan
                continue
            k = _bf16_f64(cache_bits[pages, idx % page])
            oi, li = orc.attention(_bf16_f64(q_bits[bi, i]), k, k[:, :d_v], scale)
            o[bi, i], lse[bi, i] = oi, li
    return o, lse


def transposed_attention(q, k, v, scale: float):
    """ETAP ordering: S^T = K Q^T, softmax down each column (the key axis), O = (V^T P^T)^T."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    st = scale * (k @ q.T)                       # [n_k, n_q]
    colmax = st.max(axis=0, keepdims=True)
    e = np.exp(st - colmax)
    l = e.sum(axis=0, keepdims=True)
    pt = e / l                                   # P^T, columns sum to 1
    o = (v.T @ pt).T                             # [n_q, d_v]
    lse = colmax[0] + np.log(l[0])
    return o, lse


def merge_by_lse(o_parts, lse_parts):
    """Merge normalised partial outputs over disjoint key sets.

    o_parts [n_parts, n_q, d_v], lse_parts [n_parts, n_q] -> (O, LSE) with
    LSE = log sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s.  Parts with
    LSE_s = -inf (no keys) get weight 0; if every part is empty, O = 0 and
    LSE = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    mx = lse_parts.max(axis=0)
    empty = ~np.isfinite(mx)
    safe = np.where(empty, 0.0, mx)
    w = np.exp(lse_parts - safe[None, :])        # exp(-inf) = 0 for empty parts
    tot = w.sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.einsum("sq,sqd->qd", w, o_parts) / tot[:, None]
        lse = safe + np.log(tot)
    o[empty] = 0.0
    lse[empty] = -np.inf
    return o, lse
