"""MLA decode attention (absorbed-MQA form) for AMD Instinct MI355X (gfx950).

Thin ctypes binding over the C ABI of ``libmla_decode.so`` (declared in
``include/mla_decode.h``).  The functions here only marshal arguments: they
check dtypes, shapes and devices of torch tensors, pass raw device pointers and
the current HIP stream, and turn negative status codes into exceptions.  Every
step of the computation runs in the library's HIP kernels; there is no CPU or
PyTorch fallback -- if the library is missing, :func:`lib` raises.

Names follow the C ABI:
  * :func:`workspace_size` -> ``mla_decode_workspace_size``
  * :func:`plan`           -> ``mla_decode_plan`` (``chunk_pages`` > 0: ``mla_decode_plan_chunked``)
  * :func:`fwd`            -> ``mla_decode_fwd``
  * :func:`fwd_split`      -> ``mla_decode_fwd_split``   (first half of fwd)
  * :func:`fwd_combine`    -> ``mla_decode_fwd_combine`` (second half of fwd)
  * :func:`fwd_noalloc`    -> ``mla_decode_fwd_noalloc`` (plan + fwd in the library's built-in
    workspace, no allocation)
  * :func:`status_string`  -> ``mla_decode_status_string``
  * :func:`cache_append_rope` -> ``mla_cache_append_rope`` (new tokens into the paged cache)
  * :func:`gqa_workspace_size`, :func:`gqa_plan`, :func:`gqa_fwd` -> ``mla_gqa_decode_*`` (the
    GQA path of GQLA: one group's 16 heads over its expanded key/value cache)
  * :func:`absorb_q`, :func:`unabsorb_o` -> ``mla_absorb_q`` / ``mla_unabsorb_o`` (per-head
    projections into and out of the latent space, either side of the decode path)
  * :func:`sparse_workspace_size`, :func:`sparse_plan`, :func:`sparse_fwd` ->
    ``mla_sparse_decode_workspace_size`` / ``_plan`` / ``_fwd`` (top-k decode)
plus :func:`decode`, which allocates the workspace/outputs and calls plan + fwd.
"""
from __future__ import annotations

import ctypes
import os

D_K = 576
D_V = 512
PAGE_SIZE = 64

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_decode.so")
_LIB: ctypes.CDLL | None = None

STATUS = {0: "MLA_OK", -1: "MLA_ERR_INVALID_ARG", -2: "MLA_ERR_UNSUPPORTED",
          -3: "MLA_ERR_WORKSPACE_TOO_SMALL", -4: "MLA_ERR_NO_DEVICE", -5: "MLA_ERR_HIP"}
EXPORTS = ("mla_decode_workspace_size", "mla_decode_plan", "mla_decode_fwd", "mla_decode_fwd_split",
           "mla_decode_fwd_combine", "mla_decode_status_string", "mla_cache_append_rope",
           "mla_sparse_decode_workspace_size", "mla_sparse_decode_plan", "mla_sparse_decode_fwd",
           "mla_absorb_q", "mla_unabsorb_o", "mla_gqa_decode_workspace_size", "mla_gqa_decode_plan",
           "mla_gqa_decode_fwd", "mla_decode_fwd_noalloc", "mla_decode_plan_chunked")
GQA_D_H = 128
GQA_ROW = 320
D_NOPE = 128


class MlaDecodeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


def lib() -> ctypes.CDLL:
    """Load the HIP library (built in-tree); raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m mla_decode_attention_amd.build` "
                          "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.mla_decode_workspace_size.argtypes = [I, I, I, ctypes.POINTER(SZ)]
    L.mla_decode_workspace_size.restype = I
    L.mla_decode_plan.argtypes = [P, I, I, I, P, SZ, P]
    L.mla_decode_plan.restype = I
    L.mla_decode_plan_chunked.argtypes = [P, I, I, I, I, P, SZ, P]
    L.mla_decode_plan_chunked.restype = I
    L.mla_decode_fwd.argtypes = [P, P, P, I, P, I, I, I, I, I, ctypes.c_float, I, P, SZ, P, P, P]
    L.mla_decode_fwd.restype = I
    L.mla_decode_fwd_split.argtypes = [P, P, P, I, P, I, I, I, I, I, ctypes.c_float, I, P, SZ, P]
    L.mla_decode_fwd_split.restype = I
    L.mla_decode_fwd_combine.argtypes = [P, I, I, I, I, P, SZ, P, P, P]
    L.mla_decode_fwd_combine.restype = I
    L.mla_decode_fwd_noalloc.argtypes = [P, P, P, I, P, I, I, I, I, I, ctypes.c_float, I, P, P, P]
    L.mla_decode_fwd_noalloc.restype = I
    L.mla_cache_append_rope.argtypes = [P, P, P, P, P, I, P, I, I, I, I, I, ctypes.c_float, P]
    L.mla_cache_append_rope.restype = I
    L.mla_sparse_decode_workspace_size.argtypes = [I, I, I, I, ctypes.POINTER(SZ)]
    L.mla_sparse_decode_workspace_size.restype = I
    L.mla_sparse_decode_plan.argtypes = [I, I, I, I, P, SZ, P]
    L.mla_sparse_decode_plan.restype = I
    L.mla_sparse_decode_fwd.argtypes = [P, P, P, I, P, P, I, I, I, I, I, I, ctypes.c_float, P, SZ, P, P, P]
    L.mla_sparse_decode_fwd.restype = I
    L.mla_absorb_q.argtypes = [P, P, P, I, I, I, P, P]
    L.mla_absorb_q.restype = I
    L.mla_unabsorb_o.argtypes = [P, P, I, I, I, P, P]
    L.mla_unabsorb_o.restype = I
    L.mla_gqa_decode_workspace_size.argtypes = [I, I, I, ctypes.POINTER(SZ)]
    L.mla_gqa_decode_workspace_size.restype = I
    L.mla_gqa_decode_plan.argtypes = [P, I, I, I, P, SZ, P]
    L.mla_gqa_decode_plan.restype = I
    L.mla_gqa_decode_fwd.argtypes = [P, P, P, I, P, I, I, I, I, I, ctypes.c_float, I, P, SZ, P, P, P]
    L.mla_gqa_decode_fwd.restype = I
    L.mla_decode_status_string.argtypes = [I]
    L.mla_decode_status_string.restype = ctypes.c_char_p
    _LIB = L
    return L


def status_string(status: int) -> str:
    return lib().mla_decode_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MlaDecodeError(fn, status)


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def workspace_size(batch: int, s_q: int, num_heads: int) -> int:
    out = ctypes.c_size_t(0)
    _check("mla_decode_workspace_size", lib().mla_decode_workspace_size(int(batch), int(s_q), int(num_heads),
                                                                         ctypes.byref(out)))
    return int(out.value)


def _require(t, name, dtype, ndim=None, device=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def plan(seqlens, s_q: int, num_heads: int, workspace, stream=None, chunk_pages: int = 0) -> None:
    """mla_decode_plan: split metadata for these seqlens into ``workspace`` (uint8 device tensor);
    ``chunk_pages`` > 0 caps the pages per work item (mla_decode_plan_chunked)."""
    import torch
    _require(seqlens, "seqlens", torch.int32, 1)
    _require(workspace, "workspace", torch.uint8, 1, seqlens.device)
    if chunk_pages:
        _check("mla_decode_plan_chunked", lib().mla_decode_plan_chunked(
            seqlens.data_ptr(), seqlens.shape[0], int(s_q), int(num_heads), int(chunk_pages), workspace.data_ptr(),
            workspace.numel(), _stream(stream)))
        return
    _check("mla_decode_plan", lib().mla_decode_plan(seqlens.data_ptr(), seqlens.shape[0], int(s_q), int(num_heads),
                                                    workspace.data_ptr(), workspace.numel(), _stream(stream)))


def fwd(q, kv_cache, block_table, seqlens, softmax_scale: float, causal: bool, workspace, out, lse,
        stream=None) -> None:
    """mla_decode_fwd: O bf16 [b, s_q, h, 512] into ``out`` and LSE fp32 [b, s_q, h] into ``lse``."""
    import torch
    _require(q, "q", torch.bfloat16, 4)
    dev = q.device
    _require(kv_cache, "kv_cache", torch.bfloat16, 3, dev)
    _require(block_table, "block_table", torch.int32, 2, dev)
    _require(seqlens, "seqlens", torch.int32, 1, dev)
    _require(workspace, "workspace", torch.uint8, 1, dev)
    _require(out, "out", torch.bfloat16, 4, dev)
    _require(lse, "lse", torch.float32, 3, dev)
    b, s_q, h, dk = q.shape
    if dk != D_K or kv_cache.shape[2] != D_K:
        raise ValueError("q and kv_cache rows must be 576 wide")
    if tuple(out.shape) != (b, s_q, h, D_V) or tuple(lse.shape) != (b, s_q, h):
        raise ValueError("out must be [b, s_q, h, 512] and lse [b, s_q, h]")
    if block_table.shape[0] != b or seqlens.shape[0] != b:
        raise ValueError("block_table and seqlens need one row per sequence")
    _check("mla_decode_fwd", lib().mla_decode_fwd(
        q.data_ptr(), kv_cache.data_ptr(), block_table.data_ptr(), block_table.shape[1], seqlens.data_ptr(),
        b, s_q, h, kv_cache.shape[0], kv_cache.shape[1], float(softmax_scale), int(bool(causal)),
        workspace.data_ptr(), workspace.numel(), out.data_ptr(), lse.data_ptr(), _stream(stream)))


def fwd_split(q, kv_cache, block_table, seqlens, softmax_scale: float, causal: bool, workspace,
              stream=None) -> None:
    """mla_decode_fwd_split: per-item partial outputs and LSEs into ``workspace``."""
    import torch
    _require(q, "q", torch.bfloat16, 4)
    dev = q.device
    _require(kv_cache, "kv_cache", torch.bfloat16, 3, dev)
    _require(block_table, "block_table", torch.int32, 2, dev)
    _require(seqlens, "seqlens", torch.int32, 1, dev)
    _require(workspace, "workspace", torch.uint8, 1, dev)
    b, s_q, h, _ = q.shape
    _check("mla_decode_fwd_split", lib().mla_decode_fwd_split(
        q.data_ptr(), kv_cache.data_ptr(), block_table.data_ptr(), block_table.shape[1], seqlens.data_ptr(),
        b, s_q, h, kv_cache.shape[0], kv_cache.shape[1], float(softmax_scale), int(bool(causal)),
        workspace.data_ptr(), workspace.numel(), _stream(stream)))


def fwd_combine(seqlens, bt_stride: int, s_q: int, num_heads: int, workspace, out, lse, stream=None) -> None:
    """mla_decode_fwd_combine: merge the partials in ``workspace`` into ``out`` and ``lse``."""
    import torch
    _require(seqlens, "seqlens", torch.int32, 1)
    dev = seqlens.device
    _require(workspace, "workspace", torch.uint8, 1, dev)
    _require(out, "out", torch.bfloat16, 4, dev)
    _require(lse, "lse", torch.float32, 3, dev)
    b = seqlens.shape[0]
    if tuple(out.shape) != (b, s_q, num_heads, D_V) or tuple(lse.shape) != (b, s_q, num_heads):
        raise ValueError("out must be [b, s_q, h, 512] and lse [b, s_q, h]")
    _check("mla_decode_fwd_combine", lib().mla_decode_fwd_combine(
        seqlens.data_ptr(), int(bt_stride), b, int(s_q), int(num_heads), workspace.data_ptr(), workspace.numel(),
        out.data_ptr(), lse.data_ptr(), _stream(stream)))


def fwd_noalloc(q, kv_cache, block_table, seqlens, softmax_scale: float, causal: bool, out, lse,
                stream=None) -> None:
    """mla_decode_fwd_noalloc: plan + fwd into ``out`` / ``lse`` using the library's built-in workspace."""
    import torch
    _require(q, "q", torch.bfloat16, 4)
    dev = q.device
    _require(kv_cache, "kv_cache", torch.bfloat16, 3, dev)
    _require(block_table, "block_table", torch.int32, 2, dev)
    _require(seqlens, "seqlens", torch.int32, 1, dev)
    _require(out, "out", torch.bfloat16, 4, dev)
    _require(lse, "lse", torch.float32, 3, dev)
    b, s_q, h, dk = q.shape
    if dk != D_K or kv_cache.shape[2] != D_K:
        raise ValueError("q and kv_cache rows must be 576 wide")
    if tuple(out.shape) != (b, s_q, h, D_V) or tuple(lse.shape) != (b, s_q, h):
        raise ValueError("out must be [b, s_q, h, 512] and lse [b, s_q, h]")
    if block_table.shape[0] != b or seqlens.shape[0] != b:
        raise ValueError("block_table and seqlens need one row per sequence")
    _check("mla_decode_fwd_noalloc", lib().mla_decode_fwd_noalloc(
        q.data_ptr(), kv_cache.data_ptr(), block_table.data_ptr(), block_table.shape[1], seqlens.data_ptr(),
        b, s_q, h, kv_cache.shape[0], kv_cache.shape[1], float(softmax_scale), int(bool(causal)),
        out.data_ptr(), lse.data_ptr(), _stream(stream)))


def cache_append_rope(kv_latent, k_rope, q, kv_cache, block_table, seqlens, rope_base: float = 10000.0,
                      stream=None) -> None:
    """mla_cache_append_rope: write the s_q new tokens' cache rows (latent + rotated RoPE key) and
    rotate the RoPE part of ``q`` in place."""
    import torch
    _require(q, "q", torch.bfloat16, 4)
    dev = q.device
    _require(kv_latent, "kv_latent", torch.bfloat16, 3, dev)
    _require(k_rope, "k_rope", torch.bfloat16, 3, dev)
    _require(kv_cache, "kv_cache", torch.bfloat16, 3, dev)
    _require(block_table, "block_table", torch.int32, 2, dev)
    _require(seqlens, "seqlens", torch.int32, 1, dev)
    b, s_q, h, dk = q.shape
    if dk != D_K or kv_cache.shape[2] != D_K:
        raise ValueError("q and kv_cache rows must be 576 wide")
    if tuple(kv_latent.shape) != (b, s_q, D_V) or tuple(k_rope.shape) != (b, s_q, D_K - D_V):
        raise ValueError("kv_latent must be [b, s_q, 512] and k_rope [b, s_q, 64]")
    if block_table.shape[0] != b or seqlens.shape[0] != b:
        raise ValueError("block_table and seqlens need one row per sequence")
    _check("mla_cache_append_rope", lib().mla_cache_append_rope(
        kv_latent.data_ptr(), k_rope.data_ptr(), q.data_ptr(), kv_cache.data_ptr(), block_table.data_ptr(),
        block_table.shape[1], seqlens.data_ptr(), b, s_q, h, kv_cache.shape[0], kv_cache.shape[1], float(rope_base),
        _stream(stream)))


def gqa_workspace_size(batch: int, s_q: int, num_heads: int = 16) -> int:
    out = ctypes.c_size_t(0)
    _check("mla_gqa_decode_workspace_size",
           lib().mla_gqa_decode_workspace_size(int(batch), int(s_q), int(num_heads), ctypes.byref(out)))
    return int(out.value)


def gqa_plan(seqlens, s_q: int, num_heads: int, workspace, stream=None) -> None:
    import torch
    _require(seqlens, "seqlens", torch.int32, 1)
    _require(workspace, "workspace", torch.uint8, 1, seqlens.device)
    _check("mla_gqa_decode_plan", lib().mla_gqa_decode_plan(seqlens.data_ptr(), seqlens.shape[0], int(s_q),
                                                            int(num_heads), workspace.data_ptr(), workspace.numel(),
                                                            _stream(stream)))


def gqa_fwd(q, kv_cache, block_table, seqlens, softmax_scale: float, causal: bool, workspace, out, lse,
            stream=None) -> None:
    """mla_gqa_decode_fwd: O bf16 [b, s_q, 16, 128] and LSE [b, s_q, 16] over the group's cache [pages, 64, 320]."""
    import torch
    _require(q, "q", torch.bfloat16, 4)
    dev = q.device
    _require(kv_cache, "kv_cache", torch.bfloat16, 3, dev)
    _require(block_table, "block_table", torch.int32, 2, dev)
    _require(seqlens, "seqlens", torch.int32, 1, dev)
    _require(workspace, "workspace", torch.uint8, 1, dev)
    _require(out, "out", torch.bfloat16, 4, dev)
    _require(lse, "lse", torch.float32, 3, dev)
    b, s_q, h, dk = q.shape
    if dk != GQA_D_H + 64 or kv_cache.shape[2] != GQA_ROW:
        raise ValueError("q rows must be 192 wide and cache rows 320 wide")
    if tuple(out.shape) != (b, s_q, h, GQA_D_H) or tuple(lse.shape) != (b, s_q, h):
        raise ValueError("out must be [b, s_q, h, 128] and lse [b, s_q, h]")
    _check("mla_gqa_decode_fwd", lib().mla_gqa_decode_fwd(
        q.data_ptr(), kv_cache.data_ptr(), block_table.data_ptr(), block_table.shape[1], seqlens.data_ptr(), b, s_q, h,
        kv_cache.shape[0], kv_cache.shape[1], float(softmax_scale), int(bool(causal)), workspace.data_ptr(),
        workspace.numel(), out.data_ptr(), lse.data_ptr(), _stream(stream)))


def gqa_decode(q, kv_cache, block_table, seqlens, softmax_scale: float, causal: bool = False, stream=None):
    """Allocate the workspace and outputs, plan and run one GQA-path decode step."""
    import torch
    b, s_q, h, _ = q.shape
    ws = torch.empty(gqa_workspace_size(b, s_q, h), dtype=torch.uint8, device=q.device)
    out = torch.empty((b, s_q, h, GQA_D_H), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((b, s_q, h), dtype=torch.float32, device=q.device)
    gqa_plan(seqlens, s_q, h, ws, stream)
    gqa_fwd(q, kv_cache, block_table, seqlens, softmax_scale, causal, ws, out, lse, stream)
    return out, lse


def absorb_q(q_nope, q_rope, w_uk, q=None, stream=None):
    """mla_absorb_q: the decode path's query [b, s_q, h, 576] from q_nope [b, s_q, h, 128], q_rope
    [b, s_q, h, 64] and W_UK [h, 512, 128]; allocates ``q`` if not given."""
    import torch
    _require(q_nope, "q_nope", torch.bfloat16, 4)
    dev = q_nope.device
    _require(q_rope, "q_rope", torch.bfloat16, 4, dev)
    _require(w_uk, "w_uk", torch.bfloat16, 3, dev)
    b, s_q, h, dn = q_nope.shape
    if dn != D_NOPE or tuple(q_rope.shape) != (b, s_q, h, D_K - D_V) or tuple(w_uk.shape) != (h, D_V, D_NOPE):
        raise ValueError("q_nope [b, s_q, h, 128], q_rope [b, s_q, h, 64], w_uk [h, 512, 128]")
    if q is None:
        q = torch.empty((b, s_q, h, D_K), dtype=torch.bfloat16, device=dev)
    _require(q, "q", torch.bfloat16, 4, dev)
    if tuple(q.shape) != (b, s_q, h, D_K):
        raise ValueError("q must be [b, s_q, h, 576]")
    _check("mla_absorb_q", lib().mla_absorb_q(q_nope.data_ptr(), q_rope.data_ptr(), w_uk.data_ptr(), b, s_q, h,
                                              q.data_ptr(), _stream(stream)))
    return q


def unabsorb_o(o_latent, w_uv, o=None, stream=None):
    """mla_unabsorb_o: per-head output [b, s_q, h, 128] from the decode output [b, s_q, h, 512] and
    W_UV [h, 128, 512]; allocates ``o`` if not given."""
    import torch
    _require(o_latent, "o_latent", torch.bfloat16, 4)
    dev = o_latent.device
    _require(w_uv, "w_uv", torch.bfloat16, 3, dev)
    b, s_q, h, dl = o_latent.shape
    if dl != D_V or tuple(w_uv.shape) != (h, D_NOPE, D_V):
        raise ValueError("o_latent [b, s_q, h, 512], w_uv [h, 128, 512]")
    if o is None:
        o = torch.empty((b, s_q, h, D_NOPE), dtype=torch.bfloat16, device=dev)
    _require(o, "o", torch.bfloat16, 4, dev)
    if tuple(o.shape) != (b, s_q, h, D_NOPE):
        raise ValueError("o must be [b, s_q, h, 128]")
    _check("mla_unabsorb_o", lib().mla_unabsorb_o(o_latent.data_ptr(), w_uv.data_ptr(), b, s_q, h, o.data_ptr(),
                                                  _stream(stream)))
    return o


def sparse_workspace_size(batch: int, s_q: int, num_heads: int, topk: int) -> int:
    out = ctypes.c_size_t(0)
    _check("mla_sparse_decode_workspace_size",
           lib().mla_sparse_decode_workspace_size(int(batch), int(s_q), int(num_heads), int(topk), ctypes.byref(out)))
    return int(out.value)


def sparse_plan(batch: int, s_q: int, num_heads: int, topk: int, workspace, stream=None) -> None:
    """mla_sparse_decode_plan: split metadata for this shape into ``workspace``."""
    import torch
    _require(workspace, "workspace", torch.uint8, 1)
    _check("mla_sparse_decode_plan", lib().mla_sparse_decode_plan(int(batch), int(s_q), int(num_heads), int(topk),
                                                                  workspace.data_ptr(), workspace.numel(),
                                                                  _stream(stream)))


def sparse_fwd(q, kv_cache, block_table, seqlens, indices, softmax_scale: float, workspace, out, lse,
               stream=None) -> None:
    """mla_sparse_decode_fwd: O and LSE of every head over the rows listed in ``indices`` [b, s_q, topk]."""
    import torch
    _require(q, "q", torch.bfloat16, 4)
    dev = q.device
    _require(kv_cache, "kv_cache", torch.bfloat16, 3, dev)
    _require(block_table, "block_table", torch.int32, 2, dev)
    _require(seqlens, "seqlens", torch.int32, 1, dev)
    _require(indices, "indices", torch.int32, 3, dev)
    _require(workspace, "workspace", torch.uint8, 1, dev)
    _require(out, "out", torch.bfloat16, 4, dev)
    _require(lse, "lse", torch.float32, 3, dev)
    b, s_q, h, dk = q.shape
    if dk != D_K or kv_cache.shape[2] != D_K:
        raise ValueError("q and kv_cache rows must be 576 wide")
    if tuple(indices.shape[:2]) != (b, s_q):
        raise ValueError("indices must be [b, s_q, topk]")
    if tuple(out.shape) != (b, s_q, h, D_V) or tuple(lse.shape) != (b, s_q, h):
        raise ValueError("out must be [b, s_q, h, 512] and lse [b, s_q, h]")
    _check("mla_sparse_decode_fwd", lib().mla_sparse_decode_fwd(
        q.data_ptr(), kv_cache.data_ptr(), block_table.data_ptr(), block_table.shape[1], seqlens.data_ptr(),
        indices.data_ptr(), b, s_q, h, indices.shape[2], kv_cache.shape[0], kv_cache.shape[1], float(softmax_scale),
        workspace.data_ptr(), workspace.numel(), out.data_ptr(), lse.data_ptr(), _stream(stream)))


def sparse_decode(q, kv_cache, block_table, seqlens, indices, softmax_scale: float, stream=None):
    """Allocate the workspace and outputs, plan and run one sparse decode step."""
    import torch
    b, s_q, h, _ = q.shape
    topk = indices.shape[2]
    ws = torch.empty(sparse_workspace_size(b, s_q, h, topk), dtype=torch.uint8, device=q.device)
    out = torch.empty((b, s_q, h, D_V), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((b, s_q, h), dtype=torch.float32, device=q.device)
    sparse_plan(b, s_q, h, topk, ws, stream)
    sparse_fwd(q, kv_cache, block_table, seqlens, indices, softmax_scale, ws, out, lse, stream)
    return out, lse


def decode(q, kv_cache, block_table, seqlens, softmax_scale: float, causal: bool = False, workspace=None,
           out=None, lse=None, stream=None, replan: bool = True):
    """Allocate what is missing, then plan (unless ``replan`` is False) and run one decode step."""
    import torch
    b, s_q, h, _ = q.shape
    if workspace is None:
        workspace = torch.empty(workspace_size(b, s_q, h), dtype=torch.uint8, device=q.device)
        replan = True
    if out is None:
        out = torch.empty((b, s_q, h, D_V), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((b, s_q, h), dtype=torch.float32, device=q.device)
    if replan:
        plan(seqlens, s_q, h, workspace, stream)
    fwd(q, kv_cache, block_table, seqlens, softmax_scale, causal, workspace, out, lse, stream)
    return out, lse
