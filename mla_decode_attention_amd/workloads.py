"""The five synthetic decode workloads, by name, and their algorithmic accounting.

Shapes stand in for the pages' DeepSeek-R1 decode measurements (16 heads per
GPU, 576-d latent rows, batch 16, contexts up to 64K; FlashMLA-ETAP summary,
"Resultados Experimentais"), with the 128-head absorbed case of the GQLA
summary ("Arquitetura").  No model weights or datasets are involved: every
value is drawn by :mod:`mla_decode_attention_amd.inputs`.

Accounting convention (GQLA summary, "Arquitetura": the absorbed path's
arithmetic intensity is about 242 FLOP/byte at s_q = 1 with 128 heads):
  * bytes: every visible cache row (576 bf16 = 1152 B) read once per sequence,
    plus Q, O (bf16) and LSE (fp32);
  * FLOPs: 2 * (576 + 512) per (query row, visible key): one 576-term dot
    product for the score and one 512-wide multiply-add for the value sum.
"""
from __future__ import annotations

import numpy as np

from .inputs import D_K, D_V, DecodeCase, make_case

ROW_BYTES = D_K * 2                     # one bf16 cache row
FLOPS_PER_ROW_KEY = 2 * (D_K + D_V)     # score dot product + value accumulation

WORKLOADS = {
    # tiny, contiguous cache (identity block table over 4 pages)
    "tiny_b1_h16_L256": dict(batch=1, s_q=1, heads=16, seqlen=256, seed=0, identity_table=True),
    # paged, mid context: 16 x 4096 tokens over a shared 1024-page pool
    "paged_b16_h16_L4096": dict(batch=16, s_q=1, heads=16, seqlen=4096, seed=1, pool_pages=1024),
    # MTP decode: s_q = 2 causal, lengths uniform in [8192, 16384], 1% of rows x8
    "mtp_b16_h16_sq2_L8K-16K": dict(batch=16, s_q=2, heads=16, seqlen=(8192, 16384), seed=2,
                                    causal=True, outlier_frac=0.01, outlier_scale=8.0),
    # long-context headline: 16 x 65536 tokens (1.2 GB of bf16 latent cache)
    "long_b16_h16_L65536": dict(batch=16, s_q=1, heads=16, seqlen=65536, seed=3),
    # all 128 heads on one GPU, 8 x 32768 tokens
    "allheads_b8_h128_L32768": dict(batch=8, s_q=1, heads=128, seqlen=32768, seed=4),
}

HEADLINE = "long_b16_h16_L65536"


def build(name: str, **overrides) -> DecodeCase:
    kw = dict(WORKLOADS[name])
    kw.update(overrides)
    return make_case(name, **kw)


def visible_keys(seqlens: np.ndarray, s_q: int, causal: bool) -> np.ndarray:
    """[b, s_q] number of keys each query token sees (bottom-right aligned causal rule)."""
    L = np.asarray(seqlens, dtype=np.int64)[:, None]
    i = np.arange(s_q, dtype=np.int64)[None, :]
    n = L - s_q + 1 + i if causal else np.broadcast_to(L, (L.shape[0], s_q))
    return np.clip(n, 0, L)


def algorithmic_bytes(seqlens, batch: int, s_q: int, heads: int) -> int:
    kv = int(np.asarray(seqlens, dtype=np.int64).sum()) * ROW_BYTES
    q = batch * s_q * heads * D_K * 2
    o = batch * s_q * heads * D_V * 2
    lse = batch * s_q * heads * 4
    return kv + q + o + lse


def algorithmic_flops(seqlens, s_q: int, heads: int, causal: bool) -> int:
    n = visible_keys(seqlens, s_q, causal)
    return int(n.sum()) * heads * FLOPS_PER_ROW_KEY
