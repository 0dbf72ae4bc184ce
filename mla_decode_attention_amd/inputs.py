"""Seeded synthetic inputs for MLA decode attention.

This module draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the GPU path (tests, bench, smoke) and the CPU
oracle consume exactly the bf16 bit patterns produced here, so they see
identical input values.

Shapes follow the pages' decode setting: a 1-2 token query with 16 (one GPU's
share of 128) or 128 heads, a 576-d latent cache row (512-d latent + 64-d RoPE
part) and contexts up to 64K tokens (FlashMLA-ETAP summary, "Declaracao do
Problema" and "Resultados Experimentais"; GQLA summary, "Arquitetura", for the
latent + shared RoPE key cache row).

Recipe (one ``numpy.random.default_rng(seed)`` stream, PCG64, in this order):
  1. context lengths: fixed, or ``integers(lo, hi, endpoint=True)`` per sequence;
  2. Q: ``standard_normal`` float32, shape [b, s_q, h, 576];
  3. pool: ``standard_normal`` float32, shape [pool_pages, 64, 576], drawn in
     chunks of 256 pages in pool order;
  4. page assignment: ``permutation(pool_pages)`` (identity for a contiguous
     cache); sequence b owns the next ceil(L_b/64) entries of that permutation;
  5. round-to-nearest-even to bf16 (steps 2 and 3 round as they draw);
  6. outlier rows (optional): per sequence ``choice(L_b, round(frac*L_b),
     replace=False)`` token rows scaled by a power of two (exact in bf16);
  7. poison: cache slots past L_b in a sequence's last page and every pool page
     no sequence owns are set to a bf16 quiet NaN, so any read of them shows.
Unused block_table entries are -1.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

D_K = 576          # latent (512) + RoPE (64) dims per cache row
D_V = 512          # values are the first 512 dims of the same row
PAGE_SIZE = 64     # tokens per cache page
BF16_QNAN = np.uint16(0x7FC0)
_CHUNK_PAGES = 256


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_QNAN
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (for display and statistics)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class DecodeCase:
    """One decode step's inputs, as host arrays of bf16 bit patterns and int32 metadata."""
    name: str
    q: np.ndarray             # uint16 [b, s_q, h, 576]
    cache: np.ndarray         # uint16 [num_pages, 64, 576]
    block_table: np.ndarray   # int32 [b, max_pages_per_seq], -1 where unused
    seqlens: np.ndarray       # int32 [b], context length including the s_q new tokens
    s_q: int
    heads: int
    causal: bool
    softmax_scale: float
    seed: int
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.cache.shape[0])

    @property
    def rows(self) -> int:
        return self.batch * self.s_q * self.heads


def make_case(name: str, batch: int, s_q: int, heads: int, seqlen, seed: int, *,
              causal: bool = False, pool_pages: int | None = None, identity_table: bool = False,
              outlier_frac: float = 0.0, outlier_scale: float = 8.0,
              softmax_scale: float = 1.0 / np.sqrt(192.0), poison: bool = True,
              table_slack: int = 0, zero_q: bool = False, row_dims: int = D_K,
              q_dims: int | None = None) -> DecodeCase:
    """Build one seeded case (recipe in the module docstring).

    ``seqlen`` is an int (every sequence), a (lo, hi) inclusive range, or a list
    of per-sequence lengths.  ``table_slack`` adds unused -1 columns to the
    block table; ``zero_q`` replaces Q by zeros after drawing it (the stream
    stays the same).  ``row_dims`` / ``q_dims`` set the cache-row and query
    widths (576 / 576 for the latent path; the GQA path uses 320 / 192).
    """
    q_dims = row_dims if q_dims is None else q_dims
    rng = np.random.default_rng(seed)
    if isinstance(seqlen, (tuple,)) and len(seqlen) == 2:
        lens = rng.integers(int(seqlen[0]), int(seqlen[1]), endpoint=True, size=batch).astype(np.int64)
    elif isinstance(seqlen, (list, np.ndarray)):
        lens = np.asarray(seqlen, dtype=np.int64)
        assert lens.shape == (batch,)
    else:
        lens = np.full(batch, int(seqlen), dtype=np.int64)
    assert (lens >= 0).all()
    pages = (lens + PAGE_SIZE - 1) // PAGE_SIZE
    need = int(pages.sum())
    pool = need if pool_pages is None else int(pool_pages)
    assert pool >= max(need, 1), "pool too small for the requested lengths"

    qf = rng.standard_normal((batch, s_q, heads, q_dims), dtype=np.float32)
    q_bits = f32_to_bf16_bits(qf)
    del qf
    if zero_q:
        q_bits[...] = 0

    cache = np.empty((pool, PAGE_SIZE, row_dims), dtype=np.uint16)
    for c0 in range(0, pool, _CHUNK_PAGES):
        c1 = min(pool, c0 + _CHUNK_PAGES)
        cache[c0:c1] = f32_to_bf16_bits(rng.standard_normal((c1 - c0, PAGE_SIZE, row_dims), dtype=np.float32))

    perm = np.arange(pool, dtype=np.int64) if identity_table else rng.permutation(pool)
    max_pages = int(pages.max()) if batch else 0
    table = np.full((batch, max(1, max_pages + table_slack)), -1, dtype=np.int32)
    off = 0
    for b in range(batch):
        table[b, :pages[b]] = perm[off:off + pages[b]]
        off += int(pages[b])

    if outlier_frac > 0.0:
        for b in range(batch):
            n_out = int(round(outlier_frac * lens[b]))
            if n_out == 0:
                continue
            toks = rng.choice(int(lens[b]), n_out, replace=False)
            for t in toks:
                pg = table[b, t // PAGE_SIZE]
                row = bf16_bits_to_f32(cache[pg, t % PAGE_SIZE]) * np.float32(outlier_scale)
                cache[pg, t % PAGE_SIZE] = f32_to_bf16_bits(row)

    if poison:
        owned = np.zeros(pool, dtype=bool)
        for b in range(batch):
            owned[table[b, :pages[b]]] = True
            tail = int(lens[b] % PAGE_SIZE)
            if tail:
                cache[table[b, pages[b] - 1], tail:, :] = BF16_QNAN
        cache[~owned] = BF16_QNAN

    return DecodeCase(name=name, q=q_bits, cache=cache, block_table=table,
                      seqlens=lens.astype(np.int32), s_q=s_q, heads=heads, causal=causal,
                      softmax_scale=float(softmax_scale), seed=seed,
                      meta=dict(pool_pages=pool, outlier_frac=outlier_frac,
                                outlier_scale=outlier_scale))


def make_append_inputs(case: DecodeCase, seed: int):
    """Seeded inputs of the cache-append step for the s_q new tokens of `case`: the latent rows
    (bf16 [b, s_q, 512]) and the RoPE keys before rotation (bf16 [b, s_q, 64]), N(0, 1) drawn in
    fp32 and rounded to bf16 (nearest even)."""
    rng = np.random.default_rng(seed)
    lat = rng.standard_normal((case.batch, case.s_q, D_V), dtype=np.float32)
    rope = rng.standard_normal((case.batch, case.s_q, D_K - D_V), dtype=np.float32)
    return f32_to_bf16_bits(lat), f32_to_bf16_bits(rope)


def make_sparse_indices(case: DecodeCase, topk: int, seed: int, *, pad_frac: float = 0.0,
                        duplicates: bool = False) -> np.ndarray:
    """Seeded top-k index lists int32 [b, s_q, topk] for `case`: for each query token, min(topk, L_b)
    distinct positions of its sequence drawn uniformly and shuffled; the remaining slots are -1.
    `pad_frac` turns that fraction of the chosen slots into -1 at random places; `duplicates`
    overwrites a quarter of the chosen slots with copies of others (a position listed twice)."""
    rng = np.random.default_rng(seed)
    out = np.full((case.batch, case.s_q, topk), -1, dtype=np.int32)
    for b in range(case.batch):
        L = int(case.seqlens[b])
        for i in range(case.s_q):
            n = min(topk, L)
            if n <= 0:
                continue
            sel = rng.choice(L, size=n, replace=False).astype(np.int32)
            if duplicates and n > 1:
                m = max(1, n // 4)
                sel[rng.choice(n, size=m, replace=False)] = sel[rng.integers(0, n, size=m)]
            row = np.full(topk, -1, dtype=np.int32)
            row[:n] = sel
            if pad_frac > 0:
                row[rng.random(topk) < pad_frac] = -1
            out[b, i] = rng.permutation(row)
    return out


def make_absorb_inputs(batch: int, s_q: int, heads: int, seed: int):
    """Seeded bf16 bit arrays for the absorption steps: q_nope [b, s_q, h, 128], q_rope [b, s_q, h, 64]
    ~ N(0, 1), and random per-head weights W_UK [h, 512, 128], W_UV [h, 128, 512] ~ N(0, 1/256)."""
    rng = np.random.default_rng(seed)
    qn = rng.standard_normal((batch, s_q, heads, 128), dtype=np.float32)
    qr = rng.standard_normal((batch, s_q, heads, D_K - D_V), dtype=np.float32)
    wuk = rng.standard_normal((heads, D_V, 128), dtype=np.float32) / 16
    wuv = rng.standard_normal((heads, 128, D_V), dtype=np.float32) / 16
    return f32_to_bf16_bits(qn), f32_to_bf16_bits(qr), f32_to_bf16_bits(wuk), f32_to_bf16_bits(wuv)
