/*
 * mla_decode.h -- C ABI of the MI355X (gfx950) MLA decode attention library.
 *
 * The operation is decode-time attention of Multi-Head Latent Attention in its
 * absorbed-MQA form (GQLA summary, section "Arquitetura": every query head
 * attends the shared compressed latent cache directly; a cache row is the
 * latent plus one shared RoPE key).  For every sequence b, query token
 * i < s_q and head h, with n visible keys k_0..k_{n-1} (rows of the paged cache):
 *
 *     s_j = softmax_scale * dot(q[b,i,h,0:576], k_j[0:576])
 *     LSE = ln sum_j exp(s_j)
 *     O   = sum_j exp(s_j - LSE) * k_j[0:512]        (the value is the first 512 dims)
 *
 * i.e. standard attention S = Q K^T, P = softmax(S), O = P V (FlashMLA-ETAP
 * summary, section "Mecanismo Central"), which the kernels evaluate in the
 * transposed order S^T = K Q^T, O^T = V^T P^T the same section describes.
 * Query length is 1-2 tokens and contexts reach 64K tokens (same summary,
 * "Declaracao do Problema"); 16 heads is one GPU's share of 128.
 *
 * Visible keys: n = L_b when causal == 0; when causal != 0 token i sees keys
 * 0 .. L_b - s_q + i (the s_q new tokens are the last s_q cache rows).  A row
 * with no visible key yields O = 0 and LSE = -inf.
 *
 * Conventions shared by every entry point:
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     never frees them and allocates no device memory of its own.
 *   - Every call is asynchronous and stream-ordered on `stream` (a hipStream_t,
 *     NULL = the null stream); none synchronises the host.
 *   - The current HIP device is the one used; pointers must live on it.
 *   - Arguments are validated before any HIP call; errors are returned as
 *     negative mla_status codes, never as aborts or exceptions.
 *   - Results are deterministic for a given plan (same inputs, same bits).
 */
#ifndef MLA_DECODE_H_
#define MLA_DECODE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Cache geometry fixed by the absorbed MLA layout. */
#define MLA_DECODE_D_K 576      /* latent (512) + shared RoPE key (64) */
#define MLA_DECODE_D_V 512      /* value = first 512 dims of a cache row */
#define MLA_DECODE_PAGE_SIZE 64 /* tokens per cache page */
#define MLA_DECODE_MAX_BATCH (1 << 20) /* sequences per call (decode, GQA decode, cache append) */

typedef enum mla_status {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARG = -1,         /* null pointer, non-positive size, non-finite scale ... */
    MLA_ERR_UNSUPPORTED = -2,         /* valid but unsupported: heads, s_q or page size */
    MLA_ERR_WORKSPACE_TOO_SMALL = -3, /* workspace_bytes below mla_decode_workspace_size() */
    MLA_ERR_NO_DEVICE = -4,           /* no usable gfx950 HIP device */
    MLA_ERR_HIP = -5                  /* a HIP runtime call failed (launch, attribute query) */
} mla_status;

/*
 * Bytes of device workspace that mla_decode_plan / mla_decode_fwd need for this
 * shape on the current device (the split count scales with its compute units).
 *   batch      1 .. MLA_DECODE_MAX_BATCH sequences (larger: MLA_ERR_INVALID_ARG)
 *   s_q        1 or 2 query tokens per sequence
 *   num_heads  a multiple of 16 from 16 to 128 (one GPU's share of a model's heads)
 *   bytes      out: required size
 * Returns MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED or MLA_ERR_NO_DEVICE.
 */
int mla_decode_workspace_size(int batch, int s_q, int num_heads, size_t *bytes);

/*
 * Split-KV plan: reads seqlens on the device and writes into `workspace` a
 * balanced partition of all sequences' cache pages into work items sized for
 * the device's compute units (a long sequence is cut into several items whose
 * partial results mla_decode_fwd merges by LSE).  Each item lies within one
 * sequence and holds at most `chunk` pages, where chunk is the smallest size
 * whose item count fits the resident workgroups of one launch.  One plan serves
 * every layer of a decode step as long as seqlens, batch, s_q and num_heads are
 * unchanged.
 *   seqlens    int32 [batch], device: context length L_b >= 0 of each sequence,
 *              counting the s_q new tokens
 *   workspace  device buffer of at least mla_decode_workspace_size() bytes; its
 *              contents are owned by the library until the fwd calls using it
 *              have completed on `stream`
 * Returns MLA_OK or an error code (nothing is launched on error).
 */
int mla_decode_plan(const int32_t *seqlens, int batch, int s_q, int num_heads, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * mla_decode_plan with the work-item size chosen by the caller: every item holds at most
 * chunk_pages pages (a sequence of p pages gets ceil(p / chunk_pages) items of balanced size),
 * unless that many items would exceed the workspace's capacity, in which case the automatic size
 * of mla_decode_plan is used.  chunk_pages = 0 is mla_decode_plan.  Any split gives the same
 * attention up to fp32 rounding (the partial results are merged by LSE); it serves callers that
 * fix their own split, and tests of that invariance.
 *   chunk_pages  >= 0 (negative: MLA_ERR_INVALID_ARG); other arguments as for mla_decode_plan
 */
int mla_decode_plan_chunked(const int32_t *seqlens, int batch, int s_q, int num_heads, int chunk_pages,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * Decode attention for one layer, using a plan made by mla_decode_plan with the
 * same seqlens, batch, s_q and num_heads.
 *   q            bf16 [batch][s_q][num_heads][576], contiguous
 *   kv_cache     bf16 [num_pages][64][576], contiguous paged latent cache
 *   block_table  int32 [batch][bt_stride]: entry p of row b is the pool page
 *                holding tokens 64p .. 64p+63 of sequence b; entries at or past
 *                ceil(L_b / 64) are not used (the kernels read the row in windows of up
 *                to 64 entries, always inside its bt_stride entries)
 *   bt_stride    int32 entries per block_table row (>= 1)
 *   seqlens      int32 [batch], the same values the plan was made from
 *   num_pages    pages in kv_cache (>= 1); page_size must be 64
 *   softmax_scale  scale applied to q.k (e.g. 1/sqrt(192)); it and scale * log2(e) must be finite
 *   causal       0: every query token sees all L_b keys; 1: bottom-right causal
 *   out          bf16 [batch][s_q][num_heads][512], written (round to nearest even)
 *   lse          fp32 [batch][s_q][num_heads], natural-log LSE, written
 * Device-side input errors do not fault: a sequence whose L_b is negative or
 * exceeds 64*bt_stride, or whose block_table names a page outside
 * [0, num_pages), or a plan made for other seqlens/shape, gets NaN in every
 * out/lse element of that sequence (the whole batch for a shape mismatch).
 * Cache rows past L_b in a sequence's last page are never read.
 * Returns MLA_OK or an error code (nothing is launched on error).
 */
int mla_decode_fwd(const void *q, const void *kv_cache, const int32_t *block_table, int bt_stride,
                   const int32_t *seqlens, int batch, int s_q, int num_heads, int num_pages,
                   int page_size, float softmax_scale, int causal, void *workspace,
                   size_t workspace_bytes, void *out, float *lse, void *stream);

/*
 * The two halves of mla_decode_fwd, for callers that merge partial results
 * themselves or time the halves apart.  mla_decode_fwd_split runs the split-KV
 * attention over the plan's work items and leaves each item's normalised
 * partial output (fp32) and LSE in `workspace`; mla_decode_fwd_combine merges
 * them per (sequence, query token, head) by LSE -- with M = max_s LSE_s,
 * LSE = M + ln sum_s exp(LSE_s - M) and O = sum_s exp(LSE_s - LSE) O_s -- and
 * writes `out` and `lse` exactly as mla_decode_fwd does.  Calling split then
 * combine on one stream is bit-identical to mla_decode_fwd.  Arguments mean
 * what they mean for mla_decode_fwd; the combine needs no cache inputs.
 */
int mla_decode_fwd_split(const void *q, const void *kv_cache, const int32_t *block_table,
                         int bt_stride, const int32_t *seqlens, int batch, int s_q, int num_heads,
                         int num_pages, int page_size, float softmax_scale, int causal,
                         void *workspace, size_t workspace_bytes, void *stream);

int mla_decode_fwd_combine(const int32_t *seqlens, int bt_stride, int batch, int s_q,
                           int num_heads, void *workspace, size_t workspace_bytes, void *out,
                           float *lse, void *stream);

/*
 * For callers that cannot allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid allocation): mla_decode_plan followed by mla_decode_fwd in one call, with
 * the workspace taken from a built-in device array of MLA_DECODE_NOALLOC_SCRATCH_BYTES per GPU
 * (held from the library's load until the process ends).  No allocation is made by the call.
 * Arguments mean what they mean for mla_decode_fwd; the results are bit-identical to
 * mla_decode_plan + mla_decode_fwd on the same inputs.
 *   Returns MLA_ERR_WORKSPACE_TOO_SMALL when the shape needs more than the built-in array
 *   (mla_decode_workspace_size gives what a shape needs), and the other codes of mla_decode_fwd.
 * Every call on a GPU uses that GPU's one array: calls that overlap in time on one GPU (other
 * streams, other threads) race and give undefined results.  Calls ordered on one stream are safe.
 */
/* 128 MiB: on a 256-CU MI355X up to 382 sequences of 128 heads (191 with two query tokens), or
 * 3,829 sequences of 16 heads */
#define MLA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int mla_decode_fwd_noalloc(const void *q, const void *kv_cache, const int32_t *block_table,
                           int bt_stride, const int32_t *seqlens, int batch, int s_q, int num_heads,
                           int num_pages, int page_size, float softmax_scale, int causal, void *out,
                           float *lse, void *stream);

/*
 * GQA-path decode of GQLA: the latent expanded into g groups of keys and values, decoded as
 * standard grouped-query attention over a cache holding the group's keys and values plus the
 * shared RoPE key (GQLA summary, section "Arquitetura", item 2).  One GPU's share is one group:
 * 16 query heads (h_q / g = 16).  Readings (the pages give neither): per-group width d_h = 128
 * (MLA_GQA_D_H); one cache row per token, [k (128) | shared RoPE key (64) | v (128)]
 * (MLA_GQA_ROW = 320 bf16).  For sequence b, query token i, head h and visible rows j (as for
 * mla_decode_fwd, bottom-right causal when causal != 0):
 *     s_j = softmax_scale * dot(q[b,i,h,0:192], row_j[0:192]),  LSE = ln sum_j exp(s_j),
 *     O   = sum_j exp(s_j - LSE) * row_j[192:320].
 *   q         bf16 [batch][s_q][16][192]: [q_nope (128) | q_rope (64)] of the group's heads
 *   kv_cache  bf16 [num_pages][64][320], paged as for mla_decode_fwd
 *   out       bf16 [batch][s_q][16][128]; lse fp32 [batch][s_q][16]
 *   num_heads must be 16, s_q 1 or 2; the other arguments, the plan/workspace protocol and the
 *   device-side error rules are those of mla_decode_plan / mla_decode_fwd.
 */
#define MLA_GQA_D_H 128
#define MLA_GQA_ROW 320

int mla_gqa_decode_workspace_size(int batch, int s_q, int num_heads, size_t *bytes);

int mla_gqa_decode_plan(const int32_t *seqlens, int batch, int s_q, int num_heads, void *workspace,
                        size_t workspace_bytes, void *stream);

int mla_gqa_decode_fwd(const void *q, const void *kv_cache, const int32_t *block_table, int bt_stride,
                       const int32_t *seqlens, int batch, int s_q, int num_heads, int num_pages,
                       int page_size, float softmax_scale, int causal, void *workspace,
                       size_t workspace_bytes, void *out, float *lse, void *stream);

/*
 * Absorption and un-absorption around the decode path: the up-projections are absorbed into the
 * query and output projections so every head attends the latent cache directly (GQLA summary,
 * section "Arquitetura", item 1).  The per-head no-RoPE width is 128 (MLA_DECODE_D_NOPE, a
 * reading: the pages give only the latent and RoPE widths).  Per head h and query token
 * m = b * s_q + i, in fp32 from bf16 inputs, outputs rounded once to bf16 (nearest even):
 *   mla_absorb_q:    q[m][h][0:512] = W_UK[h] q_nope[m][h],  q[m][h][512:576] = q_rope[m][h]
 *   mla_unabsorb_o:  o[m][h][0:128] = W_UV[h] o_latent[m][h]
 * so that attention of the absorbed query over the latent cache followed by the un-absorption
 * equals attention with per-head keys W_UK[h]^T c_j (plus the RoPE key) and values W_UV[h] c_j.
 *   q_nope    bf16 [batch][s_q][num_heads][128], device, 16-B aligned
 *   q_rope    bf16 [batch][s_q][num_heads][64], device, 16-B aligned
 *   w_uk      bf16 [num_heads][512][128], device: row n of W_UK[h] holds the 128 no-RoPE weights of
 *             latent dim n
 *   q         bf16 [batch][s_q][num_heads][576], device, written (the decode path's query)
 *   o_latent  bf16 [batch][s_q][num_heads][512], device (the decode path's output)
 *   w_uv      bf16 [num_heads][128][512], device: row d of W_UV[h] maps the latent to output dim d
 *   o         bf16 [batch][s_q][num_heads][128], device, written
 * num_heads and s_q as for mla_decode_fwd.  Returns MLA_OK or an error code (nothing launched).
 */
#define MLA_DECODE_D_NOPE 128

int mla_absorb_q(const void *q_nope, const void *q_rope, const void *w_uk, int batch, int s_q,
                 int num_heads, void *q, void *stream);

int mla_unabsorb_o(const void *o_latent, const void *w_uv, int batch, int s_q, int num_heads,
                   void *o, void *stream);

/*
 * Sparse (top-k) decode: every head of query token (b, i) attends exactly the cache rows that
 * token's index list names instead of all L_b rows (GQLA summary, section "GQLA Esparso":
 * fine-grained sparse attention over the latent cache; how the rows are selected is an input).
 * With the rows j listed for (b, i):
 *     s_j = softmax_scale * dot(q[b,i,h,0:576], k_j),  LSE = ln sum_j exp(s_j),
 *     O = sum_j exp(s_j - LSE) * k_j[0:512].
 * Each query token is its own split-KV sequence of topk index slots, so the plan depends only on
 * (batch, s_q, num_heads, topk) and one plan serves every layer and step with that shape.
 *   num_heads  16 (one GPU's share of 128); s_q 1 or 2; topk >= 1
 *   indices    int32 [batch][s_q][topk], device: logical token positions of sequence b (its row
 *              is page block_table[b][j / 64], slot j % 64); -1 marks an unused slot; a position
 *              listed twice counts as two keys
 *   num_pages  1 .. 2^25 (cache rows are addressed with 32-bit row ids here; 2^25 pages are
 *              2.5 TB, more than one GPU holds)
 *   other arguments as for mla_decode_fwd (there is no causal flag: the lists decide)
 * Device-side input errors do not fault: a token with an index outside [0, L_b), or whose row
 * lies on a page outside [0, num_pages), or whose sequence has L_b outside [0, 64*bt_stride],
 * gets NaN in every out/lse element of that token; a token with no index gets O = 0, LSE = -inf.
 */
int mla_sparse_decode_workspace_size(int batch, int s_q, int num_heads, int topk, size_t *bytes);

int mla_sparse_decode_plan(int batch, int s_q, int num_heads, int topk, void *workspace,
                           size_t workspace_bytes, void *stream);

int mla_sparse_decode_fwd(const void *q, const void *kv_cache, const int32_t *block_table,
                          int bt_stride, const int32_t *seqlens, const int32_t *indices, int batch,
                          int s_q, int num_heads, int topk, int num_pages, int page_size,
                          float softmax_scale, void *workspace, size_t workspace_bytes, void *out,
                          float *lse, void *stream);

/*
 * The step before the decode path for the s_q new tokens of a decode step: append each token's
 * latent cache row and rotate the 64-d RoPE parts (the cache row of the absorbed form is the
 * 512-d latent plus one shared RoPE key, GQLA summary, section "Arquitetura").  For sequence b
 * and new token i, pos = L_b - s_q + i; the row at page block_table[b][pos / 64], slot pos % 64
 * of kv_cache receives kv_latent[b][i] unchanged in dims 0..511 and k_rope[b][i] rotated by pos
 * in dims 512..575, and dims 512..575 of q[b][i][h] are rotated by pos in place for every head.
 * Rotation (the rotary embedding in its original pairwise form, a reading: the pages do not give
 * the formula): the pair (x[2p], x[2p+1]) of a 64-d part turns by pos * rope_base^(-2p/64),
 * p = 0..31; it is evaluated in fp64 and rounded once to bf16 (nearest even).
 *   kv_latent  bf16 [batch][s_q][512], device
 *   k_rope     bf16 [batch][s_q][64], device, before rotation
 *   q          bf16 [batch][s_q][num_heads][576], device, dims 512..575 rotated in place
 *   kv_cache   bf16 [num_pages][64][576], device, one row written per new token
 *   block_table, bt_stride, seqlens, batch, num_pages, page_size: as for mla_decode_fwd
 *   rope_base  finite, > 1 (e.g. 10000)
 * Device-side input errors do not fault: a token whose pos is negative, whose L_b exceeds
 * 64*bt_stride or whose page is outside [0, num_pages) writes no cache row and gets NaN in the
 * rotated query dims of every head, so a following mla_decode_fwd reports it as NaN.
 * Returns MLA_OK or an error code (nothing is launched on error).
 */
int mla_cache_append_rope(const void *kv_latent, const void *k_rope, void *q, void *kv_cache,
                          const int32_t *block_table, int bt_stride, const int32_t *seqlens, int batch,
                          int s_q, int num_heads, int num_pages, int page_size, float rope_base,
                          void *stream);

/* Static, human-readable name of a status code (never NULL). */
const char *mla_decode_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H_ */
