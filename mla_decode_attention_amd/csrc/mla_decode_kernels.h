// gfx950 (CDNA4) kernels for absorbed-MLA decode attention: split-KV plan,
// paged split kernel (bf16 MFMA score and value contractions, fp32 online
// softmax) and LSE combine.
//
// What is computed (FlashMLA-ETAP summary, "Mecanismo Central"): softmax
// attention, evaluated in the transposed order S^T = K Q^T, P^T = softmax of
// S^T down the key axis, O^T = V^T P^T.  On gfx950 the transposed order is
// what keeps every softmax statistic in one lane: in the 16x16 MFMA result
// layout a lane holds one column (here: one query row) and four consecutive
// rows (here: tokens), so the S^T accumulator is already the P^T operand of
// the value contraction, and the O^T accumulator holds the same query row in
// the same lane -- the per-row rescale needs no cross-lane traffic.
//
// Cache rows are 576 bf16 (latent 512 + shared RoPE key 64; GQLA summary,
// "Arquitetura"); the value is the first 512 dims of the same row, so a tile
// is staged once in LDS and read twice: row-major for K, transposed
// (ds_read_b64_tr_b16) for V^T.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mla {

constexpr int kDk = 576;
constexpr int kDv = 512;
constexpr int kPage = 64;
constexpr int kRowBytes = kDk * 2;          // 1152
constexpr int kChunksPerRow = kRowBytes / 16;  // 72 chunks of 16 B
constexpr int kLdsRow = kRowBytes + 32;        // LDS row stride: 1184 B = 74 chunks, see below
constexpr int kKSteps = kDk / 32;           // 18 score MFMA k-steps of 32
constexpr int kDTiles = kDv / 16;           // 32 output tiles of 16 dims
constexpr int kPlanMagic = 0x4D4C4131;      // "MLA1"
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNonTemporal = 2;             // buffer-load cache policy: stream the cache through

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
#define MLA_LDS __attribute__((address_space(3)))

// ---------------------------------------------------------------------------------------------
// Workspace layout (all offsets 256-byte aligned), written by the plan kernel and the split
// kernel, read by the split and combine kernels.
//   header      int32[16]: magic, batch, s_q, heads, n_items, item capacity, rows per sequence
//   seqlens     int32[batch]      copy of the plan's seqlens
//   batch_split int32[batch + 1]  first work item of each sequence (prefix sum)
//   items       int4[capacity]    (sequence, first page, end page, split index)
//   lse_part    fp32[capacity][rows]       log-sum-exp of each item's rows (natural log)
//   o_part      fp32[capacity][rows][512]  normalised partial output of each item
// ---------------------------------------------------------------------------------------------
struct WsLayout {
    size_t header, seqlens, batch_split, items, lse_part, o_part, total;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// dv: width of a partial output row (512 for the latent path); only the last section depends on it
__host__ __device__ inline WsLayout ws_layout(int batch, int rows, int capacity, int dv = kDv)
{
    WsLayout w;
    size_t off = 0;
    w.header = off;      off = align256(off + 16 * sizeof(int32_t));
    w.seqlens = off;     off = align256(off + size_t(batch) * sizeof(int32_t));
    w.batch_split = off; off = align256(off + size_t(batch + 1) * sizeof(int32_t));
    w.items = off;       off = align256(off + size_t(capacity) * 4 * sizeof(int32_t));
    w.lse_part = off;    off = align256(off + size_t(capacity) * rows * sizeof(float));
    w.o_part = off;      off = align256(off + size_t(capacity) * rows * dv * sizeof(float));
    w.total = off;
    return w;
}

enum HeaderField { kHMagic = 0, kHBatch, kHSq, kHHeads, kHItems, kHCapacity, kHRows };

// =============================================================================================
// Split kernel.
//
// A workgroup takes one work item (sequence b, page range) and one row group (RB blocks of 16
// query rows; rows are ordered [s_q][heads]).  Its NW waves form NG = NW/RB wave groups; each
// group streams its own share of the item's TT-token tiles (round robin) through NS LDS stages,
// the RB waves of a group sharing each stage, one 16-row block per wave.
//
// Tiles move HBM -> VGPR -> LDS: every load instruction of a wave reads one contiguous KiB of
// the tile (16 B per lane, the access that streams fastest), NR tiles per wave are in flight in
// registers, and each arrived tile is stored to LDS just before it is needed.  The buffer
// resource of a tile ends at the sequence's last valid row, so rows past L_b load as zeros and
// never reach the value contraction (0 * NaN would poison it).
//
// LDS tile layout: row r of a tile starts at r * 1184 B (32 B of padding per 1152-B row).  With
// 74 16-B chunks per row (2 x odd), the 32 lanes a K-operand read serves together -- 16 rows x
// two 16-B chunks -- land on 32 distinct 16-B bank groups of a 512-B bank line (measured: 222
// B/clk/CU for this pattern vs 122 with 16 B of padding and 62 with none).
// =============================================================================================
template <int NW_, int RB_, int DS_, int TT_, int NS_, int NR_>
struct SplitCfg {
    static constexpr int NW = NW_;            // waves per workgroup
    static constexpr int RB = RB_;            // 16-row blocks per wave group
    static constexpr int DS = DS_;            // output segments: waves sharing a row block, each
                                              // accumulating 512/DS of the value dims
    static constexpr int GW = RB * DS;        // waves per group
    static constexpr int NG = NW / GW;        // wave groups
    static constexpr int TT = TT_;            // tokens per tile (16, 32 or 64)
    static constexpr int NS = NS_;            // LDS stages per group
    static constexpr int NR = NR_;            // tiles in flight in registers per wave
    static constexpr int NST = TT / 16;       // 16-token sub-tiles per tile
    static constexpr int DTW = kDTiles / DS;  // 16-dim output tiles per wave
    static constexpr int TILE_BYTES = TT * kRowBytes;        // in HBM
    static constexpr int LDS_TILE = TT * kLdsRow;            // in LDS (padded rows)
    static constexpr int UNITS = TILE_BYTES / 1024;          // 1-KiB load units per tile
    static constexpr int NPW = UNITS / GW;                   // load units per wave per tile
    static constexpr int STAGE_BYTES = NG * NS * LDS_TILE;
    // merge scratch (reuses the stage area): m, l per wave + fp32 accumulators
    static constexpr int MERGE_BYTES = NG > 1 ? NW * (2 * 16 * 4 + 16 * (kDv / DS) * 4) : 0;
    static constexpr int LDS_BYTES = STAGE_BYTES > MERGE_BYTES ? STAGE_BYTES : MERGE_BYTES;
    static constexpr int THREADS = NW * 64;
    static_assert(NW % GW == 0, "waves must split into whole groups");
    static_assert(DS == 1 || DS == 2 || DS == 4, "output segments");
    static_assert(TT == 16 || TT == 32 || TT == 64, "tile is 1, 2 or 4 MFMA token blocks");
    static_assert(TILE_BYTES % 1024 == 0, "tile must be whole load units");
    static_assert(NPW * GW == UNITS && NPW % 9 == 0, "each wave loads whole 8-row groups (9 KiB)");
    static_assert(NR == 1 || NR == 2, "one or two tiles in flight per wave");
    static_assert(GW == 1 || NS == 2, "shared stages need double buffering");
    static_assert(NS == 1 || NS == 2, "one or two stages");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

struct FwdArgs {
    const uint16_t* q;
    const uint16_t* cache;
    const int32_t* block_table;
    const int32_t* seqlens;
    char* ws;
    uint16_t* out;
    float* lse;
    long long num_pages;
    int bt_stride;
    int batch, s_q, heads, rows, capacity;
    float scale_log2;   // softmax_scale * log2(e)
    int causal;
    int row_groups;     // workgroups per work item (wide form)
    // sparse (top-k) decode: each query token is a sequence of `topk` index slots; `batch` and
    // `s_q` above then count query tokens (batch * sparse_sq) and 1
    const int32_t* indices;   // int32 [b][sparse_sq][topk] logical token positions, -1 = unused
    int topk;
    int sparse_sq;
};

// The plan header and one work item's record, read together in one memory round trip: the
// record index is clamped into the item array, so the read stays in bounds whatever the header
// holds, and the checks use no short-circuit (which would put each header field behind its own
// load-and-wait).  ok: the header matches this launch and the item exists.
struct PlanItem {
    bool ok;
    i32x4 it;   // (sequence, first page, end page, split index)
};

__device__ inline PlanItem read_plan_item(const FwdArgs& a, const WsLayout& lay, int item)
{
    PlanItem p;
    p.it = reinterpret_cast<const i32x4*>(a.ws + lay.items)[min(item, a.capacity - 1)];
    const i32x4 h0 = *reinterpret_cast<const i32x4*>(a.ws + lay.header);
    const int2 h1 = *reinterpret_cast<const int2*>(a.ws + lay.header + 4 * sizeof(int32_t));   // items, capacity
    // the record's sequence index takes part in the check, so its load is issued with the header's
    p.ok = (h0[kHMagic] == kPlanMagic) & (h0[kHBatch] == a.batch) & (h0[kHSq] == a.s_q) &
           (h0[kHHeads] == a.heads) & (h1.y == a.capacity) & (item < h1.x) &
           ((unsigned)p.it[0] < (unsigned)a.batch);
    return p;
}

__device__ inline const MLA_LDS i16x4* lds_i16x4(const void* p)
{
    return (const MLA_LDS i16x4*)(const MLA_LDS char*)p;
}

// Reductions across the four 16-lane groups of a wave (lanes l, l^16, l^32, l^48), with the
// gfx950 row-swap permutes: permlane16_swap exchanges 16-lane rows 0<->1 and 2<->3 between its
// two results, permlane32_swap the 32-lane halves, so op(first, second) combines each lane with
// its partner.
__device__ inline float wave_max_groups(float v)
{
    auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

__device__ inline float wave_sum_groups(float v)
{
    auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

__device__ inline uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// A 64-entry window of one sequence's block table, one entry per lane of a VGPR: page ids are
// then read with v_readlane (a few cycles) instead of a scalar load per tile, whose latency
// would stall the next tile's loads.  The window moves (one vector load) every 64 pages.
struct PageWindow {
    const int32_t* row;   // block-table row of the sequence
    int len;              // entries in the row (bt_stride)
    int base;             // first entry held (wave-uniform), -1 = none
    int val;              // lane i: row[base + i]

    __device__ inline void init(const int32_t* r, int n)
    {
        row = r;
        len = n;
        base = -1;
        val = 0;
    }
    // fill the window at idx without waiting: the first page() call waits for this load alone
    __device__ inline void prefetch(int idx, int lane)
    {
        base = idx;
        const int v = row[min(idx + lane, len - 1)];   // no branch: every lane loads in bounds
        val = (idx + lane < len) ? v : -1;
    }
    __device__ inline int page(int idx, int lane)
    {
        if (base < 0 || idx < base || idx >= base + 64) {
            base = idx;
            val = (idx + lane < len) ? row[idx + lane] : -1;
            // wait here for the refill (vmcnt 0 only), so the common path needs no wait on the
            // tile loads in flight before its readlane
            __builtin_amdgcn_s_waitcnt(0x0F70);
        }
        return __builtin_amdgcn_readlane(val, idx - base);
    }
};

// Partial outputs are written once and read once by the combine kernel on whichever XCD it runs:
// streaming (non-temporal) stores send them on to memory during the kernel instead of leaving
// them dirty in this XCD's L2 for the write-back at the kernel's end.
__device__ inline void store_partial(float* p, f32x4 v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}

template <int B>
struct Idx {
    static constexpr int value = B;
};

// SPARSE: the keys of a sequence are the cache rows its index list names (gathered row by row)
// instead of its first L_b rows; see the sparse entry point of the C ABI.
template <class C, bool SPARSE = false>
__global__ void __launch_bounds__(C::THREADS) split_kernel(FwdArgs a)
{
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int gi = wave / C::GW;            // wave group
    const int wg = wave % C::GW;            // wave within the group
    const int rbl = wg / C::DS;             // row block within the group
    const int dsi = wg % C::DS;             // output segment: value dims [512 dsi / DS, ...)
    const int dt0 = dsi * C::DTW;           // first 16-dim output tile of this wave
    const int lr = lane & 15;               // lane's query row within its block (MFMA column)
    const int lg = lane >> 4;               // lane group (MFMA k / row quad)

    const WsLayout lay = ws_layout(a.batch, a.rows, a.capacity);
    // the arguments of the prologue's address computations come in with the first ones
    asm volatile("" ::"s"(a.q), "s"(a.block_table), "s"(a.seqlens), "s"(a.bt_stride));
    const int item = blockIdx.x;
    const PlanItem pi = read_plan_item(a, lay, item);
    if (!pi.ok) return;   // a plan mismatch is reported by the combine kernel
    const i32x4 it = pi.it;
    const int b = it[0];              // sequence (sparse: query token b_real * sparse_sq + i)
    // dense: L = context length; sparse: L = index slots, Lc = the context the indices point into
    const int b_tab = SPARSE ? b / a.sparse_sq : b;
    // The first block-table window, the lengths and Q go out together (one round trip) before
    // anything waits for them; every address here is valid once the plan matched.
    PageWindow pw;
    pw.init(a.block_table + (size_t)b_tab * a.bt_stride, a.bt_stride);
    if constexpr (!SPARSE) pw.prefetch(it[1], lane);
    const int32_t plan_L = reinterpret_cast<const int32_t*>(a.ws + lay.seqlens)[b];
    const int Lc = a.seqlens[b_tab];
    const int L = SPARSE ? a.topk : Lc;
    float* lse_part = reinterpret_cast<float*>(a.ws + lay.lse_part) + (size_t)item * a.rows;
    float* o_part = reinterpret_cast<float*>(a.ws + lay.o_part) + (size_t)item * a.rows * kDv;

    const int rb = blockIdx.y * C::RB + rbl;          // global 16-row block
    const int row0 = rb * 16;
    const int qi = row0 / a.heads;                    // query token of this block (heads % 16 == 0)

    // ---- Q^T operand (B of the score MFMA): lane (row lr, group lg) holds q[row][32j+8lg .. +8]
    bf16x8 qop[kKSteps];
    {
        const int row = row0 + lr;
        const uint16_t* qrow = a.q + ((size_t)(b * a.s_q + row / a.heads) * a.heads + row % a.heads) * kDk;
#pragma unroll
        for (int j = 0; j < kKSteps; ++j)
            qop[j] = *reinterpret_cast<const bf16x8*>(qrow + 32 * j + 8 * lg);
    }

    // A sequence whose length disagrees with the plan or the table gets no tiles and a NaN LSE
    // (no early exit: a branch here would make the loads above wait one after another).
    const bool bad_seq = (L != plan_L) | (L < 0) | (Lc < 0) | ((long long)Lc > (long long)kPage * a.bt_stride);
    const int n_vis = (!SPARSE && a.causal) ? min(max(L - a.s_q + 1 + qi, 0), L) : L;
    const int tok_begin = it[1] * kPage;
    const int tok_end = (int)min((long long)it[2] * kPage, (long long)L);   // it[2] * 64 may reach 2^31
    const int n_tiles = bad_seq ? 0 : (tok_end - tok_begin + C::TT - 1) / C::TT;
    const int n_it = (n_tiles + C::NG - 1) / C::NG;

    // ---- this wave's load units of a tile: unit u covers tile bytes [1024 u, 1024 u + 1024);
    // lane l takes 16-B chunk P = 64 u + l of row r = P / 72, which goes to LDS byte 16 P + 32 r.
    // Nine units cover exactly eight rows, so the lane part of the LDS offset depends only on
    // u mod 9 (st9[v]); each wave loads NPW consecutive units, a whole number of 8-row groups.
    const uint32_t lane16 = (uint32_t)lane * 16u;
    int st9[9];
#pragma unroll
    for (int v = 0; v < 9; ++v) {
        const int r0 = (64 * v) / kChunksPerRow;          // row of lane 0 within the 8-row group
        const int bnd = kChunksPerRow * (r0 + 1) - 64 * v; // first lane in row r0 + 1
        st9[v] = v * 1024 + (kLdsRow - kRowBytes) * (r0 + (lane >= bnd ? 1 : 0)) + (int)lane16;
    }
    const int unit0 = wg * C::NPW;                           // first unit of this wave
    char* const group_stages = smem + gi * C::NS * C::LDS_TILE;
    bool bad_page = bad_seq;

    i32x4 rbuf[C::NR][C::NPW];
    // sparse: validity masks (bit r = index slot r of the tile names a row) of the tiles loaded but
    // not yet computed, oldest first; tile itn of the prologue goes to slot itn, later tiles to
    // slot NR (each step shifts the queue after its compute)
    uint32_t vmq[C::NR + 1] = {};
    auto gather_tile = [&](int itn, int t0, auto buf_idx) {   // SPARSE only: rows of slots t0 .. t0+TT-1
        constexpr int B = decltype(buf_idx)::value;
        static_assert(C::TT == 16 && C::GW == 1, "the gather path takes one 16-token tile per wave");
        int rowid = 0;      // lane r < 16: page * 64 + slot of the row of slot t0 + r
        bool ok = false, bad = false;
        if (lane < C::TT && t0 + lane < tok_end) {
            const int idx = a.indices[(size_t)b * a.topk + t0 + lane];
            if (idx >= 0) {
                if (idx >= Lc) {
                    bad = true;
                } else {
                    const int page = a.block_table[(size_t)b_tab * a.bt_stride + idx / kPage];
                    if (page < 0 || (long long)page >= a.num_pages)
                        bad = true;
                    else {
                        rowid = page * kPage + idx % kPage;
                        ok = true;
                    }
                }
            }
        }
        if (__builtin_amdgcn_ballot_w64(bad) != 0) bad_page = true;   // the whole token is poisoned
        const uint32_t vmask = (uint32_t)__builtin_amdgcn_ballot_w64(ok);
        if (itn <= 0)
            vmq[0] = vmask;
        else if (C::NR == 1 || itn == 1)
            vmq[1] = vmask;
        else
            vmq[C::NR] = vmask;
#pragma unroll
        for (int kk = 0; kk < C::NPW; ++kk) {
            const int c = 64 * (unit0 + kk) + lane;   // 16-B chunk of the tile
            const int r = c / kChunksPerRow;
            const int rid = __shfl(rowid, r);
            if ((vmask >> r) & 1u) {
                const i32x4* src = reinterpret_cast<const i32x4*>(a.cache + (size_t)rid * kDk) + (c - r * kChunksPerRow);
                rbuf[B][kk] = __builtin_nontemporal_load(src);
            } else {
                rbuf[B][kk] = i32x4{0, 0, 0, 0};
            }
        }
    };
    auto load_tile = [&](int itn, auto buf_idx) {
        constexpr int B = decltype(buf_idx)::value;
        const int k = itn * C::NG + gi;
        if (itn >= n_it || k >= n_tiles) return;
        const int t0 = tok_begin + k * C::TT;
        if constexpr (SPARSE) {
            gather_tile(itn, t0, buf_idx);
            return;
        }
        const int page = pw.page(t0 / kPage, lane);
        int valid = min(C::TT, L - t0);
        if (page < 0 || (long long)page >= a.num_pages) {
            bad_page = true;
            valid = 0;
        }
        const uint16_t* base = a.cache + ((long long)(valid ? page : 0) * kPage + (t0 % kPage)) * kDk;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, valid * kRowBytes, 0x00020000);
#pragma unroll
        for (int kk = 0; kk < C::NPW; ++kk)
            rbuf[B][kk] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)lane16, (unit0 + kk) * 1024, kNonTemporal);
    };
    auto store_tile = [&](int itn, auto buf_idx) {
        constexpr int B = decltype(buf_idx)::value;
        const int k = itn * C::NG + gi;
        if (itn >= n_it || k >= n_tiles) return;
        char* stg = group_stages + (itn % C::NS) * C::LDS_TILE + (unit0 / 9) * (8 * kLdsRow);
#pragma unroll
        for (int kk = 0; kk < C::NPW; ++kk)
            *reinterpret_cast<i32x4*>(stg + st9[kk % 9] + (kk / 9) * (8 * kLdsRow)) = rbuf[B][kk];
    };

    // ---- online softmax state: row lr; acc[t] holds O^T[16 (dt0 + t) + 4 lg + i][row lr]
    f32x4 acc[C::DTW];
#pragma unroll
    for (int dt = 0; dt < C::DTW; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -__builtin_inff();
    float l_run = 0.f;   // lane-partial sum over this lane's tokens

    // K-operand LDS address: row 16 st + lr, bytes 64 j + 16 lg (chunk 4j + lg)
    const int kbase = lr * kLdsRow + 16 * lg;
    // V^T tr-read address: lane (group lg, i = lr) reads row 4 lg + (lr >> 2) (+16 st), dims
    // 16 dt + 4 (lr & 3) .. +3
    const int vbase = (4 * lg + (lr >> 2)) * kLdsRow + 8 * (lr & 3);

    // Softmax statistics are rescaled lazily: the running max m_run only moves when a tile's
    // max exceeds it by more than kLazyRescale (log2 units), so exp2(s - m_run) <= 2^kLazyRescale
    // and most tiles skip the accumulator rescale; LSE = m_run + log2(l) stays exact.
    constexpr float kLazyRescale = 8.f;
    auto kread = [&](const char* p) { return *reinterpret_cast<const bf16x8*>(p); };
    auto vread = [&](const char* p) {
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)lds_i16x4(p));
    };
    auto compute_tile = [&](int itn, int k) {
        const int t0 = tok_begin + k * C::TT;
        const char* stg = group_stages + (itn % C::NS) * C::LDS_TILE;

        // scores S^T[token][row]: a dependent MFMA chain issues only every ~50 cycles, so each
        // 16-token block accumulates NCH independent partial sums over alternating k-steps
        // (NST * NCH = 4 chains in flight) that are added at the end; K operands are read KD
        // k-steps ahead (the gather form holds more addressing state: 4 keep it clear of spills,
        // at the same speed)
        constexpr int KD = C::NST == 1 ? (SPARSE ? 4 : 6) : 3;
        constexpr int NCH = C::NST >= 4 ? 1 : 4 / C::NST;
        f32x4 s[C::NST];
        f32x4 sp[C::NST][NCH];
        bf16x8 kop[KD + 1][C::NST];
#pragma unroll
        for (int st = 0; st < C::NST; ++st) {
#pragma unroll
            for (int c = 0; c < NCH; ++c) sp[st][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KD; ++j) kop[j][st] = kread(stg + st * 16 * kLdsRow + kbase + 64 * j);
        }
#pragma unroll
        for (int j = 0; j < kKSteps; ++j) {
            if (j + KD < kKSteps) {
#pragma unroll
                for (int st = 0; st < C::NST; ++st)
                    kop[(j + KD) % (KD + 1)][st] = kread(stg + st * 16 * kLdsRow + kbase + 64 * (j + KD));
            }
#pragma unroll
            for (int st = 0; st < C::NST; ++st)
                sp[st][j % NCH] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[j % (KD + 1)][st], qop[j], sp[st][j % NCH], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int st = 0; st < C::NST; ++st) {
            s[st] = sp[st][0];
#pragma unroll
            for (int c = 1; c < NCH; ++c) s[st] += sp[st][c];
        }
        // first V^T operands of the value contraction do not depend on P: start them now
        constexpr int VD = C::NST == 1 ? 6 : 3;   // d-tiles of look-ahead
        const char* vt0 = stg + vbase + 32 * dt0;
        i16x4 vlo[VD + 1], vhi[VD + 1];
#pragma unroll
        for (int d = 0; d < VD; ++d) {
            vlo[d] = vread(vt0 + 32 * d);
            if constexpr (C::NST >= 2) vhi[d] = vread(vt0 + 16 * kLdsRow + 32 * d);
        }
        // scale into the log2 domain, mask invisible tokens (only in a tile that crosses n_vis)
#pragma unroll
        for (int st = 0; st < C::NST; ++st) s[st] *= a.scale_log2;
        if constexpr (SPARSE) {
            const uint32_t vm = vmq[0];
            if (vm != (1u << C::TT) - 1u) {
#pragma unroll
                for (int st = 0; st < C::NST; ++st)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (!((vm >> (16 * st + 4 * lg + i)) & 1u)) s[st][i] = -__builtin_inff();
            }
        } else if (t0 + C::TT > n_vis) {
#pragma unroll
            for (int st = 0; st < C::NST; ++st)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (t0 + 16 * st + 4 * lg + i >= n_vis) s[st][i] = -__builtin_inff();
        }
        float tmax = -__builtin_inff();
#pragma unroll
        for (int st = 0; st < C::NST; ++st)
            tmax = fmaxf(tmax, fmaxf(fmaxf(s[st][0], s[st][1]), fmaxf(s[st][2], s[st][3])));
        tmax = wave_max_groups(tmax);
        if (__builtin_amdgcn_ballot_w64(tmax > m_run + kLazyRescale) != 0) {
            const float m_new = fmaxf(m_run, tmax);
            const float alpha = (m_new == -__builtin_inff()) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
            // one accumulator tile at a time (the fences keep the scheduler from staging all 128
            // accumulators in temporaries at once)
#pragma unroll
            for (int dt = 0; dt < C::DTW; ++dt) {
                acc[dt] *= alpha;
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        const float m_use = (m_run == -__builtin_inff()) ? 0.f : m_run;
        float psum = 0.f;
        float p[C::NST][4];
#pragma unroll
        for (int st = 0; st < C::NST; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[st][i] = __builtin_amdgcn_exp2f(s[st][i] - m_use);
                psum += p[st][i];
            }
        l_run += psum;

        // O^T[d][row] += V^T[d][token] P^T[token][row]; V^T comes straight from the K rows in
        // LDS through transposing reads, two d-tiles ahead of their MFMA
        if constexpr (C::NST >= 2) {
#pragma unroll
            for (int h = 0; h < C::NST / 2; ++h) {   // 32-token k-steps
                bf16x8 pop;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pop[i] = (__bf16)p[2 * h][i];
                    pop[4 + i] = (__bf16)p[2 * h + 1][i];
                }
                const char* vh = vt0 + 32 * h * kLdsRow;
                if (h > 0) {
#pragma unroll
                    for (int d = 0; d < VD; ++d) {
                        vlo[d] = vread(vh + 32 * d);
                        vhi[d] = vread(vh + 16 * kLdsRow + 32 * d);
                    }
                }
#pragma unroll
                for (int dt = 0; dt < C::DTW; ++dt) {
                    if (dt + VD < C::DTW) {
                        vlo[(dt + VD) % (VD + 1)] = vread(vh + 32 * (dt + VD));
                        vhi[(dt + VD) % (VD + 1)] = vread(vh + 16 * kLdsRow + 32 * (dt + VD));
                    }
                    const bf16x8 vop = __builtin_shufflevector(__builtin_bit_cast(bf16x4, vlo[dt % (VD + 1)]),
                                                               __builtin_bit_cast(bf16x4, vhi[dt % (VD + 1)]),
                                                               0, 1, 2, 3, 4, 5, 6, 7);
                    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop, acc[dt], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
            bf16x4 pop;
#pragma unroll
            for (int i = 0; i < 4; ++i) pop[i] = (__bf16)p[0][i];
#pragma unroll
            for (int dt = 0; dt < C::DTW; ++dt) {
                if (dt + VD < C::DTW) vlo[(dt + VD) % (VD + 1)] = vread(vt0 + 32 * (dt + VD));
                acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, vlo[dt % (VD + 1)]),
                                                                   pop, acc[dt], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // ---- pipeline: tile itn+1 waits in registers while tile itn is computed from LDS; then it
    // is stored to LDS and the registers take tile itn+1+NR.
    auto step = [&](int itn, auto next_buf) {
        if (itn >= n_it) return;
        const int k = itn * C::NG + gi;
        if (k < n_tiles) compute_tile(itn, k);
        if constexpr (SPARSE) {
#pragma unroll
            for (int i = 0; i < C::NR; ++i) vmq[i] = vmq[i + 1];
        }
        store_tile(itn + 1, next_buf);
        load_tile(itn + 1 + C::NR, next_buf);
        if constexpr (C::GW > 1) __syncthreads();
    };
    load_tile(0, Idx<0>{});
    if constexpr (C::NR == 2) load_tile(1, Idx<1>{});
    store_tile(0, Idx<0>{});
    load_tile(C::NR, Idx<0>{});
    // Consume Q here, so that no wait for it lands inside the tile loop (where it would also wait
    // for the tile loads in flight)
#pragma unroll
    for (int j = 0; j < kKSteps; ++j) asm volatile("" ::"v"(qop[j]));
    if constexpr (C::GW > 1) __syncthreads();
    if constexpr (C::NR == 2) {
        for (int itn = 0; itn < n_it; itn += 2) {
            step(itn, Idx<1>{});
            step(itn + 1, Idx<0>{});
        }
    } else {
        for (int itn = 0; itn < n_it; ++itn) step(itn, Idx<0>{});
    }
    l_run = wave_sum_groups(l_run);

    // ---- epilogue: merge the NG wave groups of each (row block, segment), write the partials
    const int out_row = row0 + lr;   // row within the sequence (of a.rows)
    if constexpr (C::NG == 1) {
        const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
        float* orow = o_part + (size_t)out_row * kDv + 16 * dt0;
#pragma unroll
        for (int dt = 0; dt < C::DTW; ++dt)
            store_partial(orow + 16 * dt + 4 * lg, acc[dt] * inv);
        if (lg == 0 && dsi == 0)
            lse_part[out_row] = bad_page ? __builtin_nanf("")
                                         : (l_run > 0.f ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2
                                                        : -__builtin_inff());
    } else {
        constexpr int SEG = kDv / C::DS;                                 // value dims per wave
        __syncthreads();   // every wave is done with the stages
        float* ml = reinterpret_cast<float*>(smem);                       // [NW][2][16]
        float* accs = reinterpret_cast<float*>(smem + C::NW * 2 * 16 * 4);  // [NW][16][SEG]
        if (lg == 0) {
            ml[(wave * 2 + 0) * 16 + lr] = m_run;
            ml[(wave * 2 + 1) * 16 + lr] = bad_page ? __builtin_nanf("") : l_run;
        }
        float* my = accs + (size_t)wave * 16 * SEG + lr * SEG;
#pragma unroll
        for (int dt = 0; dt < C::DTW; ++dt) *reinterpret_cast<f32x4*>(my + 16 * dt + 4 * lg) = acc[dt];
        __syncthreads();
        // GW waves' worth of (row block, segment) outputs: 16 rows x SEG dims each, all threads
        for (int e = tid; e < C::GW * 16 * (SEG / 4); e += C::THREADS) {
            const int d4 = e % (SEG / 4);
            const int r = (e / (SEG / 4)) % 16;
            const int w0 = e / (16 * (SEG / 4));                          // wave index within a group
            float M = -__builtin_inff();
            for (int g = 0; g < C::NG; ++g) M = fmaxf(M, ml[((g * C::GW + w0) * 2) * 16 + r]);
            const float Mu = (M == -__builtin_inff()) ? 0.f : M;
            float Lsum = 0.f;
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
            bool nan = false;
            for (int g = 0; g < C::NG; ++g) {
                const int w = g * C::GW + w0;
                const float lw = ml[(w * 2 + 1) * 16 + r];
                nan |= (lw != lw);
                const float sc = __builtin_amdgcn_exp2f(ml[(w * 2) * 16 + r] - Mu);
                Lsum += sc * lw;
                o += sc * *reinterpret_cast<const f32x4*>(accs + ((size_t)w * 16 + r) * SEG + 4 * d4);
            }
            const float inv = (Lsum > 0.f) ? 1.f / Lsum : 0.f;
            const int rbi = w0 / C::DS, seg = w0 % C::DS;
            const int grow = (blockIdx.y * C::RB + rbi) * 16 + r;
            store_partial(o_part + (size_t)grow * kDv + seg * SEG + 4 * d4, o * inv);
            if (d4 == 0 && seg == 0)
                lse_part[grow] = nan ? __builtin_nanf("")
                                     : (Lsum > 0.f ? (M + __builtin_amdgcn_logf(Lsum)) * kLn2 : -__builtin_inff());
        }
    }
}

// =============================================================================================
// Combine: per (sequence, row) merge the items' normalised partials by their LSE,
//   LSE = M + ln sum_s exp(LSE_s - M),  O = sum_s exp(LSE_s - LSE) O_s,
// write O as bf16 (round to nearest even) and LSE as fp32.  NaN partials propagate; a row
// with no key gets O = 0, LSE = -inf.
// =============================================================================================
constexpr int kCombineThreads = 128;   // one (sequence, row) per workgroup, 4 dims per thread
constexpr int kCombineChunk = 512;     // split weights staged in LDS per pass

constexpr int kCombineFast = 24;       // rows with at most this many splits: one memory round trip
constexpr int kCombineFastNarrow = 64; // the same for 128-wide rows (one register per split)

template <int DV>
__global__ void __launch_bounds__(kCombineThreads) combine_kernel_t(FwdArgs a)
{
    constexpr int VW = DV / kCombineThreads;   // dims per thread: 4 (latent path) or 1
    static_assert(VW == 4 || VW == 1, "512 or 128 value dims");
    using VT = typename std::conditional<VW == 4, f32x4, float>::type;
    const WsLayout lay = ws_layout(a.batch, a.rows, a.capacity, DV);
    // the arguments used below come in with the first ones
    asm volatile("" ::"s"(a.ws), "s"(a.seqlens), "s"(a.out), "s"(a.lse), "s"(a.bt_stride));
    const int32_t* header = reinterpret_cast<const int32_t*>(a.ws + lay.header);
    const int gr = blockIdx.x;                 // global row = b * rows + r
    const int t = threadIdx.x;
    const int b = gr / a.rows;
    const int r = gr % a.rows;
    // header, lengths and this sequence's split range in one round trip (all lie inside the
    // workspace and seqlens whatever the header holds); the checks use no short-circuit
    const i32x4 h0 = reinterpret_cast<const i32x4*>(header)[0];
    const int h_cap = header[kHCapacity];
    const int L = a.seqlens[b];
    const int plan_L = reinterpret_cast<const int32_t*>(a.ws + lay.seqlens)[b];
    const int32_t* bs = reinterpret_cast<const int32_t*>(a.ws + lay.batch_split);
    const int bs0 = bs[b], bs1 = bs[b + 1];
    const bool shape_ok = (h0[kHMagic] == kPlanMagic) & (h0[kHBatch] == a.batch) & (h0[kHSq] == a.s_q) &
                          (h0[kHHeads] == a.heads) & (h_cap == a.capacity);
    const bool len_bad = (L != plan_L) | (L < 0) | ((long long)L > (long long)kPage * a.bt_stride);
    bool poison = !shape_ok | len_bad;
    const int s0 = shape_ok ? bs0 : 0;   // selects, not a branch: the loads above stay together
    const int s1 = shape_ok ? bs1 : 0;
    const int n = s1 - s0;
    const float* lse_part = reinterpret_cast<const float*>(a.ws + lay.lse_part);
    const float* o_part = reinterpret_cast<const float*>(a.ws + lay.o_part);
    const float* op = o_part + ((size_t)s0 * a.rows + r) * DV + VW * t;   // split s0, this thread's dims
    const size_t stride = (size_t)a.rows * DV;                           // between splits

    __shared__ float w[kCombineChunk];
    __shared__ float red_m[kCombineThreads / 64];
    __shared__ int red_nan[kCombineThreads / 64];

    // few splits: issue every partial-row load together with the LSE loads, before any wait
    constexpr int FAST = VW == 4 ? kCombineFast : kCombineFastNarrow;
    static_assert(FAST <= kCombineThreads, "one LSE per thread on the fast path");
    const bool fast = n <= FAST;
    VT ov[FAST];
    if (fast) {
#pragma unroll
        for (int i = 0; i < FAST; ++i)
            if (i < n) ov[i] = *reinterpret_cast<const VT*>(op + i * stride);
    }

    // M = max_s LSE_s (NaN anywhere poisons the row)
    float M = -__builtin_inff();
    int nan = 0;
    float my_lse = -__builtin_inff();   // fast path: thread t < n holds LSE of split s0 + t
    for (int s = s0 + t; s < s1; s += kCombineThreads) {
        const float v = lse_part[(size_t)s * a.rows + r];
        if (s == s0 + t) my_lse = v;
        nan |= (v != v);
        M = fmaxf(M, v);
    }
    for (int o = 32; o > 0; o >>= 1) {
        M = fmaxf(M, __shfl_xor(M, o));
        nan |= __shfl_xor(nan, o);
    }
    if ((t & 63) == 0) {
        red_m[t >> 6] = M;
        red_nan[t >> 6] = nan;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kCombineThreads / 64; ++i) {
        M = fmaxf(M, red_m[i]);
        nan |= red_nan[i];
    }
    poison |= (nan != 0);

    // weights exp(LSE_s - M) through LDS, then the weighted sum of the partial rows
    VT o{};
    float W = 0.f;
    if (fast) {
        if (t < n) w[t] = (poison || M == -__builtin_inff()) ? 0.f : expf(my_lse - M);
        __syncthreads();
        if (!poison && M != -__builtin_inff()) {
#pragma unroll
            for (int i = 0; i < FAST; ++i)
                if (i < n) {
                    o += w[i] * ov[i];
                    W += w[i];
                }
        }
    } else if (!poison && M != -__builtin_inff()) {
        for (int c0 = s0; c0 < s1; c0 += kCombineChunk) {
            const int nc = min(kCombineChunk, s1 - c0);
            __syncthreads();
            for (int i = t; i < nc; i += kCombineThreads) w[i] = expf(lse_part[(size_t)(c0 + i) * a.rows + r] - M);
            __syncthreads();
            const float* oc = op + (size_t)(c0 - s0) * stride;
            int i = 0;
            for (; i + 4 <= nc; i += 4) {
                const VT v0 = *reinterpret_cast<const VT*>(oc + (i + 0) * stride);
                const VT v1 = *reinterpret_cast<const VT*>(oc + (i + 1) * stride);
                const VT v2 = *reinterpret_cast<const VT*>(oc + (i + 2) * stride);
                const VT v3 = *reinterpret_cast<const VT*>(oc + (i + 3) * stride);
                o += w[i] * v0 + w[i + 1] * v1 + w[i + 2] * v2 + w[i + 3] * v3;
                W += (w[i] + w[i + 1]) + (w[i + 2] + w[i + 3]);
            }
            for (; i < nc; ++i) {
                o += w[i] * *reinterpret_cast<const VT*>(oc + i * stride);
                W += w[i];
            }
        }
    }
    float lse_out;
    if (poison) {
        o = VT{} + __builtin_nanf("");
        lse_out = __builtin_nanf("");
    } else if (M == -__builtin_inff()) {
        lse_out = -__builtin_inff();
    } else {
        o *= 1.f / W;
        lse_out = M + logf(W);
    }
    if constexpr (VW == 4) {
        ushort4 ob;
        ob.x = f32_to_bf16_rne(o[0]);
        ob.y = f32_to_bf16_rne(o[1]);
        ob.z = f32_to_bf16_rne(o[2]);
        ob.w = f32_to_bf16_rne(o[3]);
        *reinterpret_cast<ushort4*>(a.out + (size_t)gr * DV + 4 * t) = ob;
    } else {
        a.out[(size_t)gr * DV + t] = f32_to_bf16_rne(o);
    }
    if (t == 0) a.lse[gr] = lse_out;
}

}  // namespace mla
