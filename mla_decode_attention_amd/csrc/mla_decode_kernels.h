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

__host__ __device__ inline WsLayout ws_layout(int batch, int rows, int capacity)
{
    WsLayout w;
    size_t off = 0;
    w.header = off;      off = align256(off + 16 * sizeof(int32_t));
    w.seqlens = off;     off = align256(off + size_t(batch) * sizeof(int32_t));
    w.batch_split = off; off = align256(off + size_t(batch + 1) * sizeof(int32_t));
    w.items = off;       off = align256(off + size_t(capacity) * 4 * sizeof(int32_t));
    w.lse_part = off;    off = align256(off + size_t(capacity) * rows * sizeof(float));
    w.o_part = off;      off = align256(off + size_t(capacity) * rows * kDv * sizeof(float));
    w.total = off;
    return w;
}

enum HeaderField { kHMagic = 0, kHBatch, kHSq, kHHeads, kHItems, kHCapacity, kHRows };

// =============================================================================================
// Plan: balanced split of every sequence's pages into at most `gx + batch` work items.
// One workgroup; the chunk size is ceil(total pages / gx) so that about gx items (one per
// resident workgroup slot of the split kernel) carry equal page counts.
// =============================================================================================
constexpr int kPlanThreads = 1024;

__device__ inline int pages_of(int L) { return L <= 0 ? 0 : (L + kPage - 1) / kPage; }

__global__ void __launch_bounds__(kPlanThreads) plan_kernel(const int32_t* __restrict__ seqlens, int batch,
                                                            int s_q, int heads, int rows, int gx,
                                                            int capacity, char* __restrict__ ws)
{
    const WsLayout lay = ws_layout(batch, rows, capacity);
    int32_t* header = reinterpret_cast<int32_t*>(ws + lay.header);
    int32_t* ws_len = reinterpret_cast<int32_t*>(ws + lay.seqlens);
    int32_t* bsplit = reinterpret_cast<int32_t*>(ws + lay.batch_split);
    i32x4* items = reinterpret_cast<i32x4*>(ws + lay.items);

    __shared__ long long red[kPlanThreads / 64];
    __shared__ int scan_carry;
    __shared__ int wave_tot[kPlanThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;

    // total pages
    long long mine = 0;
    for (int b = tid; b < batch; b += kPlanThreads) {
        const int L = seqlens[b];
        ws_len[b] = L;
        mine += pages_of(L);
    }
    for (int o = 32; o > 0; o >>= 1) mine += __shfl_xor(mine, o);
    if (lane == 0) red[wid] = mine;
    if (tid == 0) scan_carry = 0;
    __syncthreads();
    long long total = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) total += red[w];
    long long chunk = (total + gx - 1) / (gx > 0 ? gx : 1);
    if (chunk < 1) chunk = 1;

    // per-sequence split counts, exclusive prefix sum in blocks of kPlanThreads
    for (int base = 0; base < batch; base += kPlanThreads) {
        const int b = base + tid;
        int n = 0, pg = 0;
        if (b < batch) {
            pg = pages_of(seqlens[b]);
            n = int((pg + chunk - 1) / chunk);
        }
        int incl = n;
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o);
            if (lane >= o) incl += t;
        }
        if (lane == 63) wave_tot[wid] = incl;
        __syncthreads();
        int before = scan_carry;
        for (int w = 0; w < wid; ++w) before += wave_tot[w];
        const int excl = before + incl - n;
        if (b < batch) {
            bsplit[b] = excl;
            for (int s = 0; s < n; ++s) {
                const int p0 = int((long long)s * pg / n), p1 = int((long long)(s + 1) * pg / n);
                items[excl + s] = i32x4{b, p0, p1, s};
            }
        }
        __syncthreads();
        if (tid == kPlanThreads - 1) scan_carry = excl + n;
        __syncthreads();
    }
    if (tid == 0) {
        bsplit[batch] = scan_carry;
        header[kHMagic] = kPlanMagic;
        header[kHBatch] = batch;
        header[kHSq] = s_q;
        header[kHHeads] = heads;
        header[kHItems] = scan_carry;
        header[kHCapacity] = capacity;
        header[kHRows] = rows;
    }
}

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
};

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
    __device__ inline int page(int idx, int lane)
    {
        if (base < 0 || idx < base || idx >= base + 64) {
            base = idx;
            val = (idx + lane < len) ? row[idx + lane] : -1;
        }
        return __builtin_amdgcn_readlane(val, idx - base);
    }
};

template <int B>
struct Idx {
    static constexpr int value = B;
};

template <class C>
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
    const int32_t* header = reinterpret_cast<const int32_t*>(a.ws + lay.header);
    if (header[kHMagic] != kPlanMagic || header[kHBatch] != a.batch || header[kHSq] != a.s_q ||
        header[kHHeads] != a.heads || header[kHCapacity] != a.capacity)
        return;  // the combine kernel reports the mismatch
    const int item = blockIdx.x;
    if (item >= header[kHItems]) return;
    const i32x4 it = reinterpret_cast<const i32x4*>(a.ws + lay.items)[item];
    const int b = it[0];
    const int L = a.seqlens[b];
    const int32_t plan_L = reinterpret_cast<const int32_t*>(a.ws + lay.seqlens)[b];
    float* lse_part = reinterpret_cast<float*>(a.ws + lay.lse_part) + (size_t)item * a.rows;
    float* o_part = reinterpret_cast<float*>(a.ws + lay.o_part) + (size_t)item * a.rows * kDv;

    const int rb = blockIdx.y * C::RB + rbl;          // global 16-row block
    const int row0 = rb * 16;
    const int qi = row0 / a.heads;                    // query token of this block (heads % 16 == 0)
    const bool bad_seq = (L != plan_L) || L < 0 || (long long)L > (long long)kPage * a.bt_stride;
    if (bad_seq) {
        if (tid < C::RB * 16) lse_part[blockIdx.y * C::RB * 16 + tid] = __builtin_nanf("");
        return;
    }
    const int n_vis = a.causal ? min(max(L - a.s_q + 1 + qi, 0), L) : L;
    const int tok_begin = it[1] * kPage;
    const int tok_end = min(it[2] * kPage, L);
    const int n_tiles = (tok_end - tok_begin + C::TT - 1) / C::TT;
    const int n_it = (n_tiles + C::NG - 1) / C::NG;

    // ---- Q^T operand (B of the score MFMA): lane (row lr, group lg) holds q[row][32j+8lg .. +8]
    bf16x8 qop[kKSteps];
    {
        const int row = row0 + lr;
        const uint16_t* qrow = a.q + ((size_t)(b * a.s_q + row / a.heads) * a.heads + row % a.heads) * kDk;
#pragma unroll
        for (int j = 0; j < kKSteps; ++j)
            qop[j] = *reinterpret_cast<const bf16x8*>(qrow + 32 * j + 8 * lg);
        // Consume Q here so the compiler's vmcnt waits for these loads land before the tile
        // loop, not inside it (where they would also wait for the tile loads in flight).
#pragma unroll
        for (int j = 0; j < kKSteps; ++j) asm volatile("" ::"v"(qop[j]));
    }

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
    PageWindow pw;
    pw.init(a.block_table + (size_t)b * a.bt_stride, a.bt_stride);
    bool bad_page = false;

    i32x4 rbuf[C::NR][C::NPW];
    auto load_tile = [&](int itn, auto buf_idx) {
        constexpr int B = decltype(buf_idx)::value;
        const int k = itn * C::NG + gi;
        if (itn >= n_it || k >= n_tiles) return;
        const int t0 = tok_begin + k * C::TT;
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
        // k-steps ahead
        constexpr int KD = C::NST == 1 ? 6 : 3;
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
        if (t0 + C::TT > n_vis) {
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
        store_tile(itn + 1, next_buf);
        load_tile(itn + 1 + C::NR, next_buf);
        if constexpr (C::GW > 1) __syncthreads();
    };
    load_tile(0, Idx<0>{});
    if constexpr (C::NR == 2) load_tile(1, Idx<1>{});
    store_tile(0, Idx<0>{});
    load_tile(C::NR, Idx<0>{});
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
            *reinterpret_cast<f32x4*>(orow + 16 * dt + 4 * lg) = acc[dt] * inv;
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
            *reinterpret_cast<f32x4*>(o_part + (size_t)grow * kDv + seg * SEG + 4 * d4) = o * inv;
            if (d4 == 0 && seg == 0)
                lse_part[grow] = nan ? __builtin_nanf("")
                                     : (Lsum > 0.f ? (M + __builtin_amdgcn_logf(Lsum)) * kLn2 : -__builtin_inff());
        }
    }
}

// =============================================================================================
// Split kernel, wide form (128 or 256 query rows per sequence: all heads on one GPU).
//
// A work item is taken by `row_groups` workgroups of 64 query rows each.  Their ids are 8 apart
// (id = 8 * row_group + item % 8 within a block of 8 * row_groups ids), so with round-robin
// dispatch over the 8 XCDs they run together on one XCD and the second read of every KV tile
// is served by that XCD's L2.
//
// Inside a workgroup the four waves split the two contractions differently (the pages' split
// of the output into segments computed by different warp groups, here by waves):
//   score:  wave w owns query rows 16w..16w+15 of the group (Q^T in registers), computes
//           S^T = K Q^T for them, keeps their online-softmax statistics and writes P^T (bf16)
//           to LDS;
//   value:  wave w owns value dims 128w..128w+127 for all 64 rows, O^T += V^T P^T, reading the
//           V^T operand once per 16 dims and reusing it across the four 16-row blocks.
// One barrier per 32-token tile separates the two; P^T is double-buffered.  Tiles stream
// HBM -> VGPR -> LDS as in the row-block form (three stages, two tiles in flight per wave).
// =============================================================================================
template <int NR_>
struct WideCfg {
    static constexpr int NW = 4;              // waves per workgroup (one per SIMD)
    static constexpr int RW = 64;             // query rows per workgroup
    static constexpr int TT = 32;             // tokens per tile
    static constexpr int NS = 3;              // LDS stages
    static constexpr int NR = NR_;            // tiles in flight in registers per wave
    static constexpr int SEG = kDv / NW;      // value dims per wave
    static constexpr int DTW = SEG / 16;      // 16-dim output tiles per wave
    static constexpr int LDS_TILE = TT * kLdsRow;
    static constexpr int UNITS = TT * kRowBytes / 1024;     // 1-KiB load units per tile
    static constexpr int NPW = UNITS / NW;                  // per wave
    static constexpr int P_BYTES = RW * TT * 2;             // bf16 P^T of one tile
    static constexpr int OFF_P = NS * LDS_TILE;
    static constexpr int OFF_ALPHA = OFF_P + 2 * P_BYTES;   // fp32 [2][RW] rescale factors
    static constexpr int OFF_FLAG = OFF_ALPHA + 2 * RW * 4; // int [2][NW] rescale flags
    static constexpr int OFF_ML = OFF_FLAG + 2 * NW * 4;    // fp32 [2][RW] final m, l
    static constexpr int LDS_BYTES = OFF_ML + 2 * RW * 4;
    static constexpr int THREADS = NW * 64;
    static_assert(NPW * NW == UNITS && NPW % 9 == 0, "each wave loads whole 8-row groups");
    static_assert(NR == 1 || NR == 2, "one or two tiles in flight per wave");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

template <class C>
__global__ void __launch_bounds__(C::THREADS) split_wide_kernel(FwdArgs a)
{
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15;
    const int lg = lane >> 4;

    const int G = a.row_groups;
    const int x = blockIdx.x;
    const int item = (x / (8 * G)) * 8 + x % 8;
    const int rg = (x / 8) % G;

    const WsLayout lay = ws_layout(a.batch, a.rows, a.capacity);
    const int32_t* header = reinterpret_cast<const int32_t*>(a.ws + lay.header);
    if (header[kHMagic] != kPlanMagic || header[kHBatch] != a.batch || header[kHSq] != a.s_q ||
        header[kHHeads] != a.heads || header[kHCapacity] != a.capacity)
        return;  // the combine kernel reports the mismatch
    if (item >= header[kHItems]) return;
    const i32x4 it = reinterpret_cast<const i32x4*>(a.ws + lay.items)[item];
    const int b = it[0];
    const int L = a.seqlens[b];
    const int32_t plan_L = reinterpret_cast<const int32_t*>(a.ws + lay.seqlens)[b];
    float* lse_part = reinterpret_cast<float*>(a.ws + lay.lse_part) + (size_t)item * a.rows;
    float* o_part = reinterpret_cast<float*>(a.ws + lay.o_part) + (size_t)item * a.rows * kDv;

    const int row_base = rg * C::RW;                  // first row of this group
    const int srow = row_base + 16 * wave + lr;       // this lane's score row
    const int qi = row_base / a.heads;                // the group's query token (heads % 64 == 0)
    const bool bad_seq = (L != plan_L) || L < 0 || (long long)L > (long long)kPage * a.bt_stride;
    if (bad_seq) {
        if (tid < C::RW) lse_part[row_base + tid] = __builtin_nanf("");
        return;
    }
    const int n_vis = a.causal ? min(max(L - a.s_q + 1 + qi, 0), L) : L;
    const int tok_begin = it[1] * kPage;
    const int tok_end = min(it[2] * kPage, L);
    const int n_tiles = (tok_end - tok_begin + C::TT - 1) / C::TT;

    bf16x8 qop[kKSteps];
    {
        const uint16_t* qrow = a.q + ((size_t)(b * a.s_q + srow / a.heads) * a.heads + srow % a.heads) * kDk;
#pragma unroll
        for (int j = 0; j < kKSteps; ++j)
            qop[j] = *reinterpret_cast<const bf16x8*>(qrow + 32 * j + 8 * lg);
#pragma unroll
        for (int j = 0; j < kKSteps; ++j) asm volatile("" ::"v"(qop[j]));
    }

    const uint32_t lane16 = (uint32_t)lane * 16u;
    int st9[9];
#pragma unroll
    for (int v = 0; v < 9; ++v) {
        const int r0 = (64 * v) / kChunksPerRow;
        const int bnd = kChunksPerRow * (r0 + 1) - 64 * v;
        st9[v] = v * 1024 + (kLdsRow - kRowBytes) * (r0 + (lane >= bnd ? 1 : 0)) + (int)lane16;
    }
    const int unit0 = wave * C::NPW;
    PageWindow pw;
    pw.init(a.block_table + (size_t)b * a.bt_stride, a.bt_stride);
    bool bad_page = false;

    i32x4 rbuf[C::NR][C::NPW];
    auto load_tile = [&](int t, auto buf_idx) {
        constexpr int B = decltype(buf_idx)::value;
        if (t >= n_tiles) return;
        const int t0 = tok_begin + t * C::TT;
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
    auto store_tile = [&](int t, auto buf_idx) {
        constexpr int B = decltype(buf_idx)::value;
        if (t >= n_tiles) return;
        char* stg = smem + (t % C::NS) * C::LDS_TILE + (unit0 / 9) * (8 * kLdsRow);
#pragma unroll
        for (int kk = 0; kk < C::NPW; ++kk)
            *reinterpret_cast<i32x4*>(stg + st9[kk % 9] + (kk / 9) * (8 * kLdsRow)) = rbuf[B][kk];
    };

    // score side: statistics of row srow (lane-partial l)
    float m_run = -__builtin_inff();
    float l_run = 0.f;
    constexpr float kLazyRescale = 8.f;
    // value side: acc[dt][rb] holds O^T[SEG w + 16 dt + 4 lg + i][row_base + 16 rb + lr]
    f32x4 acc[C::DTW][4];
#pragma unroll
    for (int dt = 0; dt < C::DTW; ++dt)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) acc[dt][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int kbase = lr * kLdsRow + 16 * lg;
    const int vbase = (4 * lg + (lr >> 2)) * kLdsRow + 8 * (lr & 3) + 32 * (wave * C::DTW);
    char* const pbuf0 = smem + C::OFF_P;
    float* const alpha_s = reinterpret_cast<float*>(smem + C::OFF_ALPHA);
    int* const flag_s = reinterpret_cast<int*>(smem + C::OFF_FLAG);
    auto kread = [&](const char* p) { return *reinterpret_cast<const bf16x8*>(p); };
    auto vread = [&](const char* p) {
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)lds_i16x4(p));
    };

    // score(t): S^T for the wave's 16 rows over tile t; softmax(t): online softmax and P^T (bf16)
    // to LDS.  P^T slot 8 lg + i of row r holds token 4 lg + i (i < 4) or 16 + 4 lg + (i - 4):
    // the lane's own accumulator values, so each lane writes one 16-B chunk.
    // value(t): O^T[dims of this wave][64 rows] += V^T P^T over tile t.
    // Score and value MFMAs of consecutive tiles are independent, so after each barrier the wave
    // runs score(t) interleaved with value(t - 1): one stream's LDS reads are in flight while the
    // other's MFMAs issue.
    constexpr int KD = 3;   // K-operand look-ahead (k-steps of two MFMAs)
    constexpr int VD = 2;   // V-operand look-ahead (16-dim tiles of four MFMAs)
    f32x4 s[2];
    auto softmax = [&](int t) {
        const int t0 = tok_begin + t * C::TT;
#pragma unroll
        for (int st = 0; st < 2; ++st) s[st] *= a.scale_log2;
        if (t0 + C::TT > n_vis) {
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (t0 + 16 * st + 4 * lg + i >= n_vis) s[st][i] = -__builtin_inff();
        }
        float tmax = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                           fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
        tmax = wave_max_groups(tmax);
        const int par = t & 1;
        int rescaled = 0;
        if (__builtin_amdgcn_ballot_w64(tmax > m_run + kLazyRescale) != 0) {
            const float m_new = fmaxf(m_run, tmax);
            const float alpha = (m_new == -__builtin_inff()) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
            if (lg == 0) alpha_s[par * C::RW + 16 * wave + lr] = alpha;
            rescaled = 1;
        }
        if (lane == 0) flag_s[par * C::NW + wave] = rescaled;
        const float m_use = (m_run == -__builtin_inff()) ? 0.f : m_run;
        float psum = 0.f;
        bf16x8 pk;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pv = __builtin_amdgcn_exp2f(s[st][i] - m_use);
                psum += pv;
                pk[4 * st + i] = (__bf16)pv;
            }
        l_run += psum;
        *reinterpret_cast<bf16x8*>(pbuf0 + par * C::P_BYTES + (16 * wave + lr) * (C::TT * 2) + 16 * lg) = pk;
    };
    // rows of a block that took a new max in tile t: rescale their accumulators
    auto rescale_acc = [&](int t) {
        const int par = t & 1;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            if (flag_s[par * C::NW + rb] != 0) {
                const float al = alpha_s[par * C::RW + 16 * rb + lr];
#pragma unroll
                for (int dt = 0; dt < C::DTW; ++dt) {
                    acc[dt][rb] *= al;
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };
    // DO_S: run score(ts); DO_V: run value(tv); both: interleaved
    auto fused = [&](int ts, int tv, auto do_s, auto do_v) {
        constexpr bool DO_S = decltype(do_s)::value != 0;
        constexpr bool DO_V = decltype(do_v)::value != 0;
        const char* sst = smem + (ts % C::NS) * C::LDS_TILE;
        const char* vst = smem + (tv % C::NS) * C::LDS_TILE;
        bf16x8 kop[KD + 1][2];
        bf16x8 pop[4];
        i16x4 vlo[VD + 1], vhi[VD + 1];
        if constexpr (DO_V) rescale_acc(tv);
        // two 16-token blocks x two k-parities = four independent score chains (a dependent
        // MFMA chain issues only every ~50 cycles)
        f32x4 sp[2][2];
        if constexpr (DO_S) {
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                sp[st][0] = f32x4{0.f, 0.f, 0.f, 0.f};
                sp[st][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < KD; ++j) kop[j][st] = kread(sst + st * 16 * kLdsRow + kbase + 64 * j);
            }
        }
        const char* vt0 = vst + vbase;
        if constexpr (DO_V) {
            const char* pb = pbuf0 + (tv & 1) * C::P_BYTES;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) pop[rb] = kread(pb + (16 * rb + lr) * (C::TT * 2) + 16 * lg);
#pragma unroll
            for (int d = 0; d < VD; ++d) {
                vlo[d] = vread(vt0 + 32 * d);
                vhi[d] = vread(vt0 + 16 * kLdsRow + 32 * d);
            }
        }
        // 18 score steps (2 MFMAs each) with the 8 value tiles (4 MFMAs each) slotted in after
        // odd steps
#pragma unroll
        for (int j = 0; j < kKSteps; ++j) {
            if constexpr (DO_S) {
                if (j + KD < kKSteps) {
#pragma unroll
                    for (int st = 0; st < 2; ++st)
                        kop[(j + KD) % (KD + 1)][st] = kread(sst + st * 16 * kLdsRow + kbase + 64 * (j + KD));
                }
#pragma unroll
                for (int st = 0; st < 2; ++st)
                    sp[st][j & 1] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[j % (KD + 1)][st], qop[j], sp[st][j & 1], 0, 0, 0);
            }
            if constexpr (DO_V) {
                if ((j & 1) && (j >> 1) < C::DTW) {
                    const int dt = j >> 1;
                    if (dt + VD < C::DTW) {
                        vlo[(dt + VD) % (VD + 1)] = vread(vt0 + 32 * (dt + VD));
                        vhi[(dt + VD) % (VD + 1)] = vread(vt0 + 16 * kLdsRow + 32 * (dt + VD));
                    }
                    const bf16x8 vop = __builtin_shufflevector(__builtin_bit_cast(bf16x4, vlo[dt % (VD + 1)]),
                                                               __builtin_bit_cast(bf16x4, vhi[dt % (VD + 1)]),
                                                               0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                    for (int rb = 0; rb < 4; ++rb)
                        acc[dt][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[rb], acc[dt][rb], 0, 0, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (DO_S) {
#pragma unroll
            for (int st = 0; st < 2; ++st) s[st] = sp[st][0] + sp[st][1];
        }
    };

    // ---- pipeline.  At the top of iteration t, stages t%3 and (t+1)%3 hold tiles t and t+1
    // and the registers hold tiles t+2 (buffer t&1) and t+3.  Iteration t scores tile t and
    // finishes the value contraction of tile t-1 (P^T(t-1) became visible at the previous
    // barrier), then publishes P^T(t) at its barrier, after which the stage of tile t-1 is free
    // and receives tile t+2 (visible at the next barrier, two iterations before it is scored).
    auto step = [&](int t, auto buf) {
        if (t >= n_tiles) return;
        if (t == 0)
            fused(t, t, Idx<1>{}, Idx<0>{});
        else
            fused(t, t - 1, Idx<1>{}, Idx<1>{});
        softmax(t);
        __syncthreads();
        store_tile(t + 2, buf);
        load_tile(t + 2 + C::NR, buf);
    };
    load_tile(0, Idx<0>{});
    if constexpr (C::NR == 2) {
        load_tile(1, Idx<1>{});
        store_tile(0, Idx<0>{});
        load_tile(2, Idx<0>{});
        store_tile(1, Idx<1>{});
        load_tile(3, Idx<1>{});
    } else {
        store_tile(0, Idx<0>{});
        load_tile(1, Idx<0>{});
        store_tile(1, Idx<0>{});
        load_tile(2, Idx<0>{});
    }
    __syncthreads();
    if constexpr (C::NR == 2) {
        for (int t = 0; t < n_tiles; t += 2) {
            step(t, Idx<0>{});
            step(t + 1, Idx<1>{});
        }
    } else {
        for (int t = 0; t < n_tiles; ++t) step(t, Idx<0>{});
    }
    if (n_tiles > 0) fused(n_tiles - 1, n_tiles - 1, Idx<0>{}, Idx<1>{});   // value of the last tile
    l_run = wave_sum_groups(l_run);

    // ---- epilogue: share final (m, l) of every row, normalise and write the item's partials
    float* ml_s = reinterpret_cast<float*>(smem + C::OFF_ML);
    if (lg == 0) {
        ml_s[16 * wave + lr] = m_run;
        ml_s[C::RW + 16 * wave + lr] = l_run;
        lse_part[srow] = bad_page ? __builtin_nanf("")
                                  : (l_run > 0.f ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2
                                                 : -__builtin_inff());
    }
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        const float l = ml_s[C::RW + 16 * rb + lr];
        const float inv = (l > 0.f) ? 1.f / l : 0.f;
        float* orow = o_part + (size_t)(row_base + 16 * rb + lr) * kDv + C::SEG * wave;
#pragma unroll
        for (int dt = 0; dt < C::DTW; ++dt)
            *reinterpret_cast<f32x4*>(orow + 16 * dt + 4 * lg) = acc[dt][rb] * inv;
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

__global__ void __launch_bounds__(kCombineThreads) combine_kernel(FwdArgs a)
{
    const WsLayout lay = ws_layout(a.batch, a.rows, a.capacity);
    const int32_t* header = reinterpret_cast<const int32_t*>(a.ws + lay.header);
    const int gr = blockIdx.x;                 // global row = b * rows + r
    const int t = threadIdx.x;
    const int b = gr / a.rows;
    const int r = gr % a.rows;
    const bool shape_ok = header[kHMagic] == kPlanMagic && header[kHBatch] == a.batch &&
                          header[kHSq] == a.s_q && header[kHHeads] == a.heads &&
                          header[kHCapacity] == a.capacity;
    bool poison = !shape_ok;
    int s0 = 0, s1 = 0;
    if (shape_ok) {
        const int L = a.seqlens[b];
        const int plan_L = reinterpret_cast<const int32_t*>(a.ws + lay.seqlens)[b];
        poison = (L != plan_L) || L < 0 || (long long)L > (long long)kPage * a.bt_stride;
        const int32_t* bs = reinterpret_cast<const int32_t*>(a.ws + lay.batch_split);
        s0 = bs[b];
        s1 = bs[b + 1];
    }
    const float* lse_part = reinterpret_cast<const float*>(a.ws + lay.lse_part);
    const float* o_part = reinterpret_cast<const float*>(a.ws + lay.o_part);

    __shared__ float w[kCombineChunk];
    __shared__ float red_m[kCombineThreads / 64];
    __shared__ int red_nan[kCombineThreads / 64];

    // pass 1: M = max_s LSE_s (NaN anywhere poisons the row)
    float M = -__builtin_inff();
    int nan = 0;
    for (int s = s0 + t; s < s1; s += kCombineThreads) {
        const float v = lse_part[(size_t)s * a.rows + r];
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

    // pass 2: weights exp(LSE_s - M) through LDS, then the weighted sum of the partial rows
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    float W = 0.f;
    if (!poison && M != -__builtin_inff()) {
        for (int c0 = s0; c0 < s1; c0 += kCombineChunk) {
            const int n = min(kCombineChunk, s1 - c0);
            __syncthreads();
            for (int i = t; i < n; i += kCombineThreads) w[i] = expf(lse_part[(size_t)(c0 + i) * a.rows + r] - M);
            __syncthreads();
            const float* op = o_part + ((size_t)c0 * a.rows + r) * kDv + 4 * t;
            const size_t stride = (size_t)a.rows * kDv;
            int i = 0;
            for (; i + 4 <= n; i += 4) {
                const f32x4 v0 = *reinterpret_cast<const f32x4*>(op + (i + 0) * stride);
                const f32x4 v1 = *reinterpret_cast<const f32x4*>(op + (i + 1) * stride);
                const f32x4 v2 = *reinterpret_cast<const f32x4*>(op + (i + 2) * stride);
                const f32x4 v3 = *reinterpret_cast<const f32x4*>(op + (i + 3) * stride);
                o += w[i] * v0 + w[i + 1] * v1 + w[i + 2] * v2 + w[i + 3] * v3;
                W += (w[i] + w[i + 1]) + (w[i + 2] + w[i + 3]);
            }
            for (; i < n; ++i) {
                o += w[i] * *reinterpret_cast<const f32x4*>(op + i * stride);
                W += w[i];
            }
        }
    }
    float lse_out;
    if (poison) {
        const float qnan = __builtin_nanf("");
        o = f32x4{qnan, qnan, qnan, qnan};
        lse_out = qnan;
    } else if (M == -__builtin_inff()) {
        lse_out = -__builtin_inff();
    } else {
        o *= 1.f / W;
        lse_out = M + logf(W);
    }
    ushort4 ob;
    ob.x = f32_to_bf16_rne(o[0]);
    ob.y = f32_to_bf16_rne(o[1]);
    ob.z = f32_to_bf16_rne(o[2]);
    ob.w = f32_to_bf16_rne(o[3]);
    *reinterpret_cast<ushort4*>(a.out + (size_t)gr * kDv + 4 * t) = ob;
    if (t == 0) a.lse[gr] = lse_out;
}

}  // namespace mla
