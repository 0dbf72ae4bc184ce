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
constexpr int kKSteps = kDk / 32;           // 18 score MFMA k-steps of 32
constexpr int kDTiles = kDv / 16;           // 32 output tiles of 16 dims
constexpr int kPlanMagic = 0x4D4C4131;      // "MLA1"
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

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
// group streams its own share of the item's TT-token tiles (round robin) through NSG LDS
// stages, the RB waves of a group sharing each stage, one 16-row block per wave.
//
// Tiles move HBM -> LDS with buffer_load_dwordx4 ... lds (16 B per lane, no VGPR staging),
// issued from inline asm so that the compiler does not put a vmcnt(0) before every LDS read;
// the waits are explicit vmcnt counts.  The buffer resource of a tile ends at the sequence's
// last valid row, so rows past L_b load as zeros and never reach the value contraction.
//
// LDS tile layout: rows of 1152 B; within each row the 16-B chunk c is stored at chunk
// c ^ (row & 7) (a permutation inside aligned 128-B groups), which spreads the 16 rows that a
// K-operand read touches over distinct bank groups.  The swizzle is applied by choosing which
// global chunk each lane loads, so every DMA still reads a contiguous 1 KiB of HBM.
// =============================================================================================
template <int NW_, int RB_, int TT_, int NSG_>
struct SplitCfg {
    static constexpr int NW = NW_;            // waves per workgroup
    static constexpr int RB = RB_;            // 16-row blocks per wave group (= waves per group)
    static constexpr int NG = NW / RB;        // wave groups
    static constexpr int TT = TT_;            // tokens per tile (16 or 32)
    static constexpr int NSG = NSG_;          // LDS stages per group
    static constexpr int NST = TT / 16;       // 16-token sub-tiles per tile
    static constexpr int TILE_BYTES = TT * kRowBytes;
    static constexpr int UNITS = TILE_BYTES / 1024;          // 1-KiB DMA units per tile
    static constexpr int NPW = (UNITS + RB - 1) / RB;        // DMA instructions per wave per tile
    static constexpr int STAGE_BYTES = TILE_BYTES;
    static constexpr int DUMMY_OFF = NG * NSG * STAGE_BYTES; // 1 KiB sink for padding DMAs
    static constexpr int LDS_BYTES = DUMMY_OFF + ((UNITS % RB) ? 1024 : 0);
    static constexpr int THREADS = NW * 64;
    static_assert(NW % RB == 0, "waves must split into whole groups");
    static_assert(TT == 16 || TT == 32, "tile is one or two MFMA token blocks");
    static_assert(TILE_BYTES % 1024 == 0, "tile must be whole DMA units");
    static_assert(NSG >= 2 && NSG <= 4, "2..4 stages");
    static_assert((NSG - 2) * NPW < 64, "outstanding DMAs must fit the vmcnt field");
    // merge scratch (reuses the stage area): m, l per wave + fp32 accumulators
    static constexpr int MERGE_BYTES = NW * (2 * 16 * 4 + 16 * kDv * 4);
    static_assert(NG == 1 || MERGE_BYTES <= LDS_BYTES, "merge scratch must fit");
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
};

#define MLA_VMCNT_CASE(n) \
    case n: asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory"); break;
// Wait until at most n of this wave's vector-memory operations are outstanding.  n is
// wave-uniform; s_waitcnt needs an immediate, hence the switch (values above 39 wait for all).
__device__ inline void wait_vmcnt_le(int n)
{
    switch (n) {
        MLA_VMCNT_CASE(1) MLA_VMCNT_CASE(2) MLA_VMCNT_CASE(3) MLA_VMCNT_CASE(4) MLA_VMCNT_CASE(5)
        MLA_VMCNT_CASE(6) MLA_VMCNT_CASE(7) MLA_VMCNT_CASE(8) MLA_VMCNT_CASE(9) MLA_VMCNT_CASE(10)
        MLA_VMCNT_CASE(11) MLA_VMCNT_CASE(12) MLA_VMCNT_CASE(13) MLA_VMCNT_CASE(14) MLA_VMCNT_CASE(15)
        MLA_VMCNT_CASE(16) MLA_VMCNT_CASE(17) MLA_VMCNT_CASE(18) MLA_VMCNT_CASE(19) MLA_VMCNT_CASE(20)
        MLA_VMCNT_CASE(21) MLA_VMCNT_CASE(22) MLA_VMCNT_CASE(23) MLA_VMCNT_CASE(24) MLA_VMCNT_CASE(25)
        MLA_VMCNT_CASE(26) MLA_VMCNT_CASE(27) MLA_VMCNT_CASE(28) MLA_VMCNT_CASE(29) MLA_VMCNT_CASE(30)
        MLA_VMCNT_CASE(31) MLA_VMCNT_CASE(32) MLA_VMCNT_CASE(33) MLA_VMCNT_CASE(34) MLA_VMCNT_CASE(35)
        MLA_VMCNT_CASE(36) MLA_VMCNT_CASE(37) MLA_VMCNT_CASE(38) MLA_VMCNT_CASE(39)
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
}
#undef MLA_VMCNT_CASE

// One 16-B-per-lane DMA from a buffer resource into LDS at m0 + 16*lane.
__device__ inline void dma16(i32x4 rsrc, uint32_t voff, uint32_t lds_addr)
{
    asm volatile(
        "s_waitcnt lgkmcnt(0)\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, 0 offen lds"
        :
        : "v"(voff), "s"(rsrc), "s"(lds_addr)
        : "memory");
}

__device__ inline uint32_t lds_u32(const void* p)
{
    return (uint32_t)(uintptr_t)(const MLA_LDS char*)p;
}

__device__ inline const MLA_LDS i16x4* lds_i16x4(const void* p)
{
    return (const MLA_LDS i16x4*)(const MLA_LDS char*)p;
}

__device__ inline float wave_max_groups(float v)
{
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

__device__ inline float wave_sum_groups(float v)
{
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

__device__ inline uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <class C>
__global__ void __launch_bounds__(C::THREADS) split_kernel(FwdArgs a)
{
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int gi = wave / C::RB;            // wave group
    const int rbl = wave % C::RB;           // row block within the group
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
        // Consume Q here so the compiler's own vmcnt waits for these loads land before the
        // tile loop, not inside it (where they would also wait for the in-flight tile DMAs).
#pragma unroll
        for (int j = 0; j < kKSteps; ++j) asm volatile("" ::"v"(qop[j]));
    }

    // ---- per-lane DMA offsets (constant across tiles) and LDS destinations
    uint32_t voff[C::NPW];
    uint32_t ldsu[C::NPW];   // unit offset inside a stage, or the dummy sink
#pragma unroll
    for (int k = 0; k < C::NPW; ++k) {
        const int u = rbl + C::RB * k;
        if (u < C::UNITS) {
            const int P = u * 64 + lane;
            const int r = P / kChunksPerRow, pc = P % kChunksPerRow;
            const int c = pc ^ (r & 7);
            voff[k] = (uint32_t)(r * kRowBytes + c * 16);
            ldsu[k] = (uint32_t)(u * 1024);
        } else {
            voff[k] = 0x7FFFFFF0u;   // beyond any num_records: loads zeros, touches no memory
            ldsu[k] = 0xFFFFFFFFu;
        }
    }
    char* const group_stages = smem + gi * C::NSG * C::STAGE_BYTES;
    const uint32_t stage0_lds = lds_u32(group_stages);
    const uint32_t dummy_lds = lds_u32(smem + C::DUMMY_OFF);
    // Block-table reads go through the constant address space so that the (wave-uniform) loads
    // become scalar loads counted by lgkmcnt; a vector load here would make the compiler wait
    // for vmcnt(0), i.e. for every tile DMA in flight.
    const __attribute__((address_space(4))) int32_t* bt_row =
        (const __attribute__((address_space(4))) int32_t*)(a.block_table + (size_t)b * a.bt_stride);
    bool bad_page = false;

    auto issue_tile = [&](int itn) {
        const int k = itn * C::NG + gi;
        if (itn >= n_it || k >= n_tiles) return;
        const int t0 = tok_begin + k * C::TT;
        const int page = bt_row[t0 / kPage];
        int valid = min(C::TT, L - t0);
        if (page < 0 || (long long)page >= a.num_pages) {
            bad_page = true;
            valid = 0;
        }
        const uint64_t base = (uint64_t)(a.cache + ((long long)(valid ? page : 0) * kPage + (t0 % kPage)) * kDk);
        i32x4 rs;
        rs[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)base);
        rs[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32));
        rs[2] = __builtin_amdgcn_readfirstlane(valid * kRowBytes);
        rs[3] = 0x00020000;
        const uint32_t sbase = stage0_lds + (uint32_t)((itn % C::NSG) * C::STAGE_BYTES);
#pragma unroll
        for (int u = 0; u < C::NPW; ++u) {
            const uint32_t dst = (ldsu[u] == 0xFFFFFFFFu) ? dummy_lds : sbase + ldsu[u];
            dma16(rs, voff[u], __builtin_amdgcn_readfirstlane(dst));
        }
    };
    // tiles of this group still in flight after tile `itn` (each is NPW DMAs of this wave)
    auto pending_after = [&](int itn) {
        const int last_issued = min(itn + C::NSG - 2, n_it - 1);
        int n = 0;
        for (int t = itn + 1; t <= last_issued; ++t)
            if (t * C::NG + gi < n_tiles) ++n;
        return n * C::NPW;
    };

    // ---- online softmax state: row lr; acc holds O^T[16 dt + 4 lg + i][row lr]
    f32x4 acc[kDTiles];
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -__builtin_inff();
    float l_run = 0.f;   // lane-partial sum over this lane's tokens

    // K-operand LDS addresses: row = 16 st + lr, chunk (4j + lg) ^ (row & 7)
    const int ksw = lr & 7;   // (16 st + lr) & 7 == lr & 7
    const int kb_even = lr * kRowBytes + 16 * (lg ^ (ksw & 3)) + 64 * (ksw >> 2);
    const int kb_odd = lr * kRowBytes + 16 * (lg ^ (ksw & 3)) - 64 * (ksw >> 2);
    // V^T tr-read addresses: lane (group lg, i = lr) reads row t = 4 lg + (lr >> 2) (+16 st),
    // dims 16 dt + 4 (lr & 3) .. +3, i.e. chunk 2 dt + ((lr & 3) >> 1), byte 8 ((lr & 3) & 1)
    const int vt = 4 * lg + (lr >> 2);
    const int vsw = vt & 7;
    const int vq = lr & 3;
    int vbase[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
        vbase[m] = vt * kRowBytes + 16 * ((vq >> 1) ^ (vsw & 1)) + 8 * (vq & 1) + 32 * ((m ^ (vsw >> 1)) - m);

    // ---- prologue
#pragma unroll
    for (int s = 0; s < C::NSG - 1; ++s) issue_tile(s);

    for (int itn = 0; itn < n_it; ++itn) {
        wait_vmcnt_le(pending_after(itn));
        if constexpr (C::RB > 1) __syncthreads();
        issue_tile(itn + C::NSG - 1);
        const int k = itn * C::NG + gi;
        if (k >= n_tiles) continue;
        const int t0 = tok_begin + k * C::TT;
        const char* stg = group_stages + (itn % C::NSG) * C::STAGE_BYTES;

        // scores S^T[token][row] for each 16-token sub-tile
        f32x4 s[C::NST];
#pragma unroll
        for (int st = 0; st < C::NST; ++st) {
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
            const char* kb = stg + st * 16 * kRowBytes;
#pragma unroll
            for (int j = 0; j < kKSteps; ++j) {
                const bf16x8 kop = *reinterpret_cast<const bf16x8*>(kb + ((j & 1) ? kb_odd : kb_even) + 64 * j);
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[j], c, 0, 0, 0);
            }
            s[st] = c;
        }
        // scale into the log2 domain, mask invisible tokens, tile max per row
        float tmax = -__builtin_inff();
#pragma unroll
        for (int st = 0; st < C::NST; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = t0 + 16 * st + 4 * lg + i;
                const float v = (tok < n_vis) ? s[st][i] * a.scale_log2 : -__builtin_inff();
                s[st][i] = v;
                tmax = fmaxf(tmax, v);
            }
        tmax = wave_max_groups(tmax);
        const float m_new = fmaxf(m_run, tmax);
        const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
        float psum = 0.f;
        float p[C::NST][4];
#pragma unroll
        for (int st = 0; st < C::NST; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[st][i] = __builtin_amdgcn_exp2f(s[st][i] - m_use);
                psum += p[st][i];
            }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int dt = 0; dt < kDTiles; ++dt) acc[dt] *= alpha;

        if constexpr (C::TT == 32) {
            bf16x8 pop;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pop[i] = (__bf16)p[0][i];
                pop[4 + i] = (__bf16)p[1][i];
            }
#pragma unroll
            for (int dt = 0; dt < kDTiles; ++dt) {
                const char* v0 = stg + vbase[dt & 3] + 32 * dt;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)lds_i16x4(v0));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (MLA_LDS i16x4*)lds_i16x4(v0 + 16 * kRowBytes));
                bf16x8 vop;
                vop = __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi),
                                              0, 1, 2, 3, 4, 5, 6, 7);
                acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop, acc[dt], 0, 0, 0);
            }
        } else {
            bf16x4 pop;
#pragma unroll
            for (int i = 0; i < 4; ++i) pop[i] = (__bf16)p[0][i];
#pragma unroll
            for (int dt = 0; dt < kDTiles; ++dt) {
                const char* v0 = stg + vbase[dt & 3] + 32 * dt;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)lds_i16x4(v0));
                acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, lo), pop, acc[dt],
                                                                   0, 0, 0);
            }
        }
    }
    wait_vmcnt_le(0);
    l_run = wave_sum_groups(l_run);

    // ---- epilogue: merge the NG wave groups of each row block, write the item's partials
    const int out_row = row0 + lr;   // row within the sequence (of a.rows)
    if constexpr (C::NG == 1) {
        const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
        float* orow = o_part + (size_t)out_row * kDv;
#pragma unroll
        for (int dt = 0; dt < kDTiles; ++dt)
            *reinterpret_cast<f32x4*>(orow + 16 * dt + 4 * lg) = acc[dt] * inv;
        if (lg == 0)
            lse_part[out_row] = bad_page ? __builtin_nanf("")
                                         : (l_run > 0.f ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2
                                                        : -__builtin_inff());
    } else {
        __syncthreads();   // every wave is done with the stages
        float* ml = reinterpret_cast<float*>(smem);                       // [NW][2][16]
        float* accs = reinterpret_cast<float*>(smem + C::NW * 2 * 16 * 4);  // [NW][16][512]
        if (lg == 0) {
            ml[(wave * 2 + 0) * 16 + lr] = m_run;
            ml[(wave * 2 + 1) * 16 + lr] = bad_page ? __builtin_nanf("") : l_run;
        }
        float* my = accs + (size_t)wave * 16 * kDv + lr * kDv;
#pragma unroll
        for (int dt = 0; dt < kDTiles; ++dt) *reinterpret_cast<f32x4*>(my + 16 * dt + 4 * lg) = acc[dt];
        __syncthreads();
        // RB row blocks x 16 rows x 512 dims, all threads
        for (int e = tid; e < C::RB * 16 * (kDv / 4); e += C::THREADS) {
            const int d4 = e % (kDv / 4);
            const int r = (e / (kDv / 4)) % 16;
            const int rbi = e / (16 * (kDv / 4));
            float M = -__builtin_inff();
            for (int g = 0; g < C::NG; ++g) M = fmaxf(M, ml[((g * C::RB + rbi) * 2) * 16 + r]);
            const float Mu = (M == -__builtin_inff()) ? 0.f : M;
            float Lsum = 0.f;
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
            bool nan = false;
            for (int g = 0; g < C::NG; ++g) {
                const int w = g * C::RB + rbi;
                const float lw = ml[(w * 2 + 1) * 16 + r];
                nan |= (lw != lw);
                const float sc = __builtin_amdgcn_exp2f(ml[(w * 2) * 16 + r] - Mu);
                Lsum += sc * lw;
                o += sc * *reinterpret_cast<const f32x4*>(accs + ((size_t)w * 16 + r) * kDv + 4 * d4);
            }
            const float inv = (Lsum > 0.f) ? 1.f / Lsum : 0.f;
            const int grow = (blockIdx.y * C::RB + rbi) * 16 + r;
            *reinterpret_cast<f32x4*>(o_part + (size_t)grow * kDv + 4 * d4) = o * inv;
            if (d4 == 0)
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
constexpr int kCombineThreads = 256;   // 2 rows x 128 threads x 4 dims

__global__ void __launch_bounds__(kCombineThreads) combine_kernel(FwdArgs a)
{
    const WsLayout lay = ws_layout(a.batch, a.rows, a.capacity);
    const int32_t* header = reinterpret_cast<const int32_t*>(a.ws + lay.header);
    const int gr = blockIdx.x * 2 + (threadIdx.x >> 7);      // global row = b * rows + r
    if (gr >= a.batch * a.rows) return;
    const int t = threadIdx.x & 127;
    const int b = gr / a.rows;
    const bool shape_ok = header[kHMagic] == kPlanMagic && header[kHBatch] == a.batch &&
                          header[kHSq] == a.s_q && header[kHHeads] == a.heads &&
                          header[kHCapacity] == a.capacity;
    uint16_t* orow = a.out + (size_t)gr * kDv + 4 * t;
    const float qnan = __builtin_nanf("");
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
    const int r = gr % a.rows;
    const float* lse_part = reinterpret_cast<const float*>(a.ws + lay.lse_part);
    const float* o_part = reinterpret_cast<const float*>(a.ws + lay.o_part);
    float M = -__builtin_inff();
    for (int s = s0; s < s1 && !poison; ++s) {
        const float v = lse_part[(size_t)s * a.rows + r];
        if (v != v) poison = true;
        M = fmaxf(M, v);
    }
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    float lse_out;
    if (poison) {
        o = f32x4{qnan, qnan, qnan, qnan};
        lse_out = qnan;
    } else if (M == -__builtin_inff()) {
        lse_out = -__builtin_inff();
    } else {
        float W = 0.f;
        for (int s = s0; s < s1; ++s) {
            const float w = expf(lse_part[(size_t)s * a.rows + r] - M);
            W += w;
            o += w * *reinterpret_cast<const f32x4*>(o_part + ((size_t)s * a.rows + r) * kDv + 4 * t);
        }
        o *= 1.f / W;
        lse_out = M + logf(W);
    }
    ushort4 ob;
    ob.x = f32_to_bf16_rne(o[0]);
    ob.y = f32_to_bf16_rne(o[1]);
    ob.z = f32_to_bf16_rne(o[2]);
    ob.w = f32_to_bf16_rne(o[3]);
    *reinterpret_cast<ushort4*>(orow) = ob;
    if (t == 0) a.lse[gr] = lse_out;
}

}  // namespace mla
