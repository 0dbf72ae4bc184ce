// gfx950 split kernel for 128 query rows per workgroup (all heads of a GPU): one wave per SIMD,
// each wave owning 32 query rows from the score product to the output.
//
// What is computed is the same as in split_kernel (FlashMLA-ETAP summary, "Mecanismo Central":
// S^T = K Q^T, P^T = softmax of S^T down the key axis, O^T = V^T P^T).  This form is for the
// case where the contractions, not the cache stream, set the pace: with 128 heads the absorbed
// path does ~242 FLOP per cache byte (GQLA summary, "Arquitetura", item 1), near MI355X's
// compute/bandwidth ridge.
//
// A workgroup takes one work item (a page range of one sequence) for up to 128 query rows, so a
// cache tile crosses the CU's memory path and LDS once for all of them.  Wave w owns rows
// 32 w .. 32 w + 31 and keeps, for the whole item,
//   Q^T of its rows   as the B operand of v_mfma_f32_32x32x16_bf16 (144 VGPRs),
//   O^T of its rows   all 512 value dims, 16 tiles of 32x32 fp32 (256 accumulation registers).
// Per 32-token tile it computes S^T (32 tokens x 32 rows, 36 MFMAs with the K tile as the A
// operand), the online softmax of its rows (a row lives in two lanes, l and l + 32, so a row
// statistic is one cross-half swap away), and O^T += V^T P^T (32 MFMAs).  In the 32x32 result
// layout, registers 8 ks .. 8 ks + 7 of the S^T accumulator are exactly the P^T B operand of
// value k-step ks once V^T is read with the matching key order, so P never leaves the lane.
//
// Pipeline (one barrier per 32-token step): step t loads tile t + 3, scores tile t + 1 with the
// softmax of tile t spread over its first k-steps, and accumulates tile t, its value MFMAs
// interleaved with the remaining score MFMAs (the score chain's dependent issue is then covered
// by independent value MFMAs).  LDS holds four tile stages; a tile's loads have two steps to land.
//
// LDS tile layout: cache row r at r * 1168 B (73 16-B chunks, the last one zero): the 32-row K
// operand read and the transposing V^T read both run without bank conflicts at this stride.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_decode_kernels.h"

// LDS-read look-ahead (K operands in score k-steps, V^T operands in value MFMAs)
#ifndef MLA_RW_KD
#define MLA_RW_KD 3
#endif
#ifndef MLA_RW_VD
#define MLA_RW_VD 3
#endif

namespace mla {

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int NW_>
struct RwCfg {
    static constexpr int NW = NW_;                               // waves = 32-row blocks
    static constexpr int RW = 32 * NW;                           // query rows per workgroup
    static constexpr int THREADS = 64 * NW;
    static constexpr int TT = 32;                                // tokens per tile
    static constexpr int NS = 4;                                 // LDS tile stages
    static constexpr int LCH = kChunksPerRow + 1;                // 73 16-B chunks per LDS row
    static constexpr int LROW = LCH * 16;                        // 1168 B
    static constexpr int UNITS = (TT * LROW + 1023) / 1024;      // 37 1-KiB load units per tile
    static constexpr int STAGE = UNITS * 1024;                   // 37888 B
    static constexpr int UW = (UNITS + NW - 1) / NW;             // load units of wave 0 (10)
    static constexpr int KSTEPS = kDk / 16;                      // 36 score k-steps of 16 dims
    static constexpr int DT = kDv / 32;                          // 16 value tiles of 32 dims
    static constexpr int SM_STEPS = 10;                          // score k-steps carrying the softmax
    static constexpr int OFF_BAD = NS * STAGE;                   // int[NW]: per-wave bad flags
    static constexpr int LDS_BYTES = OFF_BAD + 4 * NW;
    static_assert(UW * NW >= UNITS && (UW - 1) * NW < UNITS, "units per wave");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    static_assert((NS & (NS - 1)) == 0, "stage index by mask");
    static_assert(KSTEPS - SM_STEPS <= 2 * DT, "value MFMAs cover the score k-steps after the softmax");
};

// the two lanes of a row (l, l ^ 32): max / sum of their values
__device__ inline float pair_max32(float v)
{
    auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ inline float pair_sum32(float v)
{
    auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Both contractions are issued as inline asm, which pins their accumulators: O^T in the 256
// AGPRs, S^T in VGPRs.  (With builtins the compiler carried the loop's O^T through VGPR copies
// and spilled.)  Dependent MFMAs with the same accumulator are interlocked by the hardware; the
// other hazards are covered by hand: a vector-ALU read of an MFMA result waits 24 cycles
// (mfma_s_drain, mfma_o_drain), and an MFMA that reads registers a vector-ALU instruction has
// just written is preceded by two wait states (mfma_o_after_valu).
// The score chain's first MFMA adds to zero (no read of the accumulator).
__device__ inline void mfma_s_first(f32x16& c, bf16x8 a, bf16x8 b)
{
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ inline void mfma_s_next(f32x16& c, bf16x8 a, bf16x8 b)
{
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ inline void mfma_s_drain(f32x16& c) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(c)); }
__device__ inline void mfma_o(f32x16& c, bf16x8 a, bf16x8 b)
{
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ inline void mfma_o_after_valu(f32x16& c, bf16x8 a, bf16x8 b)
{
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// all 16 O^T tiles, before vector-ALU code reads them
__device__ inline void mfma_o_drain(f32x16* c)
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(c[0]), "+a"(c[1]), "+a"(c[2]), "+a"(c[3]), "+a"(c[4]), "+a"(c[5]), "+a"(c[6]), "+a"(c[7]));
    asm volatile("" : "+a"(c[8]), "+a"(c[9]), "+a"(c[10]), "+a"(c[11]), "+a"(c[12]), "+a"(c[13]), "+a"(c[14]), "+a"(c[15]));
}
// Explicit moves of an O^T tile between AGPRs and VGPRs (the compiler emits the copy for the
// tied operand).  Every other use of O^T is an asm operand with the AGPR constraint, so the
// register allocator keeps the tiles in AGPRs for their whole life.
__device__ inline f32x16 o_to_vgpr(f32x16 a)
{
    f32x16 r;
    asm volatile("" : "=v"(r) : "0"(a));
    return r;
}
__device__ inline f32x16 o_from_vgpr(f32x16 v)
{
    f32x16 r;
    asm volatile("" : "=a"(r) : "0"(v));
    return r;
}

template <class C>
__global__ void __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
split_rw_kernel(FwdArgs a)
{
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, g = lane >> 5;

    // the row groups of an item get workgroup ids 8 apart (same XCD)
    const int G = a.row_groups;
    const int x = blockIdx.x;
    const int item = (x / (8 * G)) * 8 + x % 8;
    const int rg = (x / 8) % G;

    const WsLayout lay = ws_layout(a.batch, a.rows, a.capacity);
    asm volatile("" ::"s"(a.q), "s"(a.block_table), "s"(a.seqlens), "s"(a.bt_stride));
    const PlanItem pi = read_plan_item(a, lay, item);
    if (!pi.ok) return;   // a plan mismatch is reported by the combine kernel
    const i32x4 it = pi.it;
    const int b = it[0];
    const int L = a.seqlens[b];
    const int32_t plan_L = reinterpret_cast<const int32_t*>(a.ws + lay.seqlens)[b];
    float* lse_part = reinterpret_cast<float*>(a.ws + lay.lse_part) + (size_t)item * a.rows;
    float* o_part = reinterpret_cast<float*>(a.ws + lay.o_part) + (size_t)item * a.rows * kDv;

    // A sequence whose length disagrees with the plan or the table gets no tiles and a NaN LSE.
    const bool bad_seq = (L != plan_L) | (L < 0) | ((long long)L > (long long)kPage * a.bt_stride);
    const int tok_begin = it[1] * kPage;
    const int tok_end = (int)min((long long)it[2] * kPage, (long long)L);
    const int n_tiles = bad_seq ? 0 : (tok_end - tok_begin + C::TT - 1) / C::TT;

    const int blk_row0 = rg * C::RW + 32 * wave;
    const bool has_rows = blk_row0 < a.rows;   // wave-uniform
    const int row = blk_row0 + l32;            // this lane's query row
    const bool row_ok = row < a.rows;
    // stage of tile t (t >= -1)
    auto stage = [&](int t) __attribute__((always_inline)) { return smem + (t & (C::NS - 1)) * C::STAGE; };
    int* const bad_s = reinterpret_cast<int*>(smem + C::OFF_BAD);

    // ---- tile loads: unit u = wave + NW k; lane l of unit u fills LDS chunk c = 64 u + l = 73 r + ch
    // of the stage with cache chunk 72 r + ch, or zeros for the pad chunk and past the tile (an
    // offset past the buffer resource's end reads zeros)
    PageWindow pw;
    pw.init(a.block_table + (size_t)b * a.bt_stride, a.bt_stride);
    pw.prefetch(it[1], lane);
    asm volatile("" ::"s"(a.num_pages), "s"(a.cache));
    // (offsets are recomputed per load: a few ALU ops instead of UW registers held all along)
    auto voff = [&](int k) __attribute__((always_inline)) {
        const int c = 64 * (wave + C::NW * k) + lane;
        const int r = c / C::LCH, ch = c - C::LCH * r;
        return (r < C::TT && ch < kChunksPerRow) ? 16 * (kChunksPerRow * r + ch) : (1 << 30);
    };
    const bool full_units = wave + C::NW * (C::UW - 1) < C::UNITS;   // this wave moves UW units (else UW - 1)
    bool bad_page = false;
    // Every call issues the same number of loads (a tile past the item loads zeros), so a wait
    // for "all but the last call's loads" is one fixed vmcnt per wave.
    auto load_tile = [&](int t) __attribute__((always_inline)) {
        int valid = 0, page = 0;
        const int t0 = tok_begin + t * C::TT;
        if (t >= 0 && t < n_tiles) {
            page = pw.page(t0 / kPage, lane);
            valid = min(C::TT, L - t0);
            if (page < 0 || (long long)page >= a.num_pages) {
                bad_page = true;
                valid = 0;
            }
        }
        const uint16_t* base = a.cache + ((long long)(valid ? page : 0) * kPage + (valid ? t0 % kPage : 0)) * kDk;
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, valid * kRowBytes, 0x00020000);
        const uint32_t st = (uint32_t)(uintptr_t)(MLA_LDS char*)stage(t);
#pragma unroll
        for (int k = 0; k < C::UW; ++k)
            if (k < C::UW - 1 || full_units) lds_load_16(r, st + 1024 * (wave + C::NW * k), voff(k));
    };
    // wait until only the last load_tile call's loads may be in flight
    auto wait_all_but_last = [&]() __attribute__((always_inline)) {
        constexpr int enc_full = 0x0F70 | (C::UW & 15) | ((C::UW >> 4) << 14);
        constexpr int enc_less = 0x0F70 | ((C::UW - 1) & 15) | (((C::UW - 1) >> 4) << 14);
        if (full_units)
            __builtin_amdgcn_s_waitcnt(enc_full);
        else
            __builtin_amdgcn_s_waitcnt(enc_less);
    };

    // ---- score operands.  Q^T of k-step j (dims 16 j .. 16 j + 15): lane (l32, g) holds
    // q[row][16 j + 8 g .. + 8]; K of k-step j: lane (l32, g) holds tile row l32, the same dims.
    bf16x8 qop[C::KSTEPS];
    {
        const uint16_t* qrow = a.q + ((size_t)b * a.rows + (row_ok ? row : 0)) * kDk + 8 * g;
#pragma unroll
        for (int j = 0; j < C::KSTEPS; ++j) {
            const bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + 16 * j);
            qop[j] = row_ok ? v : bf16x8{};
        }
    }
    const int kbase = l32 * C::LROW + 16 * g;
    // V^T transposing read: lane (G = lane / 16) gives the address of token 4 g + (lane % 16) / 4
    // (+ 8 for the operand's second half, + 16 ks for k-step ks), dims 32 d + 16 (G % 2) + 4 (lane % 4)
    // .. + 3; the read returns lane l32's dim 32 d + l32, tokens 16 ks + 4 g + 0..3 (+ 8).
    const int vbase = (4 * g + (lane & 15) / 4) * C::LROW + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));

    const int nvis = a.causal ? min(max(L - a.s_q + 1 + row / a.heads, 0), L) : L;
    const int nvis_blk = a.causal ? min(max(L - a.s_q + 1 + blk_row0 / a.heads, 0), L) : L;   // the block's smallest
    asm volatile("" ::"s"(a.scale_log2));

    // state of the online softmax: row max m (both lanes of a row agree) and this lane's part of
    // the row sum l, both in the log2 domain
    float m_run = -__builtin_inff(), l_run = 0.f;
    f32x16 acc[C::DT];   // acc[d] register r: O^T[32 d + 8 (r / 4) + 4 g + r % 4][row]
#pragma unroll
    for (int d = 0; d < C::DT; ++d) acc[d] = o_from_vgpr(f32x16{});
    // scaled, masked S^T of the tile awaiting its softmax, then its P; tile -1 is fully masked
    f32x16 s_cur;
#pragma unroll
    for (int r = 0; r < 16; ++r) s_cur[r] = -__builtin_inff();
    float tmax_cur = -__builtin_inff();

    // One step: S^T of tile ts (DO_S; MASK: tile ts holds some row's end of visible keys) and, for
    // tile tv (DO_V), its softmax over the first SM_STEPS k-steps and O^T += V^T P^T on the rest.
    auto step = [&](int ts, int tv) __attribute__((always_inline)) {
        constexpr bool do_s = true, do_v = true;
        constexpr int KD = MLA_RW_KD, VD = MLA_RW_VD;
        const char* kst = stage(ts) + kbase;
        const char* vst = stage(tv) + vbase;
        bf16x8 kop[KD + 1];
        i16x4 vlo[VD + 1], vhi[VD + 1];
        f32x16 sacc;
        bf16x8 pk[2];
        float m_use = 0.f, psum = 0.f;
        bool resc = false;
        float alpha = 1.f;
        auto vread = [&](int i, i16x4& lo, i16x4& hi) __attribute__((always_inline)) {   // value MFMA i = 16 ks + d
            const char* p = vst + (i / 16) * 16 * C::LROW + 64 * (i % 16);
            lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)lds_i16x4(p));
            hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)lds_i16x4(p + 8 * C::LROW));
        };
        auto value_mfma = [&](int i) __attribute__((always_inline)) {
            if (i + VD < 2 * C::DT) vread(i + VD, vlo[(i + VD) % (VD + 1)], vhi[(i + VD) % (VD + 1)]);
            const bf16x8 vop = __builtin_shufflevector(__builtin_bit_cast(bf16x4, vlo[i % (VD + 1)]),
                                                       __builtin_bit_cast(bf16x4, vhi[i % (VD + 1)]), 0, 1, 2, 3, 4, 5, 6, 7);
            if (i == 0)   // the P^T operands were just written by vector-ALU conversions
                mfma_o_after_valu(acc[0], vop, pk[0]);
            else
                mfma_o(acc[i % 16], vop, pk[i / 16]);
        };
        auto score_mfma = [&](int j) __attribute__((always_inline)) {
            if constexpr (do_s) {
                if (j + KD < C::KSTEPS) kop[(j + KD) % (KD + 1)] = *reinterpret_cast<const bf16x8*>(kst + 32 * (j + KD));
                if (j == 0)
                    mfma_s_first(sacc, kop[0], qop[0]);
                else
                    mfma_s_next(sacc, kop[j % (KD + 1)], qop[j]);
            }
        };
        if constexpr (do_s) {
#pragma unroll
            for (int j = 0; j < KD; ++j) kop[j] = *reinterpret_cast<const bf16x8*>(kst + 32 * j);
        }
        // k-step 0: the lazy max update (m moves only when a row's tile max passes it by 2^8)
        score_mfma(0);
        if constexpr (do_v) {
            const bool move = __builtin_amdgcn_ballot_w64(tmax_cur > m_run + 8.f) != 0;
            const float m_new = move ? fmaxf(m_run, tmax_cur) : m_run;
            alpha = (m_new == -__builtin_inff()) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
            // O^T needs the rescale only where it may be nonzero (a row's first tile finds it zero)
            resc = __builtin_amdgcn_ballot_w64(alpha != 1.f && m_run != -__builtin_inff()) != 0;
            m_run = m_new;
            l_run *= alpha;
            m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
#pragma unroll
            for (int i = 0; i < VD; ++i) vread(i, vlo[i], vhi[i]);
        }
        __builtin_amdgcn_sched_barrier(0);
        // k-steps 1-8: p = 2^(s - m), two per k-step
#pragma unroll
        for (int j = 1; j < 9; ++j) {
            score_mfma(j);
            if constexpr (do_v) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int r = 2 * (j - 1) + e;
                    float p = __builtin_amdgcn_exp2f(s_cur[r] - m_use);
                    asm volatile("" : "+v"(p));   // computed here, between the score MFMAs (not sunk to its use)
                    s_cur[r] = p;
                    psum += p;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // k-step 9: the P^T operands of the two value k-steps, and the rescale if any
        score_mfma(9);
        if constexpr (do_v) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) pk[ks][e] = (__bf16)s_cur[8 * ks + e];
            l_run += psum;
            if (resc) {   // one tile at a time (each passes through VGPRs)
                mfma_o_drain(acc);
#pragma unroll
                for (int d = 0; d < C::DT; ++d) {
                    acc[d] = o_from_vgpr(o_to_vgpr(acc[d]) * alpha);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // the remaining k-steps, each beside one value MFMA; then the rest of the value MFMAs
#pragma unroll
        for (int j = C::SM_STEPS; j < C::KSTEPS; ++j) {
            score_mfma(j);
            if constexpr (do_v) value_mfma(j - C::SM_STEPS);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (do_v) {
#pragma unroll
            for (int i = C::KSTEPS - C::SM_STEPS; i < 2 * C::DT; ++i) {
                value_mfma(i);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (do_s) {   // the new tile's scale, key mask and row max
            mfma_s_drain(sacc);
            s_cur = sacc * a.scale_log2;
            if (tok_begin + (ts + 1) * C::TT > nvis_blk) {   // tile ts holds some row's end of visible keys
                const int t0 = tok_begin + ts * C::TT + 4 * g;   // token of register 0
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    s_cur[r] = (t0 + 8 * (r / 4) + r % 4 >= nvis) ? -__builtin_inff() : s_cur[r];
            }
            float mx = s_cur[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s_cur[r]);
            tmax_cur = pair_max32(mx);
        }
    };
    // Steps t = -1 .. n_tiles - 1 all take the same form (one code path keeps the compiler's
    // accumulator registers in place): step t scores tile t + 1 and weights tile t.  Tile -1 and the
    // tiles past the item are zeros, and a zero tile's P is zero (its S^T is masked or never
    // weighted), so the first step's value product adds nothing and the last step's score is unused.
    if (n_tiles > 0) {
        load_tile(-1);
        load_tile(0);
        load_tile(1);
        wait_all_but_last();
        __syncthreads();   // tiles -1 and 0 are in LDS
        for (int t = -1; t < n_tiles; ++t) {
            load_tile(t + 3);
            if (has_rows) step(t + 1, t);
            wait_all_but_last();
            __syncthreads();   // tile t + 2 is in LDS; every wave is done with tiles t and t + 1
        }
        vm_wait_all();   // the zero loads past the item
    }
    if (lane == 0) bad_s[wave] = (bad_page || bad_seq) ? 1 : 0;
    __syncthreads();
    bool bad = false;
#pragma unroll
    for (int w = 0; w < C::NW; ++w) bad |= bad_s[w] != 0;
    if (!has_rows) return;

    mfma_o_drain(acc);
    const float l = pair_sum32(l_run);
    if (g == 0 && row_ok)
        lse_part[row] = bad ? __builtin_nanf("") : (l > 0.f ? (m_run + __builtin_amdgcn_logf(l)) * kLn2 : -__builtin_inff());
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    if (row_ok) {
        float* orow = o_part + (size_t)row * kDv + 4 * g;
#pragma unroll
        for (int d = 0; d < C::DT; ++d) {
            const f32x16 o = o_to_vgpr(acc[d]);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *reinterpret_cast<f32x4*>(orow + 32 * d + 8 * q4) = f32x4{o[4 * q4], o[4 * q4 + 1], o[4 * q4 + 2], o[4 * q4 + 3]} * inv;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

}  // namespace mla
