// gfx950 split kernel for 32 to 256 query rows per sequence (all heads of a GPU, or a share of
// them with two query tokens): score waves and value waves paired on every SIMD.
//
// What is computed is the same as in split_kernel (FlashMLA-ETAP summary, "Mecanismo Central":
// S^T = K Q^T, P^T = softmax of S^T down the key axis, O^T = V^T P^T).  This form is built for
// the case where the contractions, not the cache stream, set the pace: with 128 heads the
// absorbed path does ~242 FLOP per cache byte (GQLA summary, "Arquitetura", item 1), near
// MI355X's compute/bandwidth ridge.
//
// A workgroup takes one work item (a page range of one sequence) for 64 query rows (32 with
// NRB = 1).  Its eight waves, two per SIMD (waves w and w + 4 share a SIMD):
//   score waves 0-3  wave w owns the 32-row block rb = w / 2 (Q^T in registers) and the token
//                    half th = w % 2 of every 32-token tile: S^T = K Q^T with
//                    v_mfma_f32_16x16x32_bf16, one K-operand read feeding both 16-row halves of
//                    the block; the online softmax of its 32 rows x 16 tokens (the two halves of a
//                    block exchange their tile maxima through LDS and take identical decisions);
//                    P^T (bf16), rescale factors and flags go to LDS;
//   value waves 4-7  wave 4 + v owns value dims 128 v .. 128 v + 127 of all the rows:
//                    O^T += V^T P^T with v_mfma_f32_32x32x16_bf16 (V^T read straight from the
//                    row-major tile with transposing LDS reads), and moves a quarter of every
//                    tile HBM -> VGPR -> LDS (16-B non-temporal buffer loads, two tiles in flight
//                    in registers per wave).
// Per 32-token tile every SIMD runs 36 score MFMAs (16x16x32) and 16 value MFMAs (32x32x16):
// 576 + 512 cycles of its matrix pipe.  On gfx950 a wave's own vector instructions and waits
// stall its next MFMA while the other wave's do not (measured), so every SIMD keeps two
// MFMA-issuing waves, each covering the other's stalls.
//
// Pipeline (one barrier per step): step t scores tile t + 1 and runs the softmax of tile t
// (score waves), accumulates tile t - 1 (value waves), stores tile t + 2 from registers to LDS
// and loads tile t + 4 into the registers it leaves; tile k is loaded at step k - 4, stored at
// k - 2, scored at k - 1, weighted at k, accumulated at k + 1, so LDS holds four stages and
// every load has two steps to arrive.  (Loading straight into LDS would leave each load one
// step: the four stages are all in use.)
//
// LDS tile layout: row r at r * 1184 B (74 16-B chunks: the 16-row K-operand read hits 32
// distinct bank groups); a row's two pad chunks are never written or read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_decode_kernels.h"

// LDS-read look-ahead of the score waves (K operands, in k-steps) and of the value waves (V^T
// operand pairs)
#ifndef MLA_SV_KD
#define MLA_SV_KD 3
#endif
#ifndef MLA_SV_VD
#define MLA_SV_VD 2
#endif

namespace mla {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kOutRow = kDv * 4 + 16;   // LDS row of a normalised fp32 partial output (2064 B)

template <int NRB_>
struct SvCfg {
    static constexpr int NRB = NRB_;         // 32-row blocks per workgroup (1 or 2)
    static constexpr int RW = 32 * NRB;      // query rows per workgroup
    static constexpr int NW = 8;
    static constexpr int THREADS = NW * 64;
    static constexpr int TT = 32;                              // tokens per tile
    static constexpr int NS = 4;                               // LDS tile stages
    static constexpr int LCH = kChunksPerRow + 2;              // 74 16-B chunks per LDS tile row
    static constexpr int LROW = LCH * 16;                      // 1184 B
    static constexpr int LDS_TILE = TT * LROW;                 // 37888 B
    static constexpr int UNITS = TT * kRowBytes / 1024;        // 36 one-KiB load units per tile
    static constexpr int UV = UNITS / 4;                       // units per value wave
    static constexpr int KSTEPS = kDk / 32;                    // 18 score k-steps of 32
    static constexpr int OFF_P = NS * LDS_TILE;                // P^T [2 parity][rb][ks][64 lanes][16 B]
    static constexpr int P_BYTES = 2 * 2 * 1024;
    static constexpr int OFF_MX = OFF_P + 2 * P_BYTES;         // fp32 [2 parity][rb][th][32]: tile maxima
    static constexpr int OFF_ALPHA = OFF_MX + 2 * 2 * 2 * 32 * 4;   // fp32 [2 parity][64]
    static constexpr int OFF_FLAG = OFF_ALPHA + 2 * 64 * 4;    // int [2 parity][rb]
    static constexpr int OFF_ML = OFF_FLAG + 2 * 2 * 4;        // fp32 [3][64]: m, l of half 0, l of half 1
    static constexpr int OFF_BAD = OFF_ML + 3 * 64 * 4;        // int [8]: per-wave bad-page flags
    static constexpr int LDS_BYTES = OFF_BAD + 8 * 4;
    static_assert(UV * 4 == UNITS, "four value waves, whole units each");
    static_assert(NRB == 1 || NRB == 2, "32 or 64 rows per workgroup");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    static_assert(RW * kOutRow <= NS * LDS_TILE, "partial rows fit the tile stages");
};

template <class C>
__global__ void __launch_bounds__(C::THREADS) split_sv_kernel(FwdArgs a)
{
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

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
    const int row_base = rg * 64;   // row groups of 64 (the last may hold fewer valid rows)

    // A sequence whose length disagrees with the plan or the table gets no tiles and a NaN LSE.
    const bool bad_seq = (L != plan_L) | (L < 0) | ((long long)L > (long long)kPage * a.bt_stride);
    const int tok_begin = it[1] * kPage;
    const int tok_end = (int)min((long long)it[2] * kPage, (long long)L);
    const int n_tiles = bad_seq ? 0 : (tok_end - tok_begin + C::TT - 1) / C::TT;

    char* const pbuf = smem + C::OFF_P;
    float* const mx_s = reinterpret_cast<float*>(smem + C::OFF_MX);
    float* const alpha_s = reinterpret_cast<float*>(smem + C::OFF_ALPHA);
    int* const flag_s = reinterpret_cast<int*>(smem + C::OFF_FLAG);
    float* const ml_s = reinterpret_cast<float*>(smem + C::OFF_ML);
    int* const bad_s = reinterpret_cast<int*>(smem + C::OFF_BAD);
    auto stage = [&](int t) __attribute__((always_inline)) { return smem + (t % C::NS) * C::LDS_TILE; };
    constexpr float kLazyRescale = 8.f;
    bool bad_page = false;
    asm volatile("" ::"s"(a.num_pages), "s"(a.cache));
    // buffer resource of tile t (rows past L_b and past the last tile read as zeros)
    auto tile_rsrc = [&](PageWindow& pw, int t) __attribute__((always_inline)) {
        if (t >= n_tiles) return __builtin_amdgcn_make_buffer_rsrc((void*)a.cache, (short)0, 0, 0x00020000);
        const int t0 = tok_begin + t * C::TT;
        const int page = pw.page(t0 / kPage, lane);
        int valid = min(C::TT, L - t0);
        if (page < 0 || (long long)page >= a.num_pages) {
            bad_page = true;
            valid = 0;
        }
        const uint16_t* base = a.cache + ((long long)(valid ? page : 0) * kPage + (t0 % kPage)) * kDk;
        return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, valid * kRowBytes, 0x00020000);
    };

    if (wave < 4) {
        // ================= score waves =================
        const int rb = wave >> 1, th = wave & 1;
        const int lr = lane & 15, lg = lane >> 4;
        const bool has_rows = rb < C::NRB;
        const int blk_row0 = row_base + 32 * rb;
        auto nvis_of = [&](int row) __attribute__((always_inline)) {
            return a.causal ? min(max(L - a.s_q + 1 + row / a.heads, 0), L) : L;
        };
        const int nvis_blk = nvis_of(blk_row0);   // the block's smallest
        const int nvis_h0 = nvis_of(blk_row0 + lr), nvis_h1 = nvis_of(blk_row0 + 16 + lr);
        // the loop's scalar kernel argument is held in an SGPR from here on (a scalar load left
        // pending inside the loop would make every LDS wait there a wait for all LDS traffic)
        asm volatile("" ::"s"(a.scale_log2));
        // Q^T operand of k-step j, row half h: lane (lr, lg) holds q[blk_row0 + 16 h + lr][32 j + 8 lg .. + 8]
        bf16x8 qop[C::KSTEPS][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = blk_row0 + 16 * h + lr;
            const bool ok = has_rows && row < a.rows;
            const uint16_t* qrow = a.q + ((size_t)b * a.rows + (ok ? row : 0)) * kDk + 8 * lg;
#pragma unroll
            for (int j = 0; j < C::KSTEPS; ++j) {
                const bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + 32 * j);
                qop[j][h] = ok ? v : bf16x8{};
            }
        }
        // K operand of k-step j: token 16 th + lr of the tile, dims 32 j + 8 lg .. + 8
        const int kbase = (16 * th + lr) * C::LROW + 16 * lg;
        constexpr int KD = MLA_SV_KD;   // K-operand look-ahead (k-steps)
        // The 16x16 result: lane (lr, lg), register i holds S^T[token 16 th + 4 lg + i][row 16 h + lr].
        // Those four tokens are the value product's B-operand elements 4 (lg >> 1) .. + 3 of lane
        // 16 h + lr + 32 (lg & 1), k-step th.
        const int pslot = th * 1024 + 16 * (lr + 32 * (lg & 1)) + 8 * (lg >> 1);
        float m_run[2] = {-__builtin_inff(), -__builtin_inff()};   // identical in both halves of a block
        float l_run[2] = {0.f, 0.f};          // lane-partial sums (this lane's tokens), row half h
        f32x4 s[2] = {};                      // scaled, masked S^T of the tile awaiting its softmax
        float tmax_own[2] = {0.f, 0.f};       // its max over this half's 16 tokens, per row
        // score_step: S^T of tile ts (DO_S) with the softmax of tile tsm (DO_SM) spread over its
        // k-steps; after the last MFMA the new tile's scale, key mask (MASK: tile ts holds some
        // row's end of visible keys) and this half's row maxima, which go to LDS for the other half
        auto score_step = [&](auto do_s_tag, auto do_sm_tag, auto mask_tag, int ts, int tsm) __attribute__((always_inline)) {
            constexpr bool do_s = decltype(do_s_tag)::value != 0;
            constexpr bool do_sm = decltype(do_sm_tag)::value != 0;
            constexpr bool masked = decltype(mask_tag)::value != 0;
            const char* kst = stage(ts) + kbase;
            bf16x8 kop[KD + 1];
            f32x4 sp[2][2] = {};
            if constexpr (do_s) {
#pragma unroll
                for (int j = 0; j < KD; ++j) kop[j] = *reinterpret_cast<const bf16x8*>(kst + 64 * j);
            }
            const int par = tsm & 1;
            float tmax[2] = {0.f, 0.f}, m_use[2] = {0.f, 0.f}, alpha[2] = {1.f, 1.f}, psum[2] = {0.f, 0.f};
            bool resc = false;
#pragma unroll
            for (int j = 0; j < C::KSTEPS; ++j) {
                if constexpr (do_s) {
                    if (j + KD < C::KSTEPS) kop[(j + KD) % (KD + 1)] = *reinterpret_cast<const bf16x8*>(kst + 64 * (j + KD));
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        sp[h][j & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[j % (KD + 1)], qop[j][h], sp[h][j & 1], 0, 0, 0);
                }
                if constexpr (do_sm) {
                    if (j == 0) {   // the block's tile maxima: this half's and the other half's
                        const float* mo = mx_s + ((par * 2 + rb) * 2 + (th ^ 1)) * 32;
                        tmax[0] = fmaxf(tmax_own[0], mo[lr]);
                        tmax[1] = fmaxf(tmax_own[1], mo[16 + lr]);
                    } else if (j == 1) {   // lazy max update: the same decision in both halves
                        resc = __builtin_amdgcn_ballot_w64((tmax[0] > m_run[0] + kLazyRescale) |
                                                           (tmax[1] > m_run[1] + kLazyRescale)) != 0;
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const float m_new = resc ? fmaxf(m_run[h], tmax[h]) : m_run[h];
                            alpha[h] = (m_new == -__builtin_inff()) ? 1.f : __builtin_amdgcn_exp2f(m_run[h] - m_new);
                            m_run[h] = m_new;
                            l_run[h] *= alpha[h];
                            m_use[h] = (m_new == -__builtin_inff()) ? 0.f : m_new;
                        }
                    } else if (j == 2) {   // half 0 publishes the rescale factors (the lanes of a row agree)
                        if (th == 0) {
                            alpha_s[par * 64 + 32 * rb + lr] = alpha[0];
                            alpha_s[par * 64 + 32 * rb + 16 + lr] = alpha[1];
                            flag_s[par * 2 + rb] = resc ? 1 : 0;
                        }
                    } else if (j < 11) {   // p = 2^(s - m), one per k-step
                        const int h = (j - 3) / 4, i = (j - 3) % 4;
                        s[h][i] = __builtin_amdgcn_exp2f(s[h][i] - m_use[h]);
                        psum[h] += s[h][i];
                    } else if (j == 11) {   // P^T out, in the value product's B-operand layout
                        char* pb = pbuf + par * C::P_BYTES + rb * 2048 + pslot;
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const bf16x4 pk = {(__bf16)s[h][0], (__bf16)s[h][1], (__bf16)s[h][2], (__bf16)s[h][3]};
                            *reinterpret_cast<bf16x4*>(pb + 256 * h) = pk;   // value lanes 16 h + ...
                            l_run[h] += psum[h];
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (do_s) {
                const int t0 = tok_begin + ts * C::TT + 16 * th + 4 * lg;   // token of register 0
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    s[h] = (sp[h][0] + sp[h][1]) * a.scale_log2;
                    if constexpr (masked) {
                        const int nv = h ? nvis_h1 : nvis_h0;
#pragma unroll
                        for (int i = 0; i < 4; ++i) s[h][i] = (t0 + i >= nv) ? -__builtin_inff() : s[h][i];
                    }
                    tmax_own[h] = wave_max_groups(fmaxf(fmaxf(s[h][0], s[h][1]), fmaxf(s[h][2], s[h][3])));
                }
                float* mw = mx_s + (((ts & 1) * 2 + rb) * 2 + th) * 32;
                mw[lr] = tmax_own[0];
                mw[16 + lr] = tmax_own[1];
            }
        };
        // tile t needs the key mask when it ends past the block's first row's visible keys
        auto crosses = [&](int t) __attribute__((always_inline)) { return tok_begin + (t + 1) * C::TT > nvis_blk; };
        if (n_tiles > 0) {
            __syncthreads();   // tiles 0 and 1 are in LDS
            if (has_rows) {
                if (crosses(0))
                    score_step(Idx<1>{}, Idx<0>{}, Idx<1>{}, 0, 0);
                else
                    score_step(Idx<1>{}, Idx<0>{}, Idx<0>{}, 0, 0);
            }
            __syncthreads();   // tile 0's maxima are in LDS
            for (int t = 0; t + 1 < n_tiles; ++t) {   // score tile t + 1, softmax of tile t
                if (has_rows) {
                    if (crosses(t + 1))
                        score_step(Idx<1>{}, Idx<1>{}, Idx<1>{}, t + 1, t);
                    else
                        score_step(Idx<1>{}, Idx<1>{}, Idx<0>{}, t + 1, t);
                }
                __syncthreads();
            }
            if (has_rows) score_step(Idx<0>{}, Idx<1>{}, Idx<0>{}, 0, n_tiles - 1);   // softmax of the last tile
            __syncthreads();
        }
        // row sums over this half's tokens; half 0 also keeps the (common) row max
#pragma unroll
        for (int h = 0; h < 2; ++h) l_run[h] = wave_sum_groups(l_run[h]);
        ml_s[64 * (1 + th) + 32 * rb + lr] = l_run[0];
        ml_s[64 * (1 + th) + 32 * rb + 16 + lr] = l_run[1];
        if (th == 0) {
            ml_s[32 * rb + lr] = m_run[0];
            ml_s[32 * rb + 16 + lr] = m_run[1];
        }
        bad_s[wave] = bad_seq ? 1 : 0;
        __syncthreads();   // E1: (m, l) of every row and the bad-page flags are in LDS
        bool bad = false;
#pragma unroll
        for (int w = 0; w < 8; ++w) bad |= bad_s[w] != 0;
        if (th == 0 && lg == 0 && has_rows) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int r = 32 * rb + 16 * h + lr;
                const int row = row_base + r;
                const float l = ml_s[64 + r] + ml_s[128 + r];
                if (row < a.rows)
                    lse_part[row] = bad ? __builtin_nanf("")
                                        : (l > 0.f ? (ml_s[r] + __builtin_amdgcn_logf(l)) * kLn2 : -__builtin_inff());
            }
        }
        __syncthreads();   // E2: the value waves are done with the tile stages
    } else {
        // ================= value waves =================
        const int v = wave - 4;   // value dims 128 v .. 128 v + 127
        constexpr int NRB = C::NRB;
        const int l32 = lane & 31, g = lane >> 5;
        // ---- tile staging HBM -> VGPR -> LDS, two tiles in flight per wave: units u = v + 4 k of a
        // tile's 36 one-KiB units; lane l of unit u holds cache chunk c = 64 u + l (row c / 72),
        // which goes to LDS byte 16 (c + 2 (c / 72)) (rows padded to 74 chunks)
        PageWindow pw;
        pw.init(a.block_table + (size_t)b * a.bt_stride, a.bt_stride);
        pw.prefetch(it[1], lane);
        int soff[C::UV];
#pragma unroll
        for (int k = 0; k < C::UV; ++k) {
            const int c = 64 * (v + 4 * k) + lane;
            soff[k] = 16 * (c + 2 * (c / kChunksPerRow));
        }
        i32x4 sbuf[2][C::UV];
        // loads are issued on every path (past the last tile through an empty resource, which
        // reads zeros without a memory access), so every store waits only for its own units
        auto load = [&](int t, auto bi) __attribute__((always_inline)) {
            constexpr int B = decltype(bi)::value;
            const __amdgpu_buffer_rsrc_t r = tile_rsrc(pw, t);
#pragma unroll
            for (int k = 0; k < C::UV; ++k)
                sbuf[B][k] = __builtin_amdgcn_raw_buffer_load_b128(r, 16 * lane, 1024 * (v + 4 * k), kNonTemporal);
        };
        auto store = [&](int t, auto bi) __attribute__((always_inline)) {
            constexpr int B = decltype(bi)::value;
            char* st = stage(t);
#pragma unroll
            for (int k = 0; k < C::UV; ++k) *reinterpret_cast<i32x4*>(st + soff[k]) = sbuf[B][k];
        };
        // the loads of one step (unit k of tile t + 4, into the registers tile t + 2 has just left)
        // go out one per MFMA group of the value product: issued in one burst, they stall the wave
        // on a full memory queue while its MFMAs wait behind them
        auto slot = [&](int k, auto bi, __amdgpu_buffer_rsrc_t r) __attribute__((always_inline)) {
            constexpr int B = decltype(bi)::value;
            sbuf[B][k] = __builtin_amdgcn_raw_buffer_load_b128(r, 16 * lane, 1024 * (v + 4 * k), kNonTemporal);
        };

        // acc[d][rb]: O^T[128 v + 32 d + 8 (r / 4) + 4 g + r % 4][row 32 rb + l32], register r
        f32x16 acc[4][NRB];
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) acc[d][rb] = f32x16{};
        // V^T transposing read of k-step ks: lane (G = lane / 16) reads token 16 ks + 4 g + (lane % 16) / 4
        // (+ 8 for the second half of the operand), dims 128 v + 32 d + 16 (G % 2) + 4 (lane % 4) .. + 3
        const int vbase = (4 * g + (lane & 15) / 4) * C::LROW + 2 * (128 * v + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
        auto vread = [&](const char* p) __attribute__((always_inline)) {
            return __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)lds_i16x4(p));
        };
        auto value_step = [&](int tv, auto&& slot_fn) __attribute__((always_inline)) {
            const int par = tv & 1;
            const int2 flags = *reinterpret_cast<const int2*>(flag_s + par * 2);
            const char* pb = pbuf + par * C::P_BYTES + 16 * lane;
            bf16x8 pop[NRB][2];
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) pop[rb][ks] = *reinterpret_cast<const bf16x8*>(pb + rb * 2048 + ks * 1024);
            const char* vt = stage(tv) + vbase;
            constexpr int VD = MLA_SV_VD;   // look-ahead in operands (ks, d pairs)
            i16x4 vlo[VD + 1], vhi[VD + 1];
#pragma unroll
            for (int i = 0; i < VD; ++i) {
                const int ks = i / 4, d = i % 4;
                vlo[i] = vread(vt + ks * 16 * C::LROW + 64 * d);
                vhi[i] = vread(vt + ks * 16 * C::LROW + 8 * C::LROW + 64 * d);
            }
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                if (__builtin_amdgcn_readfirstlane(rb == 0 ? flags.x : flags.y) != 0) {
                    const float al = alpha_s[par * 64 + 32 * rb + l32];
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        acc[d][rb] *= al;
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {   // i = 4 ks + d
                const int ks = i / 4, d = i % 4;
                if (i + VD < 8) {
                    const int ks2 = (i + VD) / 4, d2 = (i + VD) % 4;
                    vlo[(i + VD) % (VD + 1)] = vread(vt + ks2 * 16 * C::LROW + 64 * d2);
                    vhi[(i + VD) % (VD + 1)] = vread(vt + ks2 * 16 * C::LROW + 8 * C::LROW + 64 * d2);
                }
                const bf16x8 vop = __builtin_shufflevector(__builtin_bit_cast(bf16x4, vlo[i % (VD + 1)]),
                                                           __builtin_bit_cast(bf16x4, vhi[i % (VD + 1)]), 0, 1, 2, 3, 4,
                                                           5, 6, 7);
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb)
                    acc[d][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[rb][ks], acc[d][rb], 0, 0, 0);
                slot_fn(i);
                __builtin_amdgcn_sched_barrier(0);
            }
            slot_fn(8);
        };
        // step t: store tile t + 2 from sbuf[t & 1] and load tile t + 4 into it, then accumulate
        // tile t - 1
        auto step = [&](int t, auto bi) __attribute__((always_inline)) {
            const __amdgpu_buffer_rsrc_t r = tile_rsrc(pw, t + 4);
            auto sl = [&](int k) __attribute__((always_inline)) { slot(k, bi, r); };
            if (t + 2 < n_tiles) store(t + 2, bi);
            if (t >= 1) {
                value_step(t - 1, sl);
            } else {
#pragma unroll
                for (int k = 0; k < C::UV; ++k) sl(k);
            }
            __syncthreads();
        };
        if (n_tiles > 0) {
            load(0, Idx<0>{});
            load(1, Idx<1>{});
            store(0, Idx<0>{});
            load(2, Idx<0>{});
            if (n_tiles > 1) store(1, Idx<1>{});
            load(3, Idx<1>{});
            __syncthreads();   // tiles 0 and 1 are in LDS
            __syncthreads();   // the score waves' tile-0 maxima
            int t = 0;
            for (; t + 1 < n_tiles; t += 2) {
                step(t, Idx<0>{});
                step(t + 1, Idx<1>{});
            }
            if (t < n_tiles) step(t, Idx<0>{});
        }
        bad_s[wave] = (bad_page || bad_seq) ? 1 : 0;
        __syncthreads();   // E1: (m, l) of every row are in LDS; P^T of the last tile too
        if (n_tiles > 0) value_step(n_tiles - 1, [](int) {});
        __syncthreads();   // E2: every value wave is done with the tile stages
        // normalised partial rows into LDS, [row][dim] with rows padded to 2064 B (rows 16 B apart in
        // the bank space), so that they leave as whole contiguous rows below
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            const int r = 32 * rb + l32;
            const float l = ml_s[64 + r] + ml_s[128 + r];
            const float inv = (l > 0.f) ? 1.f / l : 0.f;
            char* orow = smem + r * kOutRow + 4 * (128 * v + 4 * g);
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    *reinterpret_cast<f32x4*>(orow + 4 * (32 * d + 8 * q4)) =
                        f32x4{acc[d][rb][4 * q4], acc[d][rb][4 * q4 + 1], acc[d][rb][4 * q4 + 2], acc[d][rb][4 * q4 + 3]} *
                        inv;
        }
    }
    __syncthreads();   // E3: the partial rows are in LDS
    // every wave stores whole rows: 16 B per lane, a wave writes 1 KiB of one row
    for (int e = tid; e < C::RW * (kDv / 4); e += C::THREADS) {
        const int r = e / (kDv / 4), c4 = e % (kDv / 4);
        const int row = row_base + r;
        if (row < a.rows)
            store_partial(o_part + (size_t)row * kDv + 4 * c4, *reinterpret_cast<const f32x4*>(smem + r * kOutRow + 16 * c4));
    }
}

}  // namespace mla
