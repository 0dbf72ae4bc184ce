// GQA-path decode of GQLA (GQLA summary, section "Arquitetura", item 2: the latent is expanded into
// g groups of keys and values, and decode runs standard grouped-query attention; the cache holds the
// per-group keys and values plus the shared RoPE key).  One GPU's share is one group: 16 query heads
// (h_q / g = 16) over that group's cache.  Readings (the pages give neither): per-group key and value
// width d_h = 128; one 640-B cache row per token, [k (128) | shared RoPE key (64) | v (128)].
//
// For sequence b, query token i < s_q and head h < 16, with n visible rows j (n = L_b, or
// L_b - s_q + 1 + i when causal):
//     s_j = scale * dot(q[b,i,h,0:192], row_j[0:192]),  LSE = ln sum_j exp(s_j),
//     O   = sum_j exp(s_j - LSE) * row_j[192:320].
//
// Kernel: the 16-row-block kernel's scheme at this geometry.  Four independent waves per workgroup
// each take every 4th 16-token tile of a work item (HBM -> VGPR -> the wave's own LDS stage, rows
// padded to 672 B), hold Q^T of all s_q * 16 rows in registers, and compute S^T = K Q^T with
// 16x16x32 MFMAs (two partial chains per row block), a lazily rescaled online softmax and
// O^T += V^T P^T with 16x16x16 MFMAs (V^T read transposed from the rows in LDS).  The four waves
// merge their (m, l, O) in LDS; split-KV partials go to the workspace for the LSE combine.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_decode_kernels.h"

namespace mla {

constexpr int kGqaDh = 128;                      // per-group key / value width
constexpr int kGqaDk = kGqaDh + (kDk - kDv);     // 192: key = group key + shared RoPE key
constexpr int kGqaDv = kGqaDh;                   // 128
constexpr int kGqaRow = kGqaDk + kGqaDv;         // 320 bf16 per cache row
constexpr int kGqaRowBytes = kGqaRow * 2;        // 640
constexpr int kGqaChunks = kGqaRowBytes / 16;    // 40 16-B chunks per row
constexpr int kGqaLdsRow = kGqaRowBytes + 32;    // 672: K-operand reads hit distinct banks
constexpr int kGqaKSteps = kGqaDk / 32;          // 6
constexpr int kGqaDTiles = kGqaDv / 16;          // 8
constexpr int kGqaTT = 16;                       // tokens per tile
constexpr int kGqaUnits = kGqaTT * kGqaRowBytes / 1024;   // 10 1-KiB load units per tile
constexpr int kGqaWaves = 4;
constexpr int kGqaHeads = 16;
constexpr int kGqaThreads = kGqaWaves * 64;

template <int NRB_, int NR_>   // NRB: 16-row blocks per wave = query tokens per sequence (s_q)
struct GqaCfg {
    static constexpr int NRB = NRB_;
    static constexpr int NR = NR_;   // tiles in flight in registers per wave
    static constexpr int STAGE = kGqaTT * kGqaLdsRow;                                   // 10,752 B
    static constexpr int MERGE = kGqaWaves * NRB * 16 * (2 + kGqaDv) * 4;               // m, l, O per wave
    static constexpr int LDS_BYTES = kGqaWaves * STAGE > MERGE ? kGqaWaves * STAGE : MERGE;
    static_assert(NRB == 1 || NRB == 2, "one or two query tokens");
    static_assert(NR == 1 || NR == 2, "one or two tiles in flight per wave");
};

template <class C>
__global__ void __launch_bounds__(kGqaThreads) gqa_split_kernel(FwdArgs a)
{
    constexpr int NRB = C::NRB;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15;
    const int lg = lane >> 4;

    const WsLayout lay = ws_layout(a.batch, a.rows, a.capacity, kGqaDv);
    // the arguments of the prologue's address computations come in with the first ones
    asm volatile("" ::"s"(a.q), "s"(a.block_table), "s"(a.seqlens), "s"(a.bt_stride));
    const int item = blockIdx.x;
    const PlanItem pi = read_plan_item(a, lay, item);
    if (!pi.ok) return;   // a plan mismatch is reported by the combine kernel
    const i32x4 it = pi.it;
    const int b = it[0];
    // the first block-table window, the lengths and Q go out together (one round trip)
    PageWindow pw;
    pw.init(a.block_table + (size_t)b * a.bt_stride, a.bt_stride);
    pw.prefetch(it[1], lane);
    const int L = a.seqlens[b];
    const int32_t plan_L = reinterpret_cast<const int32_t*>(a.ws + lay.seqlens)[b];
    float* lse_part = reinterpret_cast<float*>(a.ws + lay.lse_part) + (size_t)item * a.rows;
    float* o_part = reinterpret_cast<float*>(a.ws + lay.o_part) + (size_t)item * a.rows * kGqaDv;
    // A sequence whose length disagrees with the plan or the table gets no tiles and a NaN LSE
    // (no early exit: a branch here would make the loads above wait one after another).
    const bool bad_seq = (L != plan_L) | (L < 0) | ((long long)L > (long long)kPage * a.bt_stride);
    const int tok_begin = it[1] * kPage;
    const int tok_end = (int)min((long long)it[2] * kPage, (long long)L);   // it[2] * 64 may reach 2^31
    const int n_tiles = bad_seq ? 0 : (tok_end - tok_begin + kGqaTT - 1) / kGqaTT;
    const int n_it = (n_tiles + kGqaWaves - 1) / kGqaWaves;
    int n_vis[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) n_vis[rb] = a.causal ? min(max(L - a.s_q + 1 + rb, 0), L) : L;

    // Q^T (B of the score MFMA): row block rb = query token rb, lane (row lr, group lg) holds
    // q[token rb][head lr][32 j + 8 lg .. + 8]
    bf16x8 qop[NRB][kGqaKSteps];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        const uint16_t* qrow = a.q + ((size_t)(b * a.s_q + rb) * kGqaHeads + lr) * kGqaDk;
#pragma unroll
        for (int j = 0; j < kGqaKSteps; ++j) qop[rb][j] = *reinterpret_cast<const bf16x8*>(qrow + 32 * j + 8 * lg);
    }

    // tiles: wave w takes tiles w, w + 4, ...; lane l of unit u moves 16-B chunk 64 u + l of the
    // tile (row (64 u + l) / 40) into the wave's own stage
    const uint32_t lane16 = (uint32_t)lane * 16u;
    char* const stage = smem + wave * C::STAGE;
    bool bad_page = bad_seq;
    i32x4 rbuf[C::NR][kGqaUnits];
    auto load_tile = [&](int itn, auto buf_idx) __attribute__((always_inline)) {
        constexpr int B = decltype(buf_idx)::value;
        const int k = itn * kGqaWaves + wave;
        if (itn >= n_it || k >= n_tiles) return;
        const int t0 = tok_begin + k * kGqaTT;
        const int page = pw.page(t0 / kPage, lane);
        int valid = min(kGqaTT, L - t0);
        if (page < 0 || (long long)page >= a.num_pages) {
            bad_page = true;
            valid = 0;
        }
        const uint16_t* base = a.cache + ((long long)(valid ? page : 0) * kPage + (t0 % kPage)) * kGqaRow;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, valid * kGqaRowBytes, 0x00020000);
#pragma unroll
        for (int kk = 0; kk < kGqaUnits; ++kk)
            rbuf[B][kk] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)lane16, kk * 1024, kNonTemporal);
    };
    auto store_tile = [&](int itn, auto buf_idx) __attribute__((always_inline)) {
        constexpr int B = decltype(buf_idx)::value;
        const int k = itn * kGqaWaves + wave;
        if (itn >= n_it || k >= n_tiles) return;
#pragma unroll
        for (int kk = 0; kk < kGqaUnits; ++kk) {
            const int c = 64 * kk + lane;
            const int r = c / kGqaChunks;
            *reinterpret_cast<i32x4*>(stage + r * kGqaLdsRow + 16 * (c - r * kGqaChunks)) = rbuf[B][kk];
        }
    };

    f32x4 acc[kGqaDTiles][NRB];   // acc[dt][rb]: O^T[16 dt + 4 lg + i][row lr of block rb]
#pragma unroll
    for (int dt = 0; dt < kGqaDTiles; ++dt)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) acc[dt][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[NRB], l_run[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        m_run[rb] = -__builtin_inff();
        l_run[rb] = 0.f;
    }
    constexpr float kLazyRescale = 8.f;
    const int kbase = lr * kGqaLdsRow + 16 * lg;
    const int vbase = (4 * lg + (lr >> 2)) * kGqaLdsRow + 8 * (lr & 3) + 2 * kGqaDk;

    auto compute_tile = [&](int k) __attribute__((always_inline)) {
        const int t0 = tok_begin + k * kGqaTT;
        // S^T[token][row]: two partial chains per row block
        f32x4 sp[NRB][2];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) sp[rb][0] = sp[rb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        bf16x8 kop[kGqaKSteps];
#pragma unroll
        for (int j = 0; j < kGqaKSteps; ++j) kop[j] = *reinterpret_cast<const bf16x8*>(stage + kbase + 64 * j);
        i16x4 vop[kGqaDTiles];
#pragma unroll
        for (int j = 0; j < kGqaKSteps; ++j) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
                sp[rb][j & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[j], qop[rb][j], sp[rb][j & 1], 0, 0, 0);
        }
        // V^T operands (A of the value MFMA) do not depend on P: issue them now
#pragma unroll
        for (int dt = 0; dt < kGqaDTiles; ++dt)
            vop[dt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)lds_i16x4(stage + vbase + 32 * dt));
        bf16x4 pop[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            f32x4 s = (sp[rb][0] + sp[rb][1]) * a.scale_log2;
            if (t0 + kGqaTT > n_vis[rb]) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (t0 + 4 * lg + i >= n_vis[rb]) s[i] = -__builtin_inff();
            }
            float tmax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
            tmax = wave_max_groups(tmax);
            if (__builtin_amdgcn_ballot_w64(tmax > m_run[rb] + kLazyRescale) != 0) {
                const float m_new = fmaxf(m_run[rb], tmax);
                const float alpha = (m_new == -__builtin_inff()) ? 1.f : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
                m_run[rb] = m_new;
                l_run[rb] *= alpha;
#pragma unroll
                for (int dt = 0; dt < kGqaDTiles; ++dt) acc[dt][rb] *= alpha;
            }
            const float m_use = (m_run[rb] == -__builtin_inff()) ? 0.f : m_run[rb];
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = __builtin_amdgcn_exp2f(s[i] - m_use);
                psum += p;
                pop[rb][i] = (__bf16)p;
            }
            l_run[rb] += psum;
        }
        // O^T[d][row] += V^T[d][token] P^T[token][row]
#pragma unroll
        for (int dt = 0; dt < kGqaDTiles; ++dt)
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
                acc[dt][rb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, vop[dt]), pop[rb],
                                                                       acc[dt][rb], 0, 0, 0);
    };

    // pipeline: tiles itn+1 .. itn+NR wait in registers while tile itn is computed from the stage;
    // then tile itn+1 is stored to the stage and its registers take tile itn+1+NR
    load_tile(0, Idx<0>{});
    if constexpr (C::NR == 2) load_tile(1, Idx<1>{});
    store_tile(0, Idx<0>{});
    load_tile(C::NR, Idx<0>{});
    // Consume Q here, so that no wait for it lands inside the tile loop (where it would also wait
    // for the tile loads in flight)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int j = 0; j < kGqaKSteps; ++j) asm volatile("" ::"v"(qop[rb][j]));
    auto step = [&](int itn, auto next_buf) __attribute__((always_inline)) {
        if (itn >= n_it) return;
        const int k = itn * kGqaWaves + wave;
        if (k < n_tiles) compute_tile(k);
        store_tile(itn + 1, next_buf);
        load_tile(itn + 1 + C::NR, next_buf);
    };
    if constexpr (C::NR == 2) {
        for (int itn = 0; itn < n_it; itn += 2) {
            step(itn, Idx<1>{});
            step(itn + 1, Idx<0>{});
        }
    } else {
        for (int itn = 0; itn < n_it; ++itn) step(itn, Idx<0>{});
    }
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) l_run[rb] = wave_sum_groups(l_run[rb]);

    // ---- merge the four waves' (m, l, O) of every row and write the item's partials
    __syncthreads();   // every wave is done with its stage
    float* ml = reinterpret_cast<float*>(smem);                                   // [wave][2][NRB*16]
    float* accs = reinterpret_cast<float*>(smem + kGqaWaves * 2 * NRB * 16 * 4);  // [wave][NRB*16][128]
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        if (lg == 0) {
            ml[(wave * 2 + 0) * NRB * 16 + rb * 16 + lr] = m_run[rb];
            ml[(wave * 2 + 1) * NRB * 16 + rb * 16 + lr] = bad_page ? __builtin_nanf("") : l_run[rb];
        }
        float* my = accs + ((size_t)wave * NRB * 16 + rb * 16 + lr) * kGqaDv;
#pragma unroll
        for (int dt = 0; dt < kGqaDTiles; ++dt) *reinterpret_cast<f32x4*>(my + 16 * dt + 4 * lg) = acc[dt][rb];
    }
    __syncthreads();
    for (int e = tid; e < NRB * 16 * (kGqaDv / 4); e += kGqaThreads) {
        const int d4 = e % (kGqaDv / 4);
        const int row = e / (kGqaDv / 4);   // rb * 16 + r
        float M = -__builtin_inff();
        for (int w = 0; w < kGqaWaves; ++w) M = fmaxf(M, ml[(w * 2) * NRB * 16 + row]);
        const float Mu = (M == -__builtin_inff()) ? 0.f : M;
        float Lsum = 0.f;
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
        bool nan = false;
        for (int w = 0; w < kGqaWaves; ++w) {
            const float lw = ml[(w * 2 + 1) * NRB * 16 + row];
            nan |= (lw != lw);
            const float sc = __builtin_amdgcn_exp2f(ml[(w * 2) * NRB * 16 + row] - Mu);
            Lsum += sc * lw;
            o += sc * *reinterpret_cast<const f32x4*>(accs + ((size_t)w * NRB * 16 + row) * kGqaDv + 4 * d4);
        }
        const float inv = (Lsum > 0.f) ? 1.f / Lsum : 0.f;
        store_partial(o_part + (size_t)row * kGqaDv + 4 * d4, o * inv);
        if (d4 == 0)
            lse_part[row] = nan ? __builtin_nanf("")
                                : (Lsum > 0.f ? (M + __builtin_amdgcn_logf(Lsum)) * kLn2 : -__builtin_inff());
    }
}

}  // namespace mla
