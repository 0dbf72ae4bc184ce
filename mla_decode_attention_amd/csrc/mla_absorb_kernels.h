// Absorption and un-absorption around the decode path (the absorbed-MQA form: the up-projections
// are absorbed into the query and output projections so every head attends the latent cache
// directly, GQLA summary, section "Arquitetura", item 1).
//
// With a per-head no-RoPE dim of 128 (a reading: the pages give the latent and RoPE widths only):
//   absorb:    q[b,i,h,0:512]  = W_UK[h] q_nope[b,i,h]     (W_UK[h]: 512 x 128; q[..,512:576] = q_rope)
//   un-absorb: o[b,i,h,0:128]  = W_UV[h] O_lat[b,i,h]      (W_UV[h]: 128 x 512)
// Both are C[m][n] = sum_k A[m][k] W[n][k] per head with m the query token (b * s_q + i), W
// row-major [N][K]: a skinny product (M = b*s_q tokens) read once per weight byte, done with
// 16x16x32 bf16 MFMA tiles fed straight from global memory, fp32 accumulation, bf16 output
// rounded to nearest even.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_decode_kernels.h"

namespace mla {

constexpr int kDNope = 128;
constexpr int kAbsorbThreads = 256;   // 4 waves: one 16-column tile each, 64 columns per workgroup

struct HeadGemmArgs {
    const uint16_t* a;   // A[m][k] at a[m * lda + h * a_head + k]
    const uint16_t* w;   // W[n][k] at w[h * w_head + n * K + k]
    uint16_t* c;         // C[m][n] at c[m * ldc + h * c_head + n]
    long long lda, a_head, w_head, ldc, c_head;
    int M, N, K;
    // absorb only: q_rope[m][h][0:64] copied to c[m * ldc + h * c_head + 512 ..] (null = none)
    const uint16_t* rope;
    int heads;
};

// grid (heads, N / 64, ceil(M / 16)); wave w: rows 16 z .. 16 z + 15, columns 64 y + 16 w ..
__global__ void __launch_bounds__(kAbsorbThreads) head_gemm_kernel(HeadGemmArgs g)
{
    const int h = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int m = blockIdx.z * 16 + lr;                 // A row this lane feeds
    const int n = blockIdx.y * 64 + wave * 16 + lr;     // W row (C column) this lane feeds
    const bool m_ok = m < g.M;
    const uint16_t* arow = g.a + (size_t)(m_ok ? m : 0) * g.lda + (size_t)h * g.a_head + 8 * lg;
    const uint16_t* wrow = g.w + (size_t)h * g.w_head + (size_t)n * g.K + 8 * lg;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < g.K; k0 += 32) {
        bf16x8 av = m_ok ? *reinterpret_cast<const bf16x8*>(arow + k0) : bf16x8{};
        const bf16x8 wv = *reinterpret_cast<const bf16x8*>(wrow + k0);
        // D[row = token][col = n]: A = tokens x k, B = k x columns
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, wv, acc, 0, 0, 0);
    }
    // D layout: lane (lr, lg) holds D[4 lg + i][lr]: token 16 z + 4 lg + i, column n
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int mo = blockIdx.z * 16 + 4 * lg + i;
        if (mo < g.M) g.c[(size_t)mo * g.ldc + (size_t)h * g.c_head + n] = f32_to_bf16_rne(acc[i]);
    }
    // absorb: the RoPE part travels unchanged into dims 512..575 of the absorbed query
    if (g.rope && blockIdx.y == 0) {
        for (int e = threadIdx.x; e < 16 * (kDk - kDv) / 8; e += kAbsorbThreads) {
            const int r = e / ((kDk - kDv) / 8), c8 = e % ((kDk - kDv) / 8);
            const int mo = blockIdx.z * 16 + r;
            if (mo < g.M)
                *reinterpret_cast<i32x4*>(g.c + (size_t)mo * g.ldc + (size_t)h * g.c_head + kDv + 8 * c8) =
                    *reinterpret_cast<const i32x4*>(g.rope + ((size_t)mo * g.heads + h) * (kDk - kDv) + 8 * c8);
        }
    }
}

}  // namespace mla
