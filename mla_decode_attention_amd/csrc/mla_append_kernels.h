// Paged cache append with rotary position embedding of the shared RoPE key, for the s_q new
// tokens of a decode step (the step that feeds the decode path: the latent cache row of MLA's
// absorbed form is the latent plus one shared RoPE key, GQLA summary, section "Arquitetura").
//
// For sequence b and new token i the position is pos = L_b - s_q + i.  The token's cache row
// (page block_table[b][pos / 64], slot pos % 64) receives the 512-d latent unchanged and the
// 64-d RoPE key rotated by pos; the 64-d RoPE part of every head of the token's query is
// rotated by pos in place.  Rotation: dims (2p, 2p+1) of the 64-d part turn by the angle
// pos * base^(-2p/64), p = 0..31 (the rotary embedding in its original pairwise form; the pages
// name the RoPE key without giving its formula).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_decode_kernels.h"

namespace mla {

constexpr int kRopeDim = kDk - kDv;     // 64
constexpr int kAppendThreads = 256;

struct AppendArgs {
    const uint16_t* kv_latent;   // bf16 [b][s_q][512]
    const uint16_t* k_rope;      // bf16 [b][s_q][64], before rotation
    uint16_t* q;                 // bf16 [b][s_q][h][576], RoPE part rotated in place
    uint16_t* cache;             // bf16 [num_pages][64][576]
    const int32_t* block_table;  // int32 [b][bt_stride]
    const int32_t* seqlens;      // int32 [b], counting the s_q new tokens
    long long num_pages;
    int bt_stride, batch, s_q, heads;
    double log2_base;            // log2 of the rotary base
};

__device__ inline double bf16_bits_to_double(uint16_t h) { return (double)__uint_as_float((uint32_t)h << 16); }

// fp64 -> bf16, round to nearest even, in one rounding: the fp32 step rounds toward zero and
// marks any discarded bits in its last place (round to odd), which keeps the final rounding
// correct because fp32 carries 16 more mantissa bits than bf16.
__device__ inline uint16_t double_to_bf16_rne(double d)
{
    float f = __double2float_rz(d);
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u || d != d) return 0x7fc0;
    if ((double)f != d && (u & 0x7f800000u) != 0x7f800000u) u |= 1u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// rotate the bf16 pair src[0], src[1] by the angle whose cosine and sine are c, s
__device__ inline void rope_pair(const uint16_t* src, uint16_t* dst, double c, double s)
{
    const double x = bf16_bits_to_double(src[0]);
    const double y = bf16_bits_to_double(src[1]);
    dst[0] = double_to_bf16_rne(x * c - y * s);
    dst[1] = double_to_bf16_rne(x * s + y * c);
}

// One workgroup per new token (b, i).
__global__ void __launch_bounds__(kAppendThreads) append_rope_kernel(AppendArgs a)
{
    __shared__ double cs[kRopeDim / 2][2];   // cos, sin of the token's angle for each pair
    const int tok = blockIdx.x;   // b * s_q + i
    const int b = tok / a.s_q;
    const int i = tok % a.s_q;
    const int t = threadIdx.x;
    const int L = a.seqlens[b];
    const int pos = L - a.s_q + i;
    bool ok = pos >= 0 && (long long)L <= (long long)kPage * a.bt_stride;
    int page = -1;
    if (ok) {
        page = a.block_table[(size_t)b * a.bt_stride + pos / kPage];
        ok = page >= 0 && (long long)page < a.num_pages;
    }
    if (ok && t < kRopeDim / 2) {
        const double theta = exp2(-(2.0 * t / kRopeDim) * a.log2_base);
        double s, c;
        sincos((double)pos * theta, &s, &c);
        cs[t][0] = c;
        cs[t][1] = s;
    }
    __syncthreads();
    if (ok) {
        uint16_t* row = a.cache + ((size_t)page * kPage + pos % kPage) * kDk;
        if (t < kDv / 8) {   // latent: 64 x 16 B
            *reinterpret_cast<i32x4*>(row + 8 * t) = *reinterpret_cast<const i32x4*>(a.kv_latent + (size_t)tok * kDv + 8 * t);
        } else if (t < kDv / 8 + kRopeDim / 2) {
            const int p = t - kDv / 8;
            rope_pair(a.k_rope + (size_t)tok * kRopeDim + 2 * p, row + kDv + 2 * p, cs[p][0], cs[p][1]);
        }
    }
    // the query's RoPE part of every head; NaN when the token has no valid cache slot, so the
    // decode that follows reports the sequence as NaN
    for (int e = t; e < a.heads * (kRopeDim / 2); e += kAppendThreads) {
        const int h = e / (kRopeDim / 2);
        const int p = e % (kRopeDim / 2);
        uint16_t* qr = a.q + ((size_t)tok * a.heads + h) * kDk + kDv + 2 * p;
        if (ok) {
            uint16_t r[2];
            rope_pair(qr, r, cs[p][0], cs[p][1]);
            qr[0] = r[0];
            qr[1] = r[1];
        } else {
            qr[0] = 0x7fc0;
            qr[1] = 0x7fc0;
        }
    }
}

}  // namespace mla
