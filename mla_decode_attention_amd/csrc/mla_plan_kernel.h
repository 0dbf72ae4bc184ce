// gfx950 plan kernel of the absorbed-MLA decode: the balanced split of every sequence's pages
// into work items for the split kernels (written to the workspace header and item array).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_decode_kernels.h"

namespace mla {

// =============================================================================================
// Plan: balanced split of every sequence's pages into at most `gx + batch` work items.
// One workgroup.  A sequence of p pages gets ceil(p / chunk) items of at most `chunk` pages; the
// chunk is the smallest one whose item count fits the gx resident workgroup slots of the split
// kernel (one wave of workgroups: with uneven lengths, ceil(total / gx) rounds up to a few items
// more than gx, and those would run as a second wave).  With batch >= gx every sequence is one
// item.
// =============================================================================================
constexpr int kPlanThreads = 1024;
constexpr long long kEvenXcdWeight = 16;   // relative work of an item on an even XCD
constexpr long long kOddXcdWeight = 15;    // ... and on an odd one (see the plan kernel)
constexpr long long kWeightMinPages = 8192; // plans this large stream from HBM (>= 604 MB of rows)
constexpr int kPlanCache = 4;               // sequences per thread whose page counts stay in registers

// no L + 63 (which overflows int for L within 63 of INT_MAX)
__device__ inline int pages_of(int L) { return L <= 0 ? 0 : L / kPage + (L % kPage != 0 ? 1 : 0); }

// uniform_len >= 0: every sequence has that length and `seqlens` is not read (sparse decode: each
// query token is a sequence of top-k index slots).  force_chunk > 0: items of at most that many
// pages, unless their count would exceed the workspace's capacity (then the automatic chunk)
__global__ void __launch_bounds__(kPlanThreads) plan_kernel(const int32_t* __restrict__ seqlens, int batch,
                                                            int s_q, int heads, int rows, int gx,
                                                            int capacity, char* __restrict__ ws, int uniform_len,
                                                            int force_chunk = 0)
{
    auto len_of = [&](int b) { return uniform_len >= 0 ? uniform_len : seqlens[b]; };
    const WsLayout lay = ws_layout(batch, rows, capacity);
    int32_t* header = reinterpret_cast<int32_t*>(ws + lay.header);
    int32_t* ws_len = reinterpret_cast<int32_t*>(ws + lay.seqlens);
    int32_t* bsplit = reinterpret_cast<int32_t*>(ws + lay.batch_split);
    i32x4* items = reinterpret_cast<i32x4*>(ws + lay.items);

    __shared__ long long red[kPlanThreads / 64];
    __shared__ int scan_carry;
    __shared__ int wave_tot[kPlanThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;

    // page counts, read once: the first kPlanCache * kPlanThreads sequences' counts stay in
    // registers for the passes below (each pass would otherwise wait on a memory round trip)
    int pg_c[kPlanCache];
    long long mine = 0;
#pragma unroll
    for (int i = 0; i < kPlanCache; ++i) {
        const int b = tid + i * kPlanThreads;
        int p = 0;
        if (b < batch) {
            const int L = len_of(b);
            ws_len[b] = L;
            p = pages_of(L);
        }
        pg_c[i] = p;
        mine += p;
    }
    for (int b = tid + kPlanCache * kPlanThreads; b < batch; b += kPlanThreads) {
        const int L = len_of(b);
        ws_len[b] = L;
        mine += pages_of(L);
    }
    // f(pages) summed over this thread's sequences
    auto sum_pages = [&](auto f) {
        long long n = 0;
#pragma unroll
        for (int i = 0; i < kPlanCache; ++i) n += f(pg_c[i]);   // 0 pages for b >= batch: f(0) == 0 below
        for (int b = tid + kPlanCache * kPlanThreads; b < batch; b += kPlanThreads) n += f(pages_of(len_of(b)));
        return n;
    };
    // block-wide sum (every thread gets it); two barriers so that red[] can be reused
    auto block_sum = [&](long long v) {
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
        __syncthreads();
        if (lane == 0) red[wid] = v;
        __syncthreads();
        long long t = 0;
        for (int w = 0; w < kPlanThreads / 64; ++w) t += red[w];
        return t;
    };
    if (tid == 0) scan_carry = 0;
    const long long total = block_sum(mine);
    // (chunks are at most 2^25 pages: 32-bit divisions)
    auto items_for = [&](long long c) {
        const int c32 = (int)c;
        return block_sum(sum_pages([&](int pg) { return (long long)((pg + c32 - 1) / c32); }));
    };
    const long long slots = gx > 0 ? gx : 1;
    long long chunk;
    if (slots > batch) {
        // items(c) <= total / c + batch, so c = ceil(total / (slots - batch)) always fits
        long long lo = (total + slots - 1) / slots, hi = (total + (slots - batch) - 1) / (slots - batch);
        if (lo < 1) lo = 1;
        if (hi < lo) hi = lo;
        while (lo < hi) {   // uniform across the workgroup: every thread takes the same branch
            const long long mid = (lo + hi) / 2;
            if (items_for(mid) <= slots)
                hi = mid;
            else
                lo = mid + 1;
        }
        chunk = lo;
    } else {
        long long mx = 0;
#pragma unroll
        for (int i = 0; i < kPlanCache; ++i) mx = max(mx, (long long)pg_c[i]);
        for (int b = tid + kPlanCache * kPlanThreads; b < batch; b += kPlanThreads)
            mx = max(mx, (long long)pages_of(len_of(b)));
        for (int o = 32; o > 0; o >>= 1) mx = max(mx, __shfl_xor(mx, o));
        __syncthreads();
        if (lane == 0) red[wid] = mx;
        __syncthreads();
        for (int w = 0; w < kPlanThreads / 64; ++w) mx = max(mx, red[w]);
        chunk = mx;
    }
    if (chunk < 1) chunk = 1;
    // a caller-chosen chunk replaces the automatic one when its items fit the workspace
    if (force_chunk > 0 && items_for(force_chunk) <= capacity) chunk = force_chunk;

    // per-sequence split counts, exclusive prefix sum in blocks of kPlanThreads
    auto block_items = [&](int base, int pg) __attribute__((always_inline)) {
        const int b = base + tid;
        const int n = b < batch ? int((pg + chunk - 1) / chunk) : 0;
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
            // Item x runs on XCD x % 8 (workgroups go round robin over the XCDs; the wide form keeps
            // that by giving an item's row groups ids 8 apart).  On MI355X the odd XCDs stream this
            // access pattern from HBM ~4-9 % slower than the even ones (measured on five GPUs, every
            // one the same way round), so when the plan's pages clearly exceed the 256 MB
            // last-level cache (kWeightMinPages) and items have 8 pages or more, an item on an odd
            // XCD gets weight kOddXcdWeight against kEvenXcdWeight on an even one.  (Where the keys
            // fit the cache the asymmetry does not show, and the weighting only lengthened the
            // largest items.)  Deterministic: the split points depend only on the lengths.
            const bool weighted = total >= kWeightMinPages && (long long)pg >= 8LL * n;
            const int ev0 = (excl & 1) == 0 ? 1 : 0;   // item excl + s is even for s of this parity
            // floor(a * b / c) in double precision: a * b < 2^53 is exact, the quotient is below
            // 2^25, where doubles are 2^-28 apart, and a non-integer quotient is at least 1/c > 2^-27
            // from the next integer, so the correctly rounded division floors to the exact result
            // (an integer division of 64 bits would be a long software sequence per item)
            auto muldiv = [](long long a, long long b, long long c) { return int(floor(double(a * b) / double(c))); };
            auto point = [&](int s) {
                if (!weighted) return muldiv(s, pg, n);   // s * pg <= pg^2 < 2^50
                const long long e = (s + ev0) / 2;   // even items among the first s
                const long long w = kEvenXcdWeight * e + kOddXcdWeight * (s - e);
                const long long en = (n + ev0) / 2;
                const long long wt = kEvenXcdWeight * en + kOddXcdWeight * (n - en);
                return muldiv(pg, w, wt);   // weighted: n <= pg / 8, so pg * w <= 2 pg^2 < 2^51
            };
            for (int s = 0; s < n; ++s) items[excl + s] = i32x4{b, point(s), point(s + 1), s};
        }
        __syncthreads();
        if (tid == kPlanThreads - 1) scan_carry = excl + n;
        __syncthreads();
    };
#pragma unroll
    for (int i = 0; i < kPlanCache; ++i)
        if (i * kPlanThreads < batch) block_items(i * kPlanThreads, pg_c[i]);   // uniform branch
    for (int base = kPlanCache * kPlanThreads; base < batch; base += kPlanThreads)
        block_items(base, base + tid < batch ? pages_of(len_of(base + tid)) : 0);
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

}  // namespace mla
