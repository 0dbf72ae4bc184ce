/*
 * A plain C client of the decode library: no Python, no torch.  It reads the inputs of one decode
 * step from raw files, runs mla_decode_workspace_size, mla_decode_plan and mla_decode_fwd on the
 * default stream through include/mla_decode.h alone, and writes O and LSE back as raw files.
 * Test infrastructure for tests/test_gpu_c_client.py; it holds none of the method's arithmetic.
 *
 * usage: decode_from_c DIR batch s_q heads num_pages bt_stride softmax_scale causal
 *   DIR/q.bin        bf16  [batch][s_q][heads][576]
 *   DIR/cache.bin    bf16  [num_pages][64][576]
 *   DIR/bt.bin       int32 [batch][bt_stride]
 *   DIR/seqlens.bin  int32 [batch]
 * writes DIR/out.bin (bf16 [batch][s_q][heads][512]) and DIR/lse.bin (fp32 [batch][s_q][heads]).
 * Exit status 0 on success; on failure the failing call and its status are printed.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mla_decode.h"

static void* read_file(const char* dir, const char* name, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) return NULL;
    void* p = malloc(bytes ? bytes : 1);
    const size_t got = p ? fread(p, 1, bytes, f) : 0;
    fclose(f);
    if (got != bytes) {
        free(p);
        return NULL;
    }
    return p;
}

static int write_file(const char* dir, const char* name, const void* p, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    if (!f) return -1;
    const size_t put = fwrite(p, 1, bytes, f);
    fclose(f);
    return put == bytes ? 0 : -1;
}

#define HIP_OK(call)                                                             \
    do {                                                                         \
        hipError_t e_ = (call);                                                  \
        if (e_ != hipSuccess) {                                                  \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));    \
            return 2;                                                            \
        }                                                                        \
    } while (0)

#define MLA_OK_(call)                                                                      \
    do {                                                                                   \
        int s_ = (call);                                                                   \
        if (s_ != MLA_OK) {                                                                \
            fprintf(stderr, "%s returned %d (%s)\n", #call, s_, mla_decode_status_string(s_)); \
            return 3;                                                                      \
        }                                                                                  \
    } while (0)

int main(int argc, char** argv)
{
    if (argc != 9) {
        fprintf(stderr, "usage: %s DIR batch s_q heads num_pages bt_stride softmax_scale causal\n", argv[0]);
        return 1;
    }
    const char* dir = argv[1];
    const int batch = atoi(argv[2]), s_q = atoi(argv[3]), heads = atoi(argv[4]);
    const int num_pages = atoi(argv[5]), bt_stride = atoi(argv[6]);
    const float scale = (float)atof(argv[7]);
    const int causal = atoi(argv[8]);
    if (batch < 1 || s_q < 1 || heads < 1 || num_pages < 1 || bt_stride < 1) return 1;

    const size_t rows = (size_t)batch * s_q * heads;
    const size_t q_bytes = rows * MLA_DECODE_D_K * 2;
    const size_t cache_bytes = (size_t)num_pages * MLA_DECODE_PAGE_SIZE * MLA_DECODE_D_K * 2;
    const size_t bt_bytes = (size_t)batch * bt_stride * 4;
    const size_t sl_bytes = (size_t)batch * 4;
    const size_t out_bytes = rows * MLA_DECODE_D_V * 2;
    const size_t lse_bytes = rows * 4;

    void* h_q = read_file(dir, "q.bin", q_bytes);
    void* h_cache = read_file(dir, "cache.bin", cache_bytes);
    void* h_bt = read_file(dir, "bt.bin", bt_bytes);
    void* h_sl = read_file(dir, "seqlens.bin", sl_bytes);
    void* h_out = malloc(out_bytes);
    void* h_lse = malloc(lse_bytes);
    if (!h_q || !h_cache || !h_bt || !h_sl || !h_out || !h_lse) {
        fprintf(stderr, "cannot read the inputs in %s\n", dir);
        return 1;
    }

    void *d_q, *d_cache, *d_bt, *d_sl, *d_out, *d_lse, *d_ws;
    HIP_OK(hipMalloc(&d_q, q_bytes));
    HIP_OK(hipMalloc(&d_cache, cache_bytes));
    HIP_OK(hipMalloc(&d_bt, bt_bytes));
    HIP_OK(hipMalloc(&d_sl, sl_bytes));
    HIP_OK(hipMalloc(&d_out, out_bytes));
    HIP_OK(hipMalloc(&d_lse, lse_bytes));
    HIP_OK(hipMemcpy(d_q, h_q, q_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_cache, h_cache, cache_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_bt, h_bt, bt_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_sl, h_sl, sl_bytes, hipMemcpyHostToDevice));

    size_t ws_bytes = 0;
    MLA_OK_(mla_decode_workspace_size(batch, s_q, heads, &ws_bytes));
    HIP_OK(hipMalloc(&d_ws, ws_bytes));   /* hipMalloc returns 256-byte aligned memory */
    MLA_OK_(mla_decode_plan((const int32_t*)d_sl, batch, s_q, heads, d_ws, ws_bytes, NULL));
    MLA_OK_(mla_decode_fwd(d_q, d_cache, (const int32_t*)d_bt, bt_stride, (const int32_t*)d_sl, batch, s_q, heads,
                           num_pages, MLA_DECODE_PAGE_SIZE, scale, causal, d_ws, ws_bytes, d_out, (float*)d_lse, NULL));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(h_out, d_out, out_bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_lse, d_lse, lse_bytes, hipMemcpyDeviceToHost));
    if (write_file(dir, "out.bin", h_out, out_bytes) || write_file(dir, "lse.bin", h_lse, lse_bytes)) {
        fprintf(stderr, "cannot write the outputs in %s\n", dir);
        return 1;
    }
    hipFree(d_q);
    hipFree(d_cache);
    hipFree(d_bt);
    hipFree(d_sl);
    hipFree(d_out);
    hipFree(d_lse);
    hipFree(d_ws);
    free(h_q);
    free(h_cache);
    free(h_bt);
    free(h_sl);
    free(h_out);
    free(h_lse);
    printf("decode_from_c: %d sequences, %d query tokens, %d heads: ok\n", batch, s_q, heads);
    return 0;
}
