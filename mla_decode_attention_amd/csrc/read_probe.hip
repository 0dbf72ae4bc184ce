// Streaming-read bandwidth probe.  Measurement context only: it is built into its own library
// (libmla_read_probe.so), which bench.py loads to put the decode kernels' rates beside what a
// plain read of HBM reaches on the same GPU in the same run.  It is not part of the decode
// library's C ABI.
//
// Every wave reads whole 18 KiB chunks (eighteen 1 KiB units, 16 B per lane, non-temporal),
// two chunks in flight (ping-pong register sets), and folds them into one word per thread so
// the loads stay live.  Loads past the buffer go through an empty buffer resource and return
// zeros, so every load is issued on every path and each fold waits for its own chunk only.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int kUnits = 18;
constexpr long long kChunk = kUnits * 1024;
constexpr int kThreads = 256;
constexpr int kBlocksPerCu = 2;       // the kernel takes ~231 VGPRs: two 4-wave blocks per CU

__device__ inline void load_chunk(i32x4 (&v)[kUnits], const char* buf, long long ch, long long chunks, int lane)
{
    const bool ok = ch < chunks;
    const char* base = buf + (ok ? ch : 0) * kChunk;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, ok ? (int)kChunk : 0, 0x00020000);
#pragma unroll
    for (int j = 0; j < kUnits; ++j) v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16, j * 1024, 2);
}

__device__ inline void fold(i32x4& acc, const i32x4 (&v)[kUnits])
{
#pragma unroll
    for (int j = 0; j < kUnits; ++j) acc ^= v[j];
}

__global__ void __launch_bounds__(kThreads) read_probe_kernel(const char* __restrict__ buf, long long chunks,
                                                               int* __restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const long long stride = (long long)gridDim.x * (kThreads / 64);
    long long c = (long long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    i32x4 acc = {0, 0, 0, 0};
    i32x4 a[kUnits], b[kUnits];
    load_chunk(a, buf, c, chunks, lane);
    for (; c < chunks; c += 2 * stride) {
        load_chunk(b, buf, c + stride, chunks, lane);
        fold(acc, a);
        load_chunk(a, buf, c + 2 * stride, chunks, lane);
        fold(acc, b);
    }
    fold(acc, a);   // the last loads in flight (zeros past the end)
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

// Reads `bytes` (rounded down to whole 18 KiB chunks) of device buffer `buf` once.  `out` is a
// device buffer of `out_words` int32 the kernel writes (one word per thread; its content is
// meaningless).  Returns 0 on success, -1 on bad arguments (nothing launched: null pointers, or
// `out_words` below what mla_read_probe_out_words() returns), or the HIP error code of the launch.
extern "C" int mla_read_probe_out_words(void)
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return -1;
    return cus * kBlocksPerCu * kThreads;
}

extern "C" int mla_read_probe(const void* buf, long long bytes, int* out, long long out_words, void* stream)
{
    const int need = mla_read_probe_out_words();
    if (buf == nullptr || out == nullptr || bytes < kChunk || need < 0 || out_words < need) return -1;
    const int blocks = need / kThreads;
    hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                       (const char*)buf, bytes / kChunk, out);
    return (int)hipGetLastError();
}
