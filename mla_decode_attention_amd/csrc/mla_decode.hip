// Host side of the C ABI declared in include/mla_decode.h: argument validation (before any HIP
// call), per-device launch geometry, workspace sizing and the kernel launches.
#include "mla_decode.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "mla_absorb_kernels.h"
#include "mla_append_kernels.h"
#include "mla_gqa_kernels.h"
#include "mla_decode_kernels.h"
#include "mla_plan_kernel.h"
#include "mla_sv_kernel.h"

namespace {

using namespace mla;

// Launch configurations by query rows per sequence (s_q * heads).
// 16 rows: four independent waves per CU, each streaming its own 16-token tiles (the work per
// byte is small enough that one wave per SIMD keeps HBM busy).  32 rows and more: the
// eight-wave score/value form, whose two waves per SIMD overlap MFMA, LDS and vector work.
//                         waves  row-blocks  segments  tile tokens  LDS stages  register tiles
using CfgR16 = SplitCfg<4, 1, 1, 16, 1, 1>;    // 4 independent waves, one 18 KiB tile each
//                 32-row blocks
using CfgSV1 = SvCfg<1>;                       // 32 rows per workgroup
using CfgSV2 = SvCfg<2>;                       // 64 rows per workgroup (row groups of 64 above)

using CfgG1 = GqaCfg<1, 2>;                     // GQA path, one query token per step
using CfgG2 = GqaCfg<2, 2>;                     // GQA path, two query tokens per step

// kS16: sparse (gathered-row) form of kR16; kG1 / kG2: GQA path
enum CfgId { kR16 = 0, kS16, kG1, kG2, kSV1, kSV2, kNumCfg };

struct LaunchGeom {
    CfgId cfg;
    int row_groups;   // grid.y
    int threads;
    int lds_bytes;
};

bool geom_for(int s_q, int heads, LaunchGeom* g)
{
    const int rows = s_q * heads;
    if (rows == 16) {
        *g = {kR16, 1, CfgR16::THREADS, CfgR16::LDS_BYTES};
        return true;
    }
    if (rows % 16 != 0 || rows > 256) return false;
    if (rows == 32) {
        *g = {kSV1, 1, CfgSV1::THREADS, CfgSV1::LDS_BYTES};
        return true;
    }
    *g = {kSV2, (rows + 63) / 64, CfgSV2::THREADS, CfgSV2::LDS_BYTES};
    return true;
}

const void* split_fn(CfgId c)
{
    switch (c) {
    case kR16: return reinterpret_cast<const void*>(&split_kernel<CfgR16>);
    case kS16: return reinterpret_cast<const void*>(&split_kernel<CfgR16, true>);
    case kG1: return reinterpret_cast<const void*>(&gqa_split_kernel<CfgG1>);
    case kG2: return reinterpret_cast<const void*>(&gqa_split_kernel<CfgG2>);
    case kSV1: return reinterpret_cast<const void*>(&split_sv_kernel<CfgSV1>);
    default: return reinterpret_cast<const void*>(&split_sv_kernel<CfgSV2>);
    }
}

struct DeviceInfo {
    bool ready = false;
    int status = MLA_OK;
    int num_cu = 0;
    int occupancy[kNumCfg] = {};
};

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
DeviceInfo g_dev[kMaxDevices];

// Built-in workspace of mla_decode_fwd_noalloc (every GPU the library runs on holds its own copy
// until the process ends).  Host code never uses the array's name as an address: the device
// address comes from hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) char scratch[MLA_DECODE_NOALLOC_SCRATCH_BYTES];
void* g_scratch_ptr[kMaxDevices];
int g_scratch_status[kMaxDevices];
bool g_scratch_ready[kMaxDevices];

// the calling thread's current device's scratch address (nullptr on error)
int scratch_address(void** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return MLA_ERR_NO_DEVICE;
    }
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch_ready[dev]) {
        g_scratch_ready[dev] = true;
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            g_scratch_status[dev] = MLA_ERR_HIP;
        } else {
            g_scratch_ptr[dev] = ptr;
            g_scratch_status[dev] = MLA_OK;
        }
    }
    *out = g_scratch_ptr[dev];
    return g_scratch_status[dev];
}

int device_info(const DeviceInfo** out)
{
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        return MLA_ERR_NO_DEVICE;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return MLA_ERR_NO_DEVICE;
    }
    std::lock_guard<std::mutex> lock(g_mutex);
    DeviceInfo& d = g_dev[dev];
    if (!d.ready) {
        d.ready = true;
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            d.status = MLA_ERR_NO_DEVICE;
        } else if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
            d.status = MLA_ERR_NO_DEVICE;   // the code objects are built for gfx950 only
        } else {
            d.num_cu = prop.multiProcessorCount;
            const int threads[kNumCfg] = {CfgR16::THREADS, CfgR16::THREADS, kGqaThreads,
                                          kGqaThreads,     CfgSV1::THREADS, CfgSV2::THREADS};
            const int lds[kNumCfg] = {CfgR16::LDS_BYTES, CfgR16::LDS_BYTES, CfgG1::LDS_BYTES,
                                      CfgG2::LDS_BYTES,  CfgSV1::LDS_BYTES, CfgSV2::LDS_BYTES};
            for (int c = 0; c < kNumCfg; ++c) {
                const void* fn = split_fn(static_cast<CfgId>(c));
                int occ = 0;
                if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds[c]) != hipSuccess ||
                    hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, threads[c], lds[c]) != hipSuccess ||
                    occ < 1) {
                    (void)hipGetLastError();
                    d.status = MLA_ERR_HIP;
                    break;
                }
                d.occupancy[c] = occ;
            }
        }
    }
    *out = &d;
    return d.status;
}

bool batch_ok(int batch) { return batch >= 1 && batch <= MLA_DECODE_MAX_BATCH; }

bool heads_ok(int s_q, int heads)
{
    return (s_q == 1 || s_q == 2) && heads >= 16 && heads <= 128 && heads % 16 == 0;
}

// Work items the split kernel can take per row group: the plan makes at most one per resident
// workgroup slot, or one per sequence when the batch has at least as many sequences as slots.
int item_capacity(const DeviceInfo& d, const LaunchGeom& g, int batch)
{
    int gx = d.num_cu * d.occupancy[g.cfg] / g.row_groups;
    if (gx < 1) gx = 1;
    return gx + batch;
}

int gx_of(const DeviceInfo& d, const LaunchGeom& g)
{
    int gx = d.num_cu * d.occupancy[g.cfg] / g.row_groups;
    return gx < 1 ? 1 : gx;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

extern "C" {

int mla_decode_workspace_size(int batch, int s_q, int num_heads, size_t* bytes)
{
    if (!bytes || !batch_ok(batch)) return MLA_ERR_INVALID_ARG;
    if (!heads_ok(s_q, num_heads)) return MLA_ERR_UNSUPPORTED;
    const DeviceInfo* d = nullptr;
    const int st = device_info(&d);
    if (st != MLA_OK) return st;
    LaunchGeom g;
    geom_for(s_q, num_heads, &g);
    *bytes = ws_layout(batch, s_q * num_heads, item_capacity(*d, g, batch)).total;
    return MLA_OK;
}

int mla_decode_plan_chunked(const int32_t* seqlens, int batch, int s_q, int num_heads, int chunk_pages,
                            void* workspace, size_t workspace_bytes, void* stream)
{
    if (!seqlens || !workspace || !batch_ok(batch) || chunk_pages < 0) return MLA_ERR_INVALID_ARG;
    if (!aligned(workspace, 256) || !aligned(seqlens, 4)) return MLA_ERR_INVALID_ARG;
    if (!heads_ok(s_q, num_heads)) return MLA_ERR_UNSUPPORTED;
    const DeviceInfo* d = nullptr;
    const int st = device_info(&d);
    if (st != MLA_OK) return st;
    LaunchGeom g;
    geom_for(s_q, num_heads, &g);
    const int cap = item_capacity(*d, g, batch);
    if (workspace_bytes < ws_layout(batch, s_q * num_heads, cap).total) return MLA_ERR_WORKSPACE_TOO_SMALL;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, static_cast<hipStream_t>(stream), seqlens,
                       batch, s_q, num_heads, s_q * num_heads, gx_of(*d, g), cap, static_cast<char*>(workspace), -1,
                       chunk_pages);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_decode_plan(const int32_t* seqlens, int batch, int s_q, int num_heads, void* workspace,
                    size_t workspace_bytes, void* stream)
{
    return mla_decode_plan_chunked(seqlens, batch, s_q, num_heads, 0, workspace, workspace_bytes, stream);
}

namespace {

int prepare_fwd(const void* q, const void* kv_cache, const int32_t* block_table, int bt_stride,
                const int32_t* seqlens, int batch, int s_q, int num_heads, int num_pages, int page_size,
                float softmax_scale, int causal, void* workspace, size_t workspace_bytes, void* out, float* lse,
                bool need_inputs, bool need_outputs, FwdArgs* a, LaunchGeom* g)
{
    if (!seqlens || !workspace) return MLA_ERR_INVALID_ARG;
    if (need_inputs && (!q || !kv_cache || !block_table)) return MLA_ERR_INVALID_ARG;
    if (need_outputs && (!out || !lse)) return MLA_ERR_INVALID_ARG;
    if (!batch_ok(batch) || bt_stride < 1) return MLA_ERR_INVALID_ARG;
    if (need_inputs && num_pages < 1) return MLA_ERR_INVALID_ARG;
    if (need_inputs && (!std::isfinite(softmax_scale * kLog2e) || (causal != 0 && causal != 1)))
        return MLA_ERR_INVALID_ARG;
    if (!aligned(workspace, 256) || !aligned(seqlens, 4)) return MLA_ERR_INVALID_ARG;
    if (need_inputs && (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(block_table, 4)))
        return MLA_ERR_INVALID_ARG;
    if (need_outputs && (!aligned(out, 8) || !aligned(lse, 4))) return MLA_ERR_INVALID_ARG;
    if (!heads_ok(s_q, num_heads) || (need_inputs && page_size != MLA_DECODE_PAGE_SIZE)) return MLA_ERR_UNSUPPORTED;
    const DeviceInfo* d = nullptr;
    const int st = device_info(&d);
    if (st != MLA_OK) return st;
    geom_for(s_q, num_heads, g);
    const int rows = s_q * num_heads;
    const int cap = item_capacity(*d, *g, batch);
    if (workspace_bytes < ws_layout(batch, rows, cap).total) return MLA_ERR_WORKSPACE_TOO_SMALL;
    a->q = static_cast<const uint16_t*>(q);
    a->cache = static_cast<const uint16_t*>(kv_cache);
    a->block_table = block_table;
    a->seqlens = seqlens;
    a->ws = static_cast<char*>(workspace);
    a->out = static_cast<uint16_t*>(out);
    a->lse = lse;
    a->num_pages = num_pages;
    a->bt_stride = bt_stride;
    a->batch = batch;
    a->s_q = s_q;
    a->heads = num_heads;
    a->rows = rows;
    a->capacity = cap;
    a->scale_log2 = softmax_scale * kLog2e;
    a->causal = causal;
    a->row_groups = g->row_groups;
    return MLA_OK;
}

int launch_split(const FwdArgs& a, const LaunchGeom& g, hipStream_t s)
{
    // wide forms: the row groups of an item get ids 8 apart within blocks of 8 * row_groups ids
    const int blocks = ((a.capacity + 7) / 8) * 8 * g.row_groups;
    switch (g.cfg) {
    case kR16:
        hipLaunchKernelGGL(split_kernel<CfgR16>, dim3(a.capacity, g.row_groups), dim3(g.threads), g.lds_bytes, s, a);
        break;
    case kSV1: hipLaunchKernelGGL(split_sv_kernel<CfgSV1>, dim3(blocks), dim3(g.threads), g.lds_bytes, s, a); break;
    case kSV2: hipLaunchKernelGGL(split_sv_kernel<CfgSV2>, dim3(blocks), dim3(g.threads), g.lds_bytes, s, a); break;
    default: return MLA_ERR_HIP;   // not a split configuration of this entry point
    }
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int launch_combine(const FwdArgs& a, hipStream_t s)
{
    hipLaunchKernelGGL(combine_kernel_t<kDv>, dim3(a.batch * a.rows), dim3(kCombineThreads), 0, s, a);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace

int mla_decode_fwd(const void* q, const void* kv_cache, const int32_t* block_table, int bt_stride,
                   const int32_t* seqlens, int batch, int s_q, int num_heads, int num_pages, int page_size,
                   float softmax_scale, int causal, void* workspace, size_t workspace_bytes, void* out,
                   float* lse, void* stream)
{
    FwdArgs a;
    LaunchGeom g;
    int st = prepare_fwd(q, kv_cache, block_table, bt_stride, seqlens, batch, s_q, num_heads, num_pages, page_size,
                         softmax_scale, causal, workspace, workspace_bytes, out, lse, true, true, &a, &g);
    if (st != MLA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = launch_split(a, g, s);
    if (st != MLA_OK) return st;
    return launch_combine(a, s);
}

int mla_decode_fwd_split(const void* q, const void* kv_cache, const int32_t* block_table, int bt_stride,
                         const int32_t* seqlens, int batch, int s_q, int num_heads, int num_pages, int page_size,
                         float softmax_scale, int causal, void* workspace, size_t workspace_bytes, void* stream)
{
    FwdArgs a;
    LaunchGeom g;
    const int st = prepare_fwd(q, kv_cache, block_table, bt_stride, seqlens, batch, s_q, num_heads, num_pages,
                               page_size, softmax_scale, causal, workspace, workspace_bytes, nullptr, nullptr, true,
                               false, &a, &g);
    if (st != MLA_OK) return st;
    return launch_split(a, g, static_cast<hipStream_t>(stream));
}

int mla_decode_fwd_combine(const int32_t* seqlens, int bt_stride, int batch, int s_q, int num_heads,
                           void* workspace, size_t workspace_bytes, void* out, float* lse, void* stream)
{
    FwdArgs a;
    LaunchGeom g;
    const int st = prepare_fwd(nullptr, nullptr, nullptr, bt_stride, seqlens, batch, s_q, num_heads, 1,
                               MLA_DECODE_PAGE_SIZE, 1.f, 0, workspace, workspace_bytes, out, lse, false, true, &a,
                               &g);
    if (st != MLA_OK) return st;
    return launch_combine(a, static_cast<hipStream_t>(stream));
}

int mla_decode_fwd_noalloc(const void* q, const void* kv_cache, const int32_t* block_table, int bt_stride,
                           const int32_t* seqlens, int batch, int s_q, int num_heads, int num_pages, int page_size,
                           float softmax_scale, int causal, void* out, float* lse, void* stream)
{
    // argument checks and the size check against the built-in scratch, before its address is
    // taken (the placeholder is never dereferenced)
    FwdArgs a;
    LaunchGeom g;
    void* const placeholder = reinterpret_cast<void*>(uintptr_t(256));
    int st = prepare_fwd(q, kv_cache, block_table, bt_stride, seqlens, batch, s_q, num_heads, num_pages, page_size,
                         softmax_scale, causal, placeholder, MLA_DECODE_NOALLOC_SCRATCH_BYTES, out, lse, true, true,
                         &a, &g);
    if (st != MLA_OK) return st;
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != MLA_OK) return st;
    a.ws = static_cast<char*>(ws);
    const DeviceInfo* d = nullptr;
    st = device_info(&d);
    if (st != MLA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the plan writes every workspace field the split and combine kernels read: nothing needs
    // clearing between calls
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, seqlens, batch, s_q, num_heads,
                       s_q * num_heads, gx_of(*d, g), a.capacity, a.ws, -1);
    if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
    st = launch_split(a, g, s);
    if (st != MLA_OK) return st;
    return launch_combine(a, s);
}

int mla_cache_append_rope(const void* kv_latent, const void* k_rope, void* q, void* kv_cache,
                          const int32_t* block_table, int bt_stride, const int32_t* seqlens, int batch, int s_q,
                          int num_heads, int num_pages, int page_size, float rope_base, void* stream)
{
    if (!kv_latent || !k_rope || !q || !kv_cache || !block_table || !seqlens) return MLA_ERR_INVALID_ARG;
    if (!batch_ok(batch) || bt_stride < 1 || num_pages < 1) return MLA_ERR_INVALID_ARG;
    if (!std::isfinite(rope_base) || !(rope_base > 1.f)) return MLA_ERR_INVALID_ARG;
    if (!aligned(kv_latent, 16) || !aligned(k_rope, 4) || !aligned(q, 4) || !aligned(kv_cache, 16) ||
        !aligned(block_table, 4) || !aligned(seqlens, 4))
        return MLA_ERR_INVALID_ARG;
    if (!heads_ok(s_q, num_heads) || page_size != MLA_DECODE_PAGE_SIZE) return MLA_ERR_UNSUPPORTED;
    const DeviceInfo* d = nullptr;
    const int st = device_info(&d);
    if (st != MLA_OK) return st;
    AppendArgs a;
    a.kv_latent = static_cast<const uint16_t*>(kv_latent);
    a.k_rope = static_cast<const uint16_t*>(k_rope);
    a.q = static_cast<uint16_t*>(q);
    a.cache = static_cast<uint16_t*>(kv_cache);
    a.block_table = block_table;
    a.seqlens = seqlens;
    a.num_pages = num_pages;
    a.bt_stride = bt_stride;
    a.batch = batch;
    a.s_q = s_q;
    a.heads = num_heads;
    a.log2_base = std::log2((double)rope_base);
    hipLaunchKernelGGL(append_rope_kernel, dim3(batch * s_q), dim3(kAppendThreads), 0,
                       static_cast<hipStream_t>(stream), a);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

namespace {

// Sparse decode: each of the batch * s_q query tokens is a sequence of `topk` index slots with
// num_heads (16) rows; the plan, the split workspace and the combine work per query token.
constexpr LaunchGeom kSparseGeom = {kS16, 1, CfgR16::THREADS, CfgR16::LDS_BYTES};

int sparse_shape_ok(int batch, int s_q, int num_heads, int topk)
{
    if (batch < 1 || topk < 1) return MLA_ERR_INVALID_ARG;
    if ((s_q != 1 && s_q != 2) || num_heads != 16) return MLA_ERR_UNSUPPORTED;
    if ((long long)batch * s_q > (1 << 24)) return MLA_ERR_INVALID_ARG;
    return MLA_OK;
}

}  // namespace

int mla_sparse_decode_workspace_size(int batch, int s_q, int num_heads, int topk, size_t* bytes)
{
    if (!bytes) return MLA_ERR_INVALID_ARG;
    int st = sparse_shape_ok(batch, s_q, num_heads, topk);
    if (st != MLA_OK) return st;
    const DeviceInfo* d = nullptr;
    st = device_info(&d);
    if (st != MLA_OK) return st;
    const int nt = batch * s_q;
    *bytes = ws_layout(nt, num_heads, item_capacity(*d, kSparseGeom, nt)).total;
    return MLA_OK;
}

int mla_sparse_decode_plan(int batch, int s_q, int num_heads, int topk, void* workspace, size_t workspace_bytes,
                           void* stream)
{
    if (!workspace || !aligned(workspace, 256)) return MLA_ERR_INVALID_ARG;
    int st = sparse_shape_ok(batch, s_q, num_heads, topk);
    if (st != MLA_OK) return st;
    const DeviceInfo* d = nullptr;
    st = device_info(&d);
    if (st != MLA_OK) return st;
    const int nt = batch * s_q;
    const int cap = item_capacity(*d, kSparseGeom, nt);
    if (workspace_bytes < ws_layout(nt, num_heads, cap).total) return MLA_ERR_WORKSPACE_TOO_SMALL;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, static_cast<hipStream_t>(stream), nullptr, nt,
                       1, num_heads, num_heads, gx_of(*d, kSparseGeom), cap, static_cast<char*>(workspace), topk);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_sparse_decode_fwd(const void* q, const void* kv_cache, const int32_t* block_table, int bt_stride,
                          const int32_t* seqlens, const int32_t* indices, int batch, int s_q, int num_heads,
                          int topk, int num_pages, int page_size, float softmax_scale, void* workspace,
                          size_t workspace_bytes, void* out, float* lse, void* stream)
{
    if (!q || !kv_cache || !block_table || !seqlens || !indices || !workspace || !out || !lse)
        return MLA_ERR_INVALID_ARG;
    // the gather forms 32-bit cache row ids (page * 64 + slot)
    if (bt_stride < 1 || num_pages < 1 || num_pages > (1 << 25) || !std::isfinite(softmax_scale * kLog2e))
        return MLA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(block_table, 4) || !aligned(seqlens, 4) ||
        !aligned(indices, 4) || !aligned(workspace, 256) || !aligned(out, 8) || !aligned(lse, 4))
        return MLA_ERR_INVALID_ARG;
    int st = sparse_shape_ok(batch, s_q, num_heads, topk);
    if (st != MLA_OK) return st;
    if (page_size != MLA_DECODE_PAGE_SIZE) return MLA_ERR_UNSUPPORTED;
    const DeviceInfo* d = nullptr;
    st = device_info(&d);
    if (st != MLA_OK) return st;
    const int nt = batch * s_q;
    const int cap = item_capacity(*d, kSparseGeom, nt);
    const WsLayout lay = ws_layout(nt, num_heads, cap);
    if (workspace_bytes < lay.total) return MLA_ERR_WORKSPACE_TOO_SMALL;
    FwdArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.cache = static_cast<const uint16_t*>(kv_cache);
    a.block_table = block_table;
    a.seqlens = seqlens;
    a.ws = static_cast<char*>(workspace);
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    a.num_pages = num_pages;
    a.bt_stride = bt_stride;
    a.batch = nt;
    a.s_q = 1;
    a.heads = num_heads;
    a.rows = num_heads;
    a.capacity = cap;
    a.scale_log2 = softmax_scale * kLog2e;
    a.causal = 0;
    a.row_groups = 1;
    a.indices = indices;
    a.topk = topk;
    a.sparse_sq = s_q;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL((split_kernel<CfgR16, true>), dim3(cap, 1), dim3(CfgR16::THREADS), CfgR16::LDS_BYTES, s, a);
    if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
    // the combine checks each token's length against the plan's copy of it and the table width
    FwdArgs c = a;
    c.seqlens = reinterpret_cast<const int32_t*>(a.ws + lay.seqlens);
    c.bt_stride = topk / kPage + (topk % kPage != 0 ? 1 : 0);   // no topk + 63 (overflow near INT_MAX)
    return launch_combine(c, s);
}

namespace {

int launch_head_gemm(const HeadGemmArgs& g, int heads, hipStream_t s)
{
    hipLaunchKernelGGL(head_gemm_kernel, dim3(heads, g.N / 64, (g.M + 15) / 16), dim3(kAbsorbThreads), 0, s, g);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int absorb_shape_ok(int batch, int s_q, int num_heads)
{
    if (batch < 1 || (long long)batch * s_q > (1 << 20)) return MLA_ERR_INVALID_ARG;
    return heads_ok(s_q, num_heads) ? MLA_OK : MLA_ERR_UNSUPPORTED;
}

}  // namespace

int mla_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk, int batch, int s_q, int num_heads,
                 void* q, void* stream)
{
    if (!q_nope || !q_rope || !w_uk || !q) return MLA_ERR_INVALID_ARG;
    if (!aligned(q_nope, 16) || !aligned(q_rope, 16) || !aligned(w_uk, 16) || !aligned(q, 16))
        return MLA_ERR_INVALID_ARG;
    int st = absorb_shape_ok(batch, s_q, num_heads);
    if (st != MLA_OK) return st;
    const DeviceInfo* d = nullptr;
    st = device_info(&d);
    if (st != MLA_OK) return st;
    HeadGemmArgs g{};
    g.a = static_cast<const uint16_t*>(q_nope);
    g.w = static_cast<const uint16_t*>(w_uk);
    g.c = static_cast<uint16_t*>(q);
    g.lda = (long long)num_heads * kDNope;
    g.a_head = kDNope;
    g.w_head = (long long)kDv * kDNope;
    g.ldc = (long long)num_heads * kDk;
    g.c_head = kDk;
    g.M = batch * s_q;
    g.N = kDv;
    g.K = kDNope;
    g.rope = static_cast<const uint16_t*>(q_rope);
    g.heads = num_heads;
    return launch_head_gemm(g, num_heads, static_cast<hipStream_t>(stream));
}

int mla_unabsorb_o(const void* o_latent, const void* w_uv, int batch, int s_q, int num_heads, void* o, void* stream)
{
    if (!o_latent || !w_uv || !o) return MLA_ERR_INVALID_ARG;
    if (!aligned(o_latent, 16) || !aligned(w_uv, 16) || !aligned(o, 2)) return MLA_ERR_INVALID_ARG;
    int st = absorb_shape_ok(batch, s_q, num_heads);
    if (st != MLA_OK) return st;
    const DeviceInfo* d = nullptr;
    st = device_info(&d);
    if (st != MLA_OK) return st;
    HeadGemmArgs g{};
    g.a = static_cast<const uint16_t*>(o_latent);
    g.w = static_cast<const uint16_t*>(w_uv);
    g.c = static_cast<uint16_t*>(o);
    g.lda = (long long)num_heads * kDv;
    g.a_head = kDv;
    g.w_head = (long long)kDNope * kDv;
    g.ldc = (long long)num_heads * kDNope;
    g.c_head = kDNope;
    g.M = batch * s_q;
    g.N = kDNope;
    g.K = kDv;
    g.rope = nullptr;
    g.heads = num_heads;
    return launch_head_gemm(g, num_heads, static_cast<hipStream_t>(stream));
}

namespace {

int gqa_geom(int batch, int s_q, int num_heads, LaunchGeom* g)
{
    if (!batch_ok(batch)) return MLA_ERR_INVALID_ARG;
    if ((s_q != 1 && s_q != 2) || num_heads != kGqaHeads) return MLA_ERR_UNSUPPORTED;
    *g = s_q == 1 ? LaunchGeom{kG1, 1, kGqaThreads, CfgG1::LDS_BYTES} : LaunchGeom{kG2, 1, kGqaThreads, CfgG2::LDS_BYTES};
    return MLA_OK;
}

}  // namespace

int mla_gqa_decode_workspace_size(int batch, int s_q, int num_heads, size_t* bytes)
{
    if (!bytes) return MLA_ERR_INVALID_ARG;
    LaunchGeom g;
    int st = gqa_geom(batch, s_q, num_heads, &g);
    if (st != MLA_OK) return st;
    const DeviceInfo* d = nullptr;
    st = device_info(&d);
    if (st != MLA_OK) return st;
    *bytes = ws_layout(batch, s_q * num_heads, item_capacity(*d, g, batch), kGqaDv).total;
    return MLA_OK;
}

int mla_gqa_decode_plan(const int32_t* seqlens, int batch, int s_q, int num_heads, void* workspace,
                        size_t workspace_bytes, void* stream)
{
    if (!seqlens || !workspace || !aligned(workspace, 256) || !aligned(seqlens, 4)) return MLA_ERR_INVALID_ARG;
    LaunchGeom g;
    int st = gqa_geom(batch, s_q, num_heads, &g);
    if (st != MLA_OK) return st;
    const DeviceInfo* d = nullptr;
    st = device_info(&d);
    if (st != MLA_OK) return st;
    const int rows = s_q * num_heads;
    const int cap = item_capacity(*d, g, batch);
    if (workspace_bytes < ws_layout(batch, rows, cap, kGqaDv).total) return MLA_ERR_WORKSPACE_TOO_SMALL;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, static_cast<hipStream_t>(stream), seqlens, batch,
                       s_q, num_heads, rows, gx_of(*d, g), cap, static_cast<char*>(workspace), -1);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_gqa_decode_fwd(const void* q, const void* kv_cache, const int32_t* block_table, int bt_stride,
                       const int32_t* seqlens, int batch, int s_q, int num_heads, int num_pages, int page_size,
                       float softmax_scale, int causal, void* workspace, size_t workspace_bytes, void* out, float* lse,
                       void* stream)
{
    if (!q || !kv_cache || !block_table || !seqlens || !workspace || !out || !lse) return MLA_ERR_INVALID_ARG;
    if (bt_stride < 1 || num_pages < 1 || !std::isfinite(softmax_scale * kLog2e) || (causal != 0 && causal != 1))
        return MLA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(block_table, 4) || !aligned(seqlens, 4) ||
        !aligned(workspace, 256) || !aligned(out, 2) || !aligned(lse, 4))
        return MLA_ERR_INVALID_ARG;
    LaunchGeom g;
    int st = gqa_geom(batch, s_q, num_heads, &g);
    if (st != MLA_OK) return st;
    if (page_size != MLA_DECODE_PAGE_SIZE) return MLA_ERR_UNSUPPORTED;
    const DeviceInfo* d = nullptr;
    st = device_info(&d);
    if (st != MLA_OK) return st;
    const int rows = s_q * num_heads;
    const int cap = item_capacity(*d, g, batch);
    if (workspace_bytes < ws_layout(batch, rows, cap, kGqaDv).total) return MLA_ERR_WORKSPACE_TOO_SMALL;
    FwdArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.cache = static_cast<const uint16_t*>(kv_cache);
    a.block_table = block_table;
    a.seqlens = seqlens;
    a.ws = static_cast<char*>(workspace);
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    a.num_pages = num_pages;
    a.bt_stride = bt_stride;
    a.batch = batch;
    a.s_q = s_q;
    a.heads = num_heads;
    a.rows = rows;
    a.capacity = cap;
    a.scale_log2 = softmax_scale * kLog2e;
    a.causal = causal;
    a.row_groups = 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (s_q == 1)
        hipLaunchKernelGGL(gqa_split_kernel<CfgG1>, dim3(cap), dim3(kGqaThreads), CfgG1::LDS_BYTES, s, a);
    else
        hipLaunchKernelGGL(gqa_split_kernel<CfgG2>, dim3(cap), dim3(kGqaThreads), CfgG2::LDS_BYTES, s, a);
    if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
    hipLaunchKernelGGL(combine_kernel_t<kGqaDv>, dim3(batch * rows), dim3(kCombineThreads), 0, s, a);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

const char* mla_decode_status_string(int status)
{
    switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: null pointer, bad size, alignment or non-finite scale";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: heads must be a multiple of 16 in 16..128, s_q 1 or 2, page size 64";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL: see mla_decode_workspace_size";
    case MLA_ERR_NO_DEVICE: return "MLA_ERR_NO_DEVICE: no usable gfx950 HIP device";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: a HIP runtime call failed";
    default: return "unknown mla_status";
    }
}

}  // extern "C"
