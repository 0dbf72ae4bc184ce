// The 128-row split kernel in a translation unit of its own: its 256 output accumulators per
// lane live in the accumulation registers (AGPRs), so this file is compiled without the option
// that keeps MFMA accumulators in arch VGPRs for the other kernels.
#include <hip/hip_runtime.h>

#include "mla_rw_kernel.h"

namespace mla {

using CfgRW4 = RwCfg<4>;   // 4 waves x 32 rows

const void* split_rw_fn() { return reinterpret_cast<const void*>(&split_rw_kernel<CfgRW4>); }
int split_rw_threads() { return CfgRW4::THREADS; }
int split_rw_lds_bytes() { return CfgRW4::LDS_BYTES; }

void launch_split_rw(const FwdArgs& a, int blocks, hipStream_t s)
{
    hipLaunchKernelGGL(split_rw_kernel<CfgRW4>, dim3(blocks), dim3(CfgRW4::THREADS), CfgRW4::LDS_BYTES, s, a);
}

}  // namespace mla
