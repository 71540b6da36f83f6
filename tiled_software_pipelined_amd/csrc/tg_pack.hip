// Operand repack for gemm_run_ws: copy a matrix whose rows are not 16-byte
// aligned into a caller-owned workspace with 16-byte aligned rows, so that
// the GEMM that follows can move every slice with the direct global->LDS
// copy.  Padding misaligned operands is the pages' other remedy besides a
// guarded narrow loader (the "流水化 GPU 内核" skill's pitfall list: the
// asynchronous copy needs aligned sources; the SM80 ablation plan,
// section 1.4, note 2).
#include <hip/hip_runtime.h>

#include "tg_pack.hpp"

namespace tg {

__global__ __launch_bounds__(256) void pack_rows(PackArgs a) { pack_chunks(a, blockIdx.x, gridDim.x); }

hipError_t launch_pack(const PackArgs& a, hipStream_t stream) {
    const int64_t blocks = pack_blocks(a);
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(pack_rows, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tg
