// Operand repack for gemm_run_ws: copy a matrix whose rows are not 16-byte
// aligned into a caller-owned workspace with 16-byte aligned rows, for the
// kernels whose 16-byte reads expect aligned rows (the fp32 kernels and the
// register-staged matrix-core tiles; the direct-copy and thin kernels read
// any alignment in place and their plans never repack).  Padding misaligned
// operands is the pages' other remedy besides a guarded narrow loader (the
// "流水化 GPU 内核" skill's pitfall list: the asynchronous copy needs aligned
// sources; the SM80 ablation plan, section 1.4, note 2).
#include <hip/hip_runtime.h>

#include "tg_device.hpp"
#include "tg_pack.hpp"

namespace tg {

// Each thread writes 16-byte chunks of destination rows (a grid-stride loop
// over them): one 16-byte load from the source at any byte address, byte
// loads where those 16 bytes would leave the source's valid bytes
// [src, src + (rows-1) ld_s + row_bytes).  Bytes of a destination row past
// row_bytes are written as zero.
__global__ __launch_bounds__(256) void pack_rows(PackArgs a) {
    const int64_t cpr = a.ld_d / 16;
    const int64_t total = a.rows * cpr;
    const uintptr_t beg = reinterpret_cast<uintptr_t>(a.src);
    const uintptr_t end = beg + (uintptr_t)((a.rows - 1) * a.ld_s + a.row_bytes);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / cpr;
        const int64_t off = (i - r * cpr) * 16;  // byte offset in the row
        i32x4 v = {0, 0, 0, 0};
        if (off < a.row_bytes) {
            const uintptr_t p = beg + (uintptr_t)(r * a.ld_s + off);
            if (p + 16 <= end) {
                v = load16(reinterpret_cast<const void*>(p));
            } else {
                union { i32x4 v; uint8_t b[16]; } u;
#pragma unroll
                for (int t = 0; t < 16; ++t)
                    u.b[t] = load_or_zero(reinterpret_cast<const uint8_t*>(p + t), p + t < end);
                v = u.v;
            }
            if (off + 16 > a.row_bytes) {  // the row's last, partial chunk
                union { i32x4 v; uint8_t b[16]; } u;
                u.v = v;
#pragma unroll
                for (int t = 0; t < 16; ++t)
                    if (off + t >= a.row_bytes) u.b[t] = 0;
                v = u.v;
            }
        }
        *reinterpret_cast<i32x4*>(a.dst + r * a.ld_d + off) = v;
    }
}

hipError_t launch_pack(const PackArgs& a, hipStream_t stream) {
    // one 16-byte chunk per thread, at most 8192 workgroups
    const int64_t total = a.rows * (a.ld_d / 16);
    const int64_t blocks = (total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(pack_rows, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tg
