// Operand repack for gemm_run_ws: copy a matrix whose rows are not 16-byte
// aligned into a caller-owned workspace with 16-byte aligned rows, so that
// the GEMM that follows can move every slice with the direct global->LDS
// copy.  Padding misaligned operands is the pages' other remedy besides a
// guarded narrow loader (the "流水化 GPU 内核" skill's pitfall list: the
// asynchronous copy needs aligned sources; the SM80 ablation plan,
// section 1.4, note 2).
#include <hip/hip_runtime.h>

#include "tg_device.hpp"
#include "tg_pack.hpp"

namespace tg {

// rows x row_bytes bytes at src (row stride ld_s bytes) -> dst (row stride
// ld_d bytes, a multiple of 16; dst 16-byte aligned).  Each thread writes
// one 16-byte chunk of a destination row: the two aligned 16-byte blocks of
// the source that cover it, funnel-shifted; byte loads where that pair would
// leave the source's valid bytes [src, src + (rows-1) ld_s + row_bytes).
// Bytes of the destination row past row_bytes are written as zero.  With
// `compact`, the thread whose chunk holds bytes [col_beg, col_beg +
// col_bytes) of the row also writes them to compact[r * col_bytes ..].
__global__ __launch_bounds__(256) void pack_rows(const char* src, char* dst, int64_t rows, int64_t row_bytes,
                                                 int64_t ld_s, int64_t ld_d, char* compact, int64_t col_beg,
                                                 int64_t col_bytes) {
    const int64_t cpr = ld_d / 16;
    const int64_t total = rows * cpr;
    const uintptr_t beg = reinterpret_cast<uintptr_t>(src);
    const uintptr_t end = beg + (uintptr_t)((rows - 1) * ld_s + row_bytes);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / cpr;
        const int64_t off = (i - r * cpr) * 16;  // byte offset in the row
        i32x4 v = {0, 0, 0, 0};
        if (off < row_bytes) {
            const uintptr_t a = beg + (uintptr_t)(r * ld_s + off);
            const uintptr_t lo = a & ~uintptr_t(15);
            if (lo >= beg && lo + 32 <= end) {
                const i32x4 x = *reinterpret_cast<const i32x4*>(lo);
                const i32x4 y = *reinterpret_cast<const i32x4*>(lo + 16);
                v = funnel16(x, y, uint32_t(a - lo));
            } else {
                union { i32x4 v; uint8_t b[16]; } u;
#pragma unroll
                for (int t = 0; t < 16; ++t) u.b[t] = a + t < end ? *reinterpret_cast<const uint8_t*>(a + t) : 0;
                v = u.v;
            }
            if (off + 16 > row_bytes) {  // the row's last, partial chunk
                union { i32x4 v; uint8_t b[16]; } u;
                u.v = v;
#pragma unroll
                for (int t = 0; t < 16; ++t)
                    if (off + t >= row_bytes) u.b[t] = 0;
                v = u.v;
            }
        }
        *reinterpret_cast<i32x4*>(dst + r * ld_d + off) = v;
        if (compact && off + 16 > col_beg && off < col_beg + col_bytes) {
            union { i32x4 v; char b[16]; } u;
            u.v = v;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const int64_t c = off + t - col_beg;
                if (c >= 0 && c < col_bytes) compact[r * col_bytes + c] = u.b[t];
            }
        }
    }
}

hipError_t launch_pack(const void* src, void* dst, int64_t rows, int64_t row_bytes, int64_t ld_s, int64_t ld_d,
                       hipStream_t stream, void* compact, int64_t col_beg, int64_t col_bytes) {
    const int64_t total = rows * (ld_d / 16);
    if (total <= 0) return hipSuccess;
    const int64_t want = (total + 255) / 256;
    const unsigned blocks = (unsigned)(want < 8192 ? want : 8192);
    hipLaunchKernelGGL(pack_rows, dim3(blocks), dim3(256), 0, stream, static_cast<const char*>(src),
                       static_cast<char*>(dst), rows, row_bytes, ld_s, ld_d, static_cast<char*>(compact), col_beg,
                       col_bytes);
    return hipGetLastError();
}

}  // namespace tg
