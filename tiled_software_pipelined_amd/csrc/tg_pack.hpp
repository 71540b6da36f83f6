// Operand repack: the device body shared by the standalone repack kernel
// (tg_pack.hip) and the fused repack + thin kernel (tg_kernels.hpp), and the
// host entry of the standalone one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tg_device.hpp"

namespace tg {

// Workgroup `block` of `nblocks` (256 threads each) of the repack described
// by `a`.  Each thread writes 16-byte chunks of destination rows (a grid-
// stride loop over them): the two aligned 16-byte blocks of the source that
// cover the chunk, funnel-shifted; byte loads where that pair would leave
// the source's valid bytes [src, src + (rows-1) ld_s + row_bytes).  Bytes of
// a destination row past row_bytes are written as zero.
__device__ __forceinline__ void pack_chunks(const PackArgs& a, int64_t block, int64_t nblocks) {
    const int64_t cpr = a.ld_d / 16;
    const int64_t total = a.rows * cpr;
    const uintptr_t beg = reinterpret_cast<uintptr_t>(a.src);
    const uintptr_t end = beg + (uintptr_t)((a.rows - 1) * a.ld_s + a.row_bytes);
    for (int64_t i = block * 256 + threadIdx.x; i < total; i += nblocks * 256) {
        const int64_t r = i / cpr;
        const int64_t off = (i - r * cpr) * 16;  // byte offset in the row
        i32x4 v = {0, 0, 0, 0};
        if (off < a.row_bytes) {
            const uintptr_t p = beg + (uintptr_t)(r * a.ld_s + off);
            const uintptr_t lo = p & ~uintptr_t(15);
            if (lo >= beg && lo + 32 <= end) {
                const i32x4 x = *reinterpret_cast<const i32x4*>(lo);
                const i32x4 y = *reinterpret_cast<const i32x4*>(lo + 16);
                v = funnel16(x, y, uint32_t(p - lo));
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

// Workgroups of the repack: one 16-byte chunk per thread, at most 8192.
inline int64_t pack_blocks(const PackArgs& a) {
    const int64_t total = a.rows * (a.ld_d / 16);
    const int64_t want = (total + 255) / 256;
    return want < 8192 ? want : 8192;
}

// Enqueue the repack of `a` on `stream`.
hipError_t launch_pack(const PackArgs& a, hipStream_t stream);

}  // namespace tg
