// Host entry of the operand repack kernel (tg_pack.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

// Enqueue a copy of `rows` rows of `row_bytes` bytes from src (row stride
// ld_s bytes) to dst (row stride ld_d bytes: a multiple of 16, >= row_bytes;
// dst 16-byte aligned), zero-filling each destination row past row_bytes.
// With `compact`, bytes [col_beg, col_beg + col_bytes) of every row are also
// written, densely, to compact[row * col_bytes ..].
hipError_t launch_pack(const void* src, void* dst, int64_t rows, int64_t row_bytes, int64_t ld_s, int64_t ld_d,
                       hipStream_t stream, void* compact = nullptr, int64_t col_beg = 0, int64_t col_bytes = 0);

}  // namespace tg
