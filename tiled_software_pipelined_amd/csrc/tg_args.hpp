// Kernel argument block and the registry record that describes one compiled
// kernel variant to the host library.
#pragma once

#include <stdint.h>

namespace tg {

// Passed by value to every GEMM kernel.  Row-major operands, leading
// dimensions in elements; sizes already validated by the host.
struct GemmArgs {
    const void* A;
    const void* B;
    void* C;
    int32_t M, N, K;
    int32_t tiles_m, tiles_n;  // ceil(M / BM), ceil(N / BN)
    int64_t lda, ldb, ldc;
    int32_t wg_group;          // <= 0: row-major workgroup order
    int32_t a_guard;           // 1: A rows not 16-byte aligned, for a kernel that needs them aligned
    int32_t b_guard;           // 1: the same for B, or N not a whole number of 16-byte chunks
    int32_t c_stream;          // 1: non-temporal C stores (C rows 128-byte aligned; 256 x 256 tiles: K >= 4 KiB per row)
    uint64_t* clocks;          // NULL, or 6 values per workgroup (tiled kernels): shader-clock and
                               // 100 MHz real-time counters at its start, at the end of its
                               // K loop, then at its end
};

typedef void (*KernelFn)(GemmArgs);

// One operand repack (tg_pack.hpp): `rows` rows of `row_bytes` bytes from
// src (row stride ld_s bytes) to dst (row stride ld_d bytes, a multiple of
// 16; dst 16-byte aligned), zero past row_bytes.
struct PackArgs {
    const char* src;
    char* dst;
    int64_t rows, row_bytes, ld_s, ld_d;
};


// Values per workgroup in GemmArgs::clocks (TGEMM_CLOCK_VALUES of the C ABI).
constexpr int CLOCK_VALUES = 6;

// Widest N the thin kernel (and the remainder of a split plan) takes.
constexpr int THIN_N_MAX = 16;

enum Family { FAM_NAIVE = 1, FAM_TILED = 2, FAM_THIN = 3 };
enum Loader { LD_VGPR = 1, LD_DIRECT = 2 };
// LY_XOR_POISON: LY_XOR plus a debug fill of every LDS chunk with all-ones
// bytes just before its direct copy is issued (see MfmaGemm::issue_direct_one)
enum Layout { LY_PLAIN = 1, LY_XOR = 2, LY_XOR_POISON = 3 };
enum Access { AC_WIDE = 1, AC_NARROW = 2 };
// FR_SLICE: FR_REUSE with the fragments of a whole slice read one slice
// ahead (direct loader; see MfmaGemm::slice_ahead)
enum Frag { FR_REUSE = 1, FR_PER_MMA = 2, FR_SLICE = 3 };

struct KernelEntry {
    int dtype;       // TGEMM_* dtype
    int family;      // Family
    int bm, bn, bk;  // tile (naive: threads per block in x/y, bk = 1)
    int stages;
    int loader;      // Loader
    int layout;      // Layout
    int access;      // Access
    int frag;        // Frag
    int wm, wn;      // wave grid
    int store;       // C store width (fp32 kernels), 0 = not applicable
    int gload_bytes; // width of the global loads of full chunks (0: element loads only)
    int threads;     // threads per workgroup
    int lds_bytes;   // static LDS per workgroup
    int loads_per_stage;  // global->LDS instructions per wave per stage
    int shift_mask;  // bit 0: reads A rows that are not 16-byte aligned; bit 1: reads B rows that are not
                     // (the direct loader: B whose N is not a whole number of 16-byte pieces)
    int listed;      // 0: only reached as the fallback of a listed entry for such operands
    int tail_ok;     // handles K not a multiple of bk
    int waves_per_simd;  // occupancy the kernel is compiled for (its registers allow at least this)
    int copy_sched;  // TGEMM_COPY_BURST / TGEMM_COPY_SPREAD (direct loader; others report BURST)
    int frag_read;   // TGEMM_READ_*: how fragments come out of LDS
    int lane_map;    // TGEMM_LANES_*: outputs of a lane (fp32 kernels; others report BLOCKS)
    KernelFn fn;
    KernelFn rem_fn;       // the twin that also computes column N of an N + 1 wide product (else NULL)
    int thin_col;          // thin kernels: 1 = the twin for a contiguous B column (N = 1, ldb = 1)
    int thin_mma;          // thin kernels: 1 = on the matrix cores (B rows read as NB-column pieces)
    char name[96];
};

// Filled by each instantiation unit; the host library concatenates them.
void register_bf16(void (*add)(const KernelEntry&));
void register_i8(void (*add)(const KernelEntry&));
void register_f32(void (*add)(const KernelEntry&));

}  // namespace tg
