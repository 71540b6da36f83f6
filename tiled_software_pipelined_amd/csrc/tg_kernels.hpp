// Kernel entry points and registry records for the kernel templates.
#pragma once

#include <stdio.h>

#include <type_traits>

#include "tg_f32.hpp"
#include "tg_mfma.hpp"
#include "tg_thin.hpp"
#include "tg_thin_mfma.hpp"

namespace tg {

// WAVES: waves per SIMD the kernel is compiled for (1 lets a wave use the
// whole 512-entry register file, VGPRs plus AGPRs).
template <class Kern, int WAVES>
__global__ __launch_bounds__(Kern::NT) __attribute__((amdgpu_waves_per_eu(WAVES, WAVES)))
void gemm_kernel(GemmArgs g) {
    Kern::run(g);
}

static const char* dtype_tag(int dt) { return dt == 0 ? "f32" : dt == 1 ? "bf16" : "i8"; }

// SHIFT: which operands the kernel reads from rows that are not 16-byte
// aligned (bit 0 A, bit 1 B).  Such kernels are unlisted fallbacks.
// WITH_REM: also compile the kernel's twin that computes one more column
// of C in the same K loop (MfmaGemm's REM), for split plans.
template <class Tr, int BM, int BN, int BK, int WM, int WN, int S, int LD, int LY, int AC, int FR,
          int WAVES, int SHIFT = 0, int CST = CST_MFMA, bool SPREAD = false, int FREAD = RD_AUTO,
          bool WITH_REM = false, bool LATE = false>
KernelEntry mfma_entry(int dtype) {
    static_assert(!SPREAD || LD == LD_DIRECT, "spread copies: the direct loader");
    static_assert(!(SPREAD && LATE) && !(WITH_REM && LATE), "one copy schedule; no remainder twin");
    typedef MfmaGemm<Tr, BM, BN, BK, WM, WN, S, LD, LY, AC, FR, SHIFT, CST, SPREAD, FREAD, false, LATE> K;
    KernelEntry e{};
    e.dtype = dtype;
    e.family = FAM_TILED;
    e.bm = BM;
    e.bn = BN;
    e.bk = BK;
    e.stages = S;
    e.loader = LD;
    e.layout = LY;
    e.access = AC;
    e.frag = FR;
    e.wm = WM;
    e.wn = WN;
    e.store = CST == CST_SWAP ? 1 : 2;  // TGEMM_STORE_VECTOR / TGEMM_STORE_SCALAR
    e.copy_sched = LATE ? 3 : SPREAD ? 2 : 1;  // TGEMM_COPY_LATE / _SPREAD / _BURST
    e.lane_map = 1;
    e.frag_read = K::FREAD;             // TGEMM_READ_* (same values as FragRead)
    e.gload_bytes = AC == AC_WIDE ? 16 : 4;
    e.threads = K::NT;
    e.lds_bytes = K::LDS_BYTES;
    e.loads_per_stage = AC == AC_WIDE ? K::N_LD : K::A_DW + K::B_DW;
    // the direct loader reads B whose N is not a whole number of 16-byte
    // chunks (bit 1); register-staged kernels need their SHIFT bits
    e.shift_mask = SHIFT | (LD == LD_DIRECT && AC == AC_WIDE ? 2 : 0);
    e.listed = SHIFT == 0;
    e.tail_ok = 1;
    e.waves_per_simd = WAVES;
    e.fn = gemm_kernel<K, WAVES>;
    if constexpr (WITH_REM)
        e.rem_fn = gemm_kernel<MfmaGemm<Tr, BM, BN, BK, WM, WN, S, LD, LY, AC, FR, SHIFT, CST, SPREAD, FREAD, true>,
                               WAVES>;
    snprintf(e.name, sizeof e.name, "%s_t%dx%dx%d_w%dx%d_s%d_%s_%s_%s_%s%s%s%s%s", dtype_tag(dtype), BM, BN,
             BK, WM, WN, S, LD == LD_DIRECT ? "direct" : "vgpr",
             LY == LY_XOR ? "xor" : LY == LY_XOR_POISON ? "xorpoison" : "plain",
             AC == AC_WIDE ? "wide" : "narrow", FR == FR_REUSE ? "reuse" : FR == FR_SLICE ? "slice" : "permma",
             SHIFT == 1 ? "_shiftA" : SHIFT == 2 ? "_shiftB" : SHIFT == 3 ? "_shiftAB" : "",
             CST == CST_SWAP ? "_vst" : "", SPREAD ? "_spread" : LATE ? "_late" : "",
             FREAD == RD_AUTO ? "" : FREAD == RD_B32 ? "_rd32" : FREAD == RD_B64 ? "_rd64" :
             FREAD == RD_B128 ? "_rd128" : "_rdtr");
    return e;
}

template <int DT>
KernelEntry naive_entry() {
    typedef NaiveGemm<DT> K;
    KernelEntry e{};
    e.dtype = DT;
    e.family = FAM_NAIVE;
    e.bm = K::BM;
    e.bn = K::BN;
    e.bk = 1;
    e.stages = 1;
    e.loader = LD_VGPR;
    e.layout = LY_PLAIN;
    e.access = AC_NARROW;
    e.frag = FR_PER_MMA;
    e.wm = 4;
    e.wn = 1;
    e.gload_bytes = 0;
    e.threads = K::NT;
    e.lds_bytes = 0;
    e.loads_per_stage = 0;
    e.shift_mask = 3;  // element loads only
    e.listed = 1;
    e.tail_ok = 1;
    e.waves_per_simd = 4;
    e.copy_sched = 1;
    e.frag_read = 1;  // no LDS: element loads straight from memory
    e.lane_map = 1;
    e.fn = gemm_kernel<K, 4>;
    snprintf(e.name, sizeof e.name, "%s_naive", dtype_tag(DT));
    return e;
}

// The thin-N kernel (N <= NB <= THIN_N_MAX, bf16 / int8): unlisted, chosen
// by the planner for thin products and for the narrow remainder of a split
// plan (the smallest NB that covers N).  COL: the one-column twin for a
// contiguous B column (N = 1, ldb = 1): 256-thread workgroups of 4 rows
// (4095 x 1 x 4104 bf16: 6.8 us against 7.3 with 1024 threads; with B's
// column strided the 1024-thread kernel takes 11.4 us against 21.8).
// ROWS: rows of C per wave (the planner takes more for larger M).
template <int DT, int NB, bool COL = false, int ROWS = 1>
KernelEntry thin_entry() {
    static_assert(!COL || (NB == 1 && ROWS == 1), "the contiguous-column twin has one column, one row per wave");
    typedef typename std::conditional<COL, ThinGemm<DT, 1, 1, 9, 256>, ThinGemm<DT, NB, ROWS>>::type K;
    KernelEntry e{};
    e.dtype = DT;
    e.family = FAM_THIN;
    e.bm = K::BM;
    e.bn = K::BN;
    e.bk = K::KC;  // K per chunk
    e.stages = 2;
    e.loader = LD_VGPR;
    e.layout = LY_PLAIN;
    e.access = AC_WIDE;
    e.frag = FR_REUSE;
    e.wm = K::NT / 64;
    e.wn = 1;
    e.gload_bytes = 16;  // A in 16-byte (int8: 8-byte) pieces at any alignment; B by element or piece
    e.threads = K::NT;
    e.lds_bytes = K::LDS_BYTES;
    e.loads_per_stage = K::ROWS + K::BPT;
    e.shift_mask = 3;  // any alignment, any N
    e.listed = 0;
    e.tail_ok = 1;
    e.waves_per_simd = K::WAVES;
    e.copy_sched = 1;
    e.frag_read = 3;  // A streamed in 16-byte pieces
    e.lane_map = 1;
    e.fn = gemm_kernel<K, K::WAVES>;
    e.thin_col = COL;
    if (ROWS > 1)
        snprintf(e.name, sizeof e.name, "%s_thin_n%d_r%d", dtype_tag(DT), NB, ROWS);
    else
        snprintf(e.name, sizeof e.name, COL ? "%s_thin_n%d_col" : "%s_thin_n%d", dtype_tag(DT), NB);
    return e;
}

// fp32 kernels (tg_f32.hpp), by flag set.  Variant fields: loader, access
// (global load width), frag (register reuse), frag_read (A's fragment: 4-byte
// reads of row-major A, 16-byte reads of transposed A, or 16-byte reads along
// K), lds_layout (PLAIN, or XOR for the padded rows of transposed A),
// lane_map (contiguous blocks, 4 x 4 quarters, Z-order lanes) and store.
template <int S, int FLAGS, int BK = 8, int TILE = 128, int TILE_N = TILE>
KernelEntry f32_flags_entry() {
    typedef F32Gemm<S, FLAGS, BK, TILE, TILE_N> K;
    // 8 x 8 outputs per lane take ~140 registers (3 waves per SIMD); 4 x 4
    // take few enough for 4
    constexpr int WAVES = TILE == 128 ? 2 : 4;  // 8 x 16 outputs per lane: 2 as well
    KernelEntry e{};
    e.dtype = 0;
    e.family = FAM_TILED;
    e.bm = K::BM;
    e.bn = K::BN;
    e.bk = K::BK;
    e.stages = S;
    e.loader = K::DIRECT ? LD_DIRECT : LD_VGPR;
    e.layout = K::PAD_A ? LY_XOR : LY_PLAIN;
    e.access = K::WIDE_G ? AC_WIDE : AC_NARROW;
    e.frag = K::REUSE ? FR_REUSE : FR_PER_MMA;
    e.frag_read = K::TRANS_A ? RD_B128 : K::AKVEC ? 5 : RD_B32;  // 5: TGEMM_READ_KVEC
    e.lane_map = K::QUARTERS ? (K::ZORDER ? 4 : 2) : (K::ZORDER ? 3 : 1);
    e.store = K::VEC_STORE ? 1 : 2;      // TGEMM_STORE_VECTOR / TGEMM_STORE_SCALAR
    e.copy_sched = 1;
    e.gload_bytes = K::WIDE_G ? 16 : 4;
    e.wm = 2;
    e.wn = 2;
    e.threads = K::NT;
    e.lds_bytes = K::LDS_BYTES;
    e.loads_per_stage = K::WIDE_G ? K::N_LD : K::EA + K::EB;
    e.shift_mask = K::DIRECT ? 0 : 3;  // register-staged kernels have their own guarded element loads
    e.listed = 1;
    e.tail_ok = 1;
    e.waves_per_simd = WAVES;
    e.fn = gemm_kernel<K, WAVES>;
    snprintf(e.name, sizeof e.name, "f32_t%dx%dx%d_w2x2_s%d_%s_%s_%s%s_%s%s_%s", TILE, TILE_N, BK, S,
             K::DIRECT ? "direct" : "vgpr", K::WIDE_G ? "g16" : "g4",
             K::TRANS_A ? "transA" : K::AKVEC ? "kvecA" : "rowA", K::PAD_A ? "_pad" : "",
             K::QUARTERS ? (K::ZORDER ? "zquarters" : "quarters") : (K::ZORDER ? "zorder" : "blocks"),
             K::REUSE ? "" : "_permfma", K::VEC_STORE ? "vecstore" : "scalarstore");
    return e;
}

// The production form: transposed A with padded rows, quarters, 16-byte C
// stores (flags of the fully switched-on ladder), at S stages.
template <int S, int BK = 8, int TILE = 128, int TILE_N = TILE>
KernelEntry f32_entry() {
    return f32_flags_entry<S, F_TRANS_A | F_PAD_A | F_QUARTERS | F_VEC_STORE, BK, TILE, TILE_N>();
}

// The matrix-core thin kernel (bf16 NB 4, 8, 16; int8 8, 16): unlisted,
// preferred by the planner for 2..16 columns whose B rows allow its 8- or
// 16-byte row pieces (NB <= ldb + N).  RB: 16-row blocks per workgroup (the
// planner takes the most that still give 256 workgroups).  P, the matrix
// steps per wave per chunk: as many as two B slots leave room for in LDS,
// at most 9 (16 x 9 steps of 64 bytes cover K = 4608 bf16 in one chunk);
// with more row blocks the measured best (x 7 x 4104 bf16, x 9 x 4104
// int8): 2 blocks 6 bf16 (8192 rows: 15.0 us against 16.2 with 4 or 2), 4
// int8 (9.5); 4 blocks 1 bf16 (16384 rows: 26.5 us against 35.6 with 2 and
// 42.0 with 3), 2 int8 (17.7 against 18.3 with 3 and 19.6 with 1).
template <int DT, int NB, int RB>
KernelEntry thin_mma_entry() {
    constexpr int P1 = 163824 / (2048 * NB) < 9 ? 163824 / (2048 * NB) : 9;
    constexpr int PR = RB == 1 ? 9 : RB == 2 ? (DT == 1 ? 6 : 4) : (DT == 1 ? 1 : 2);
    constexpr int P = P1 < PR ? P1 : PR;
    typedef ThinMfma<DT, NB, RB, P> K;
    static_assert(K::LDS_BYTES <= 163840, "LDS");
    KernelEntry e{};
    e.dtype = DT;
    e.family = FAM_THIN;
    e.bm = K::BM;
    e.bn = K::BN;
    e.bk = K::KC;  // K per chunk
    e.stages = 2;
    e.loader = LD_VGPR;
    e.layout = LY_PLAIN;
    e.access = AC_WIDE;
    e.frag = FR_REUSE;
    e.wm = K::NT / 64;
    e.wn = 1;
    e.gload_bytes = 16;  // A in 16-byte pieces at any alignment; B in 8- or 16-byte row pieces
    e.threads = K::NT;
    e.lds_bytes = K::LDS_BYTES;
    e.loads_per_stage = P * RB + K::BPT;
    e.shift_mask = 3;  // any alignment; B only where NB <= ldb + N (the planner checks)
    e.listed = 0;
    e.tail_ok = 1;
    e.waves_per_simd = K::WAVES;
    e.copy_sched = 1;
    e.frag_read = 0;  // transposing reads of B
    e.lane_map = 1;
    e.fn = gemm_kernel<K, K::WAVES>;
    e.thin_mma = 1;
    if (RB > 1)
        snprintf(e.name, sizeof e.name, "%s_thin_mma_n%d_r%d", dtype_tag(DT), NB, RB);
    else
        snprintf(e.name, sizeof e.name, "%s_thin_mma_n%d", dtype_tag(DT), NB);
    return e;
}

}  // namespace tg
