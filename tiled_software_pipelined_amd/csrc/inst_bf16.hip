// bf16 kernel variants compiled into libtgemm.  Order matters: for a given
// set of requested fields the first matching entry wins.
#include "tg_kernels.hpp"

namespace tg {

void register_bf16(void (*add)(const KernelEntry&)) {
    typedef TraitsBF16 T;
    // production tiles (the 8-wave 256 x 256 x 64 is the default for large shapes)
    add(mfma_entry<T, 256, 256, 64, 2, 4, 2, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2, 0, CST_MFMA, false, RD_AUTO, true>(1));
    add(mfma_entry<T, 256, 256, 64, 2, 2, 2, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 1>(1));
    add(mfma_entry<T, 256, 256, 32, 2, 2, 3, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 1>(1));
    add(mfma_entry<T, 256, 256, 32, 2, 2, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 1>(1));
    add(mfma_entry<T, 256, 128, 64, 2, 2, 2, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 1>(1));
    // two workgroups per CU (2 waves per SIMD): one's barrier hidden by the other
    add(mfma_entry<T, 256, 128, 32, 2, 2, 2, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2>(1));
    add(mfma_entry<T, 128, 256, 32, 2, 2, 2, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2>(1));
    add(mfma_entry<T, 256, 256, 32, 2, 4, 2, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2>(1));
    add(mfma_entry<T, 256, 256, 32, 2, 4, 3, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2>(1));
    add(mfma_entry<T, 256, 256, 32, 2, 4, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2>(1));
    add(mfma_entry<T, 256, 256, 64, 2, 2, 2, LD_VGPR, LY_XOR, AC_WIDE, FR_REUSE, 1>(1));
    add(mfma_entry<T, 256, 256, 64, 2, 4, 2, LD_VGPR, LY_XOR, AC_WIDE, FR_REUSE, 2>(1));
    // small problems: more workgroups per CU count
    add(mfma_entry<T, 64, 64, 64, 2, 2, 3, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 4>(1));
    // a deep ring for small grids (about one workgroup per compute unit),
    // where each slice's load latency is exposed unless many are in flight
    add(mfma_entry<T, 64, 64, 64, 2, 2, 8, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 4>(1));
    // half tiles: twice the workgroups where 128 x 128 tiles fill at most
    // half the compute units
    add(mfma_entry<T, 128, 64, 32, 2, 2, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2>(1));
    add(mfma_entry<T, 64, 128, 32, 2, 2, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2>(1));
    // the 128 x 128 x 32 ladder, one change per step
    add(mfma_entry<T, 128, 128, 32, 2, 2, 3, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2>(1));
    add(mfma_entry<T, 128, 128, 32, 2, 2, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2>(1));
    add(mfma_entry<T, 128, 128, 32, 2, 2, 2, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2>(1));
    add(mfma_entry<T, 128, 128, 32, 2, 2, 2, LD_VGPR, LY_XOR, AC_WIDE, FR_REUSE, 2>(1));
    // the asynchronous copy with a single buffer: no overlap to gain
    add(mfma_entry<T, 128, 128, 32, 2, 2, 1, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2>(1));
    add(mfma_entry<T, 128, 128, 32, 2, 2, 1, LD_VGPR, LY_XOR, AC_WIDE, FR_REUSE, 2>(1));
    add(mfma_entry<T, 128, 128, 32, 2, 2, 1, LD_VGPR, LY_PLAIN, AC_WIDE, FR_REUSE, 2>(1));
    add(mfma_entry<T, 128, 128, 32, 2, 2, 1, LD_VGPR, LY_PLAIN, AC_NARROW, FR_REUSE, 2>(1));
    add(mfma_entry<T, 128, 128, 32, 2, 2, 1, LD_VGPR, LY_PLAIN, AC_NARROW, FR_PER_MMA, 2>(1));
    // 16-byte global loads and LDS writes with the narrow rung's 4-byte
    // fragment reads: the global-load width and the fragment-read width are
    // separate rungs
    add(mfma_entry<T, 128, 128, 32, 2, 2, 1, LD_VGPR, LY_PLAIN, AC_WIDE, FR_REUSE, 2, 0, CST_MFMA, false, RD_B32>(1));
    // the fragment-read ladder on the direct loader, 3 slots, XOR layout:
    // A by 4 / 8 / 16-byte reads with B by element reads (then the
    // transposing B reads: the 3-slot kernel above)
    add(mfma_entry<T, 128, 128, 32, 2, 2, 3, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2, 0, CST_MFMA, false, RD_B32>(1));
    add(mfma_entry<T, 128, 128, 32, 2, 2, 3, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2, 0, CST_MFMA, false, RD_B64>(1));
    add(mfma_entry<T, 128, 128, 32, 2, 2, 3, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2, 0, CST_MFMA, false, RD_B128>(1));
    // whole-slice fragment read-ahead for tiles whose waves issue one or two
    // matrix instructions per K step (small grids)
    add(mfma_entry<T, 64, 64, 64, 2, 2, 8, LD_DIRECT, LY_XOR, AC_WIDE, FR_SLICE, 4>(1));
    add(mfma_entry<T, 64, 64, 64, 2, 2, 3, LD_DIRECT, LY_XOR, AC_WIDE, FR_SLICE, 4>(1));
    add(mfma_entry<T, 64, 64, 128, 2, 2, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_SLICE, 4>(1));
    add(mfma_entry<T, 64, 64, 128, 2, 2, 3, LD_DIRECT, LY_XOR, AC_WIDE, FR_SLICE, 4>(1));
    add(mfma_entry<T, 128, 64, 32, 2, 2, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_SLICE, 2>(1));
    add(mfma_entry<T, 64, 128, 32, 2, 2, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_SLICE, 2>(1));
    add(mfma_entry<T, 128, 128, 32, 2, 2, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_SLICE, 2>(1));
    add(naive_entry<1>());
    // unlisted: thin products (N <= 16) and split-plan remainders: one
    // column on the vector ALUs, 2..16 on the matrix cores
    add(thin_entry<1, 1>());
    add(thin_entry<1, 1, true>());
    add(thin_entry<1, 1, false, 2>());
    add(thin_entry<1, 1, false, 4>());
    add(thin_mma_entry<1, 4, 1>());
    add(thin_mma_entry<1, 8, 1>());
    add(thin_mma_entry<1, 16, 1>());
    add(thin_mma_entry<1, 4, 2>());
    add(thin_mma_entry<1, 8, 2>());
    add(thin_mma_entry<1, 16, 2>());
    add(thin_mma_entry<1, 4, 4>());
    add(thin_mma_entry<1, 8, 4>());
    add(thin_mma_entry<1, 16, 4>());
    // unlisted: the register-staged defaults reading rows that are not
    // 16-byte aligned (A only, B only, both)
    add(mfma_entry<T, 256, 256, 64, 2, 4, 2, LD_VGPR, LY_XOR, AC_WIDE, FR_REUSE, 2, 1>(1));
    add(mfma_entry<T, 256, 256, 64, 2, 4, 2, LD_VGPR, LY_XOR, AC_WIDE, FR_REUSE, 2, 2>(1));
    add(mfma_entry<T, 256, 256, 64, 2, 4, 2, LD_VGPR, LY_XOR, AC_WIDE, FR_REUSE, 2, 3>(1));
    add(mfma_entry<T, 128, 128, 32, 2, 2, 2, LD_VGPR, LY_XOR, AC_WIDE, FR_REUSE, 2, 1>(1));
    add(mfma_entry<T, 128, 128, 32, 2, 2, 2, LD_VGPR, LY_XOR, AC_WIDE, FR_REUSE, 2, 2>(1));
    add(mfma_entry<T, 128, 128, 32, 2, 2, 2, LD_VGPR, LY_XOR, AC_WIDE, FR_REUSE, 2, 3>(1));
    // debug twins of the direct-loader defaults with poisoned slots: listed
    // last, so only a request for TGEMM_LDS_XOR_POISON reaches them
    add(mfma_entry<T, 256, 256, 64, 2, 4, 2, LD_DIRECT, LY_XOR_POISON, AC_WIDE, FR_REUSE, 2>(1));
    add(mfma_entry<T, 128, 128, 32, 2, 2, 4, LD_DIRECT, LY_XOR_POISON, AC_WIDE, FR_REUSE, 2>(1));
    add(mfma_entry<T, 64, 128, 32, 2, 2, 4, LD_DIRECT, LY_XOR_POISON, AC_WIDE, FR_REUSE, 2>(1));
    add(mfma_entry<T, 64, 64, 64, 2, 2, 8, LD_DIRECT, LY_XOR_POISON, AC_WIDE, FR_REUSE, 4>(1));
    add(mfma_entry<T, 64, 64, 64, 2, 2, 8, LD_DIRECT, LY_XOR_POISON, AC_WIDE, FR_SLICE, 4>(1));
    add(mfma_entry<T, 64, 64, 64, 2, 2, 3, LD_DIRECT, LY_XOR_POISON, AC_WIDE, FR_SLICE, 4>(1));
    // 16-byte C stores from the swapped product (TGEMM_STORE_VECTOR)
    add(mfma_entry<T, 256, 256, 64, 2, 4, 2, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2, 0, CST_SWAP>(1));
    add(mfma_entry<T, 256, 256, 32, 2, 4, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2, 0, CST_SWAP>(1));
    add(mfma_entry<T, 256, 256, 64, 2, 2, 2, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 1, 0, CST_SWAP>(1));
    add(mfma_entry<T, 256, 256, 32, 2, 2, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 1, 0, CST_SWAP>(1));
    add(mfma_entry<T, 256, 256, 32, 2, 2, 3, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 1, 0, CST_SWAP>(1));
    // copies spread over the K steps (TGEMM_COPY_SPREAD)
    add(mfma_entry<T, 256, 256, 32, 2, 2, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 1, 0, CST_SWAP, true>(1));
    add(mfma_entry<T, 256, 256, 32, 2, 2, 3, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 1, 0, CST_SWAP, true>(1));
    add(mfma_entry<T, 256, 256, 64, 2, 2, 2, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 1, 0, CST_SWAP, true>(1));
    add(mfma_entry<T, 256, 256, 32, 2, 4, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2, 0, CST_MFMA, true>(1));
    add(mfma_entry<T, 256, 256, 64, 2, 4, 2, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2, 0, CST_MFMA, true>(1));
    // the default with the slice's barrier later in the last K step
    // (TGEMM_COPY_LATE): the power-cap measurement's twin
    add(mfma_entry<T, 256, 256, 64, 2, 4, 2, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2, 0, CST_MFMA, false, RD_AUTO,
                   false, true>(1));
}

}  // namespace tg
