// int8 kernel variants compiled into libtgemm (same bytes per slice as the
// bf16 ones: BK doubles because an element is one byte).
#include "tg_kernels.hpp"

namespace tg {

void register_i8(void (*add)(const KernelEntry&)) {
    typedef TraitsI8 T;
    add(mfma_entry<T, 256, 256, 128, 2, 4, 2, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2, 0, CST_MFMA, false, RD_AUTO, true>(2));
    add(mfma_entry<T, 256, 256, 128, 2, 2, 2, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 1>(2));
    add(mfma_entry<T, 256, 256, 128, 2, 2, 2, LD_VGPR, LY_XOR, AC_WIDE, FR_REUSE, 1>(2));
    add(mfma_entry<T, 256, 256, 128, 2, 4, 2, LD_VGPR, LY_XOR, AC_WIDE, FR_REUSE, 2>(2));
    add(mfma_entry<T, 128, 128, 64, 2, 2, 3, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2>(2));
    add(mfma_entry<T, 128, 128, 64, 2, 2, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2>(2));
    add(mfma_entry<T, 128, 128, 64, 2, 2, 2, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2>(2));
    add(mfma_entry<T, 128, 128, 64, 2, 2, 2, LD_VGPR, LY_XOR, AC_WIDE, FR_REUSE, 2>(2));
    add(mfma_entry<T, 128, 128, 64, 2, 2, 1, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2>(2));
    add(mfma_entry<T, 64, 64, 128, 2, 2, 3, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 4>(2));
    add(mfma_entry<T, 64, 64, 128, 2, 2, 8, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 4>(2));
    // half tiles: twice the workgroups where 128 x 128 tiles fill at most
    // half the compute units
    add(mfma_entry<T, 128, 64, 64, 2, 2, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2>(2));
    add(mfma_entry<T, 64, 128, 64, 2, 2, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2>(2));
    // the 128 x 128 x 64 ladder below the 1-slot direct kernel, one change per
    // step: per-instruction 4-byte fragment reads -> fragment reuse ->
    // 16-byte global loads / LDS writes -> 16-byte and transposing fragment
    // reads -> XOR layout
    add(mfma_entry<T, 128, 128, 64, 2, 2, 1, LD_VGPR, LY_XOR, AC_WIDE, FR_REUSE, 2>(2));
    add(mfma_entry<T, 128, 128, 64, 2, 2, 1, LD_VGPR, LY_PLAIN, AC_WIDE, FR_REUSE, 2>(2));
    add(mfma_entry<T, 128, 128, 64, 2, 2, 1, LD_VGPR, LY_PLAIN, AC_WIDE, FR_REUSE, 2, 0, CST_MFMA, false, RD_B32>(2));
    add(mfma_entry<T, 128, 128, 64, 2, 2, 1, LD_VGPR, LY_PLAIN, AC_NARROW, FR_REUSE, 2>(2));
    add(mfma_entry<T, 128, 128, 64, 2, 2, 1, LD_VGPR, LY_PLAIN, AC_NARROW, FR_PER_MMA, 2>(2));
    // the fragment-read ladder on the direct loader, 3 slots, XOR layout
    add(mfma_entry<T, 128, 128, 64, 2, 2, 3, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2, 0, CST_MFMA, false, RD_B32>(2));
    add(mfma_entry<T, 128, 128, 64, 2, 2, 3, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2, 0, CST_MFMA, false, RD_B64>(2));
    add(mfma_entry<T, 128, 128, 64, 2, 2, 3, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2, 0, CST_MFMA, false, RD_B128>(2));
    // whole-slice fragment read-ahead for tiles whose waves issue one or two
    // matrix instructions per K step (small grids)
    add(mfma_entry<T, 64, 64, 128, 2, 2, 8, LD_DIRECT, LY_XOR, AC_WIDE, FR_SLICE, 4>(2));
    add(mfma_entry<T, 64, 64, 128, 2, 2, 3, LD_DIRECT, LY_XOR, AC_WIDE, FR_SLICE, 4>(2));
    add(mfma_entry<T, 64, 64, 256, 2, 2, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_SLICE, 4>(2));
    add(mfma_entry<T, 128, 64, 64, 2, 2, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_SLICE, 2>(2));
    add(mfma_entry<T, 64, 128, 64, 2, 2, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_SLICE, 2>(2));
    add(mfma_entry<T, 128, 128, 64, 2, 2, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_SLICE, 2>(2));
    add(naive_entry<2>());
    // unlisted: thin products (N <= 16) and split-plan remainders: up to 4
    // columns on the vector ALUs where B's rows are too short for the
    // matrix-core kernel's 8-byte pieces (8 > ldb + N), one column always;
    // otherwise the matrix cores
    add(thin_entry<2, 1>());
    add(thin_entry<2, 2>());
    add(thin_entry<2, 4>());
    add(thin_entry<2, 1, false, 2>());
    add(thin_entry<2, 2, false, 2>());
    add(thin_entry<2, 4, false, 2>());
    add(thin_entry<2, 1, false, 4>());
    add(thin_entry<2, 2, false, 4>());
    add(thin_entry<2, 4, false, 4>());
    add(thin_entry<2, 1, true>());
    add(thin_mma_entry<2, 8, 1>());
    add(thin_mma_entry<2, 16, 1>());
    add(thin_mma_entry<2, 8, 2>());
    add(thin_mma_entry<2, 16, 2>());
    add(thin_mma_entry<2, 8, 4>());
    add(thin_mma_entry<2, 16, 4>());
    // unlisted: the register-staged defaults reading rows that are not
    // 16-byte aligned (A only, B only, both)
    add(mfma_entry<T, 256, 256, 128, 2, 4, 2, LD_VGPR, LY_XOR, AC_WIDE, FR_REUSE, 2, 1>(2));
    add(mfma_entry<T, 256, 256, 128, 2, 4, 2, LD_VGPR, LY_XOR, AC_WIDE, FR_REUSE, 2, 2>(2));
    add(mfma_entry<T, 256, 256, 128, 2, 4, 2, LD_VGPR, LY_XOR, AC_WIDE, FR_REUSE, 2, 3>(2));
    add(mfma_entry<T, 128, 128, 64, 2, 2, 2, LD_VGPR, LY_XOR, AC_WIDE, FR_REUSE, 2, 1>(2));
    add(mfma_entry<T, 128, 128, 64, 2, 2, 2, LD_VGPR, LY_XOR, AC_WIDE, FR_REUSE, 2, 2>(2));
    add(mfma_entry<T, 128, 128, 64, 2, 2, 2, LD_VGPR, LY_XOR, AC_WIDE, FR_REUSE, 2, 3>(2));
    // debug twins with poisoned slots (only reached by TGEMM_LDS_XOR_POISON)
    add(mfma_entry<T, 256, 256, 128, 2, 4, 2, LD_DIRECT, LY_XOR_POISON, AC_WIDE, FR_REUSE, 2>(2));
    add(mfma_entry<T, 128, 128, 64, 2, 2, 4, LD_DIRECT, LY_XOR_POISON, AC_WIDE, FR_REUSE, 2>(2));
    add(mfma_entry<T, 64, 64, 128, 2, 2, 8, LD_DIRECT, LY_XOR_POISON, AC_WIDE, FR_REUSE, 4>(2));
    add(mfma_entry<T, 64, 64, 128, 2, 2, 8, LD_DIRECT, LY_XOR_POISON, AC_WIDE, FR_SLICE, 4>(2));
    // 16-byte C stores from the swapped product (TGEMM_STORE_VECTOR)
    add(mfma_entry<T, 256, 256, 128, 2, 4, 2, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2, 0, CST_SWAP>(2));
    add(mfma_entry<T, 256, 256, 64, 2, 4, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2, 0, CST_SWAP>(2));
    add(mfma_entry<T, 256, 256, 128, 2, 2, 2, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 1, 0, CST_SWAP>(2));
    add(mfma_entry<T, 256, 256, 64, 2, 2, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 1, 0, CST_SWAP>(2));
    // copies spread over the K steps (TGEMM_COPY_SPREAD)
    add(mfma_entry<T, 256, 256, 64, 2, 2, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 1, 0, CST_SWAP, true>(2));
    add(mfma_entry<T, 256, 256, 128, 2, 4, 2, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2, 0, CST_MFMA, true>(2));
    add(mfma_entry<T, 256, 256, 64, 2, 4, 4, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2, 0, CST_MFMA, true>(2));
    // the default with the slice's barrier later in the last K step
    // (TGEMM_COPY_LATE): the power-cap measurement's twin
    add(mfma_entry<T, 256, 256, 128, 2, 4, 2, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 2, 0, CST_MFMA, false, RD_AUTO,
                   false, true>(2));
}

}  // namespace tg
