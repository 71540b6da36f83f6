// fp32 vector-FMA kernel variants compiled into libtgemm.
#include "tg_kernels.hpp"

namespace tg {

void register_f32(void (*add)(const KernelEntry&)) {
    // production: every rung on, Z-order lanes (4096^3: 1467 against 1479 us
    // with row-major lanes, interleaved), 16-deep K slices (interleaved
    // against 8: 4096^3 1509 vs 1546 us, 2048^3 309 vs 339, 1024^3 156 vs
    // 171; 32-deep slices were no faster and take 170 VGPRs)
    add(f32_flags_entry<2, F_TRANS_A | F_PAD_A | F_QUARTERS | F_ZORDER | F_VEC_STORE, 16>());
    add(f32_entry<2, 16>());
    add(f32_entry<2>());
    // 64 x 64 tiles (4 x 4 outputs per lane) for grids that would leave most
    // SIMDs idle on 128 x 128 tiles
    add(f32_flags_entry<2, F_TRANS_A | F_PAD_A | F_QUARTERS | F_ZORDER | F_VEC_STORE, 16, 64>());
    add(f32_entry<2, 16, 64>());
    add(f32_entry<2, 16, 128, 256>());
    add(f32_entry<2, 32, 64>());
    // the SIMT ladder on the 128 x 128 x 8 tile, one change per rung (the SM80
    // ablation plan, section 1.5.4; the GEMM page, sections 4-10):
    //   block tiling, 4-byte loads, operands read from LDS for every FMA
    add(f32_flags_entry<1, F_GLOBAL4 | F_NO_REUSE>());
    //   + register tiling (fragments read once per k step)
    add(f32_flags_entry<1, F_GLOBAL4>());
    //   + 16-byte global loads and LDS writes
    add(f32_flags_entry<1, 0>());
    //   + A transposed in LDS: 16-byte fragment reads
    add(f32_flags_entry<1, F_TRANS_A>());
    //   + padded rows of transposed A (conflict-free A writes)
    add(f32_flags_entry<1, F_TRANS_A | F_PAD_A>());
    //   + 4 x 4 quarters per lane (section 8.5, scheme 4), or instead Z-order
    //     lanes (scheme 3), or both
    add(f32_flags_entry<1, F_TRANS_A | F_PAD_A | F_QUARTERS>());
    add(f32_flags_entry<1, F_TRANS_A | F_PAD_A | F_ZORDER>());
    add(f32_flags_entry<1, F_TRANS_A | F_PAD_A | F_QUARTERS | F_ZORDER>());
    //   + 16-byte C stores
    add(f32_flags_entry<1, F_TRANS_A | F_PAD_A | F_QUARTERS | F_VEC_STORE>());
    //   + register-staged double buffer: f32_entry<2> above
    //   A row-major, read as 16-byte pieces along K (the layout a direct copy
    //   gives), register-staged double buffer
    add(f32_flags_entry<2, F_AKVEC | F_QUARTERS | F_VEC_STORE>());
    //   + direct-to-LDS copies, 2 slots, then 3 and 4
    add(f32_flags_entry<2, F_AKVEC | F_QUARTERS | F_VEC_STORE | F_DIRECT>());
    add(f32_flags_entry<3, F_AKVEC | F_QUARTERS | F_VEC_STORE | F_DIRECT>());
    add(f32_flags_entry<4, F_AKVEC | F_QUARTERS | F_VEC_STORE | F_DIRECT>());
    //   the same with 16-deep slices
    add(f32_flags_entry<2, F_AKVEC | F_QUARTERS | F_VEC_STORE, 16>());
    add(f32_flags_entry<2, F_AKVEC | F_QUARTERS | F_VEC_STORE | F_DIRECT, 16>());
    add(f32_flags_entry<3, F_AKVEC | F_QUARTERS | F_VEC_STORE | F_DIRECT, 16>());
    add(f32_flags_entry<4, F_AKVEC | F_QUARTERS | F_VEC_STORE | F_DIRECT, 16>());
    add(f32_flags_entry<2, F_TRANS_A | F_PAD_A | F_QUARTERS | F_ZORDER | F_VEC_STORE, 16, 128, 256>());
    add(naive_entry<0>());
}

}  // namespace tg
