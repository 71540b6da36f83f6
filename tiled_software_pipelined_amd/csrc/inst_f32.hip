// fp32 vector-FMA kernel variants compiled into libtgemm.
#include "tg_kernels.hpp"

namespace tg {

void register_f32(void (*add)(const KernelEntry&)) {
    // production: every rung on, 16-deep K slices (interleaved against 8:
    // 4096^3 1509 vs 1546 us, 2048^3 309 vs 339, 1024^3 156 vs 171; 32-deep
    // slices were no faster and take 170 VGPRs)
    add(f32_entry<2, true, true, true, 16>());
    add(f32_entry<2, true, true, true>());
    // 64 x 64 tiles (4 x 4 outputs per lane) for grids that would leave most
    // SIMDs idle on 128 x 128 tiles
    add(f32_entry<2, true, true, true, 16, 64>());
    add(f32_entry<2, true, true, true, 16, 128, 256>());
    add(f32_entry<2, true, true, true, 32, 64>());
    // the SIMT ladder, one change per rung (the SM80 ablation plan, section
    // 1.5.4): tiling -> + A transposed -> + conflict-free layout ->
    // + coalesced write-back -> + double buffer
    add(f32_entry<1, true, true, true>());
    add(f32_entry<1, true, true, false>());
    add(f32_entry<1, true, false, false>());
    add(f32_entry<1, false, false, false>());
    add(naive_entry<0>());
}

}  // namespace tg
