// fp32 vector-FMA kernel variants compiled into libtgemm.
#include "tg_kernels.hpp"

namespace tg {

void register_f32(void (*add)(const KernelEntry&)) {
    add(f32_entry<2>());
    add(f32_entry<1>());
    add(naive_entry<0>());
}

}  // namespace tg
