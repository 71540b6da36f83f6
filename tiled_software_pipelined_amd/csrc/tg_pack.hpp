// Operand repack (tg_pack.hip): the host entry.
#pragma once

#include <hip/hip_runtime.h>

#include "tg_args.hpp"

namespace tg {

// Enqueue the repack of `a` on `stream`.
hipError_t launch_pack(const PackArgs& a, hipStream_t stream);

}  // namespace tg
