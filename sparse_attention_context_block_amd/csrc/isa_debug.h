// Diagnostic switches set through isa_debug_set_flags (include/isa.h) and read
// by the kernel launchers.
#pragma once
#include <stdint.h>

namespace isa {
// The flags last set by isa_debug_set_flags (0 by default).
uint32_t debug_flags();
// Matches ISA_DEBUG_GLOBAL_TABLES: the block-mask and Taylor kernels read
// their tables from global memory even where the copy in LDS would fit.
constexpr uint32_t kDebugGlobalTables = 1u;
}  // namespace isa
