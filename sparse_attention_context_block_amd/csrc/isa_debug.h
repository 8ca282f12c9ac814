// Kernel-path switches set through isa_debug_set_flags (include/isa_testing.h,
// test hooks only) and read by the kernel launchers.
#pragma once
#include <stdint.h>

namespace isa {
// The flags last set by isa_debug_set_flags (0 by default).
uint32_t debug_flags();
// Matches ISA_DEBUG_GLOBAL_TABLES: the block-mask and Taylor kernels read
// their tables from global memory even where the copy in LDS would fit.
constexpr uint32_t kDebugGlobalTables = 1u;
// Matches ISA_DEBUG_4WAVE_EXACT: block-table launches of the bf16 attention
// (exact path, dense baseline) run on the 4-wave kernel.
constexpr uint32_t kDebug4WaveExact = 2u;
// Matches ISA_DEBUG_PINGPONG_EXACT: the same launches run on the 8-wave
// ping-pong kernel.
constexpr uint32_t kDebugPingPongExact = 4u;
constexpr uint32_t kDebugAll = kDebugGlobalTables | kDebug4WaveExact | kDebugPingPongExact;
}  // namespace isa
