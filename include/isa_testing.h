/*
 * isa_testing.h -- test hooks of the ISA library (libisa.so).
 *
 * Not part of the product API in isa.h: nothing here is needed to run ISA, and
 * a caller that only includes isa.h never changes what these hooks control.
 * They exist for the library's own tests, which reach kernel paths and error
 * paths that the default dispatch and the shapes of small test cases do not.
 * Every hook is process-wide state read on the host when an entry point of
 * isa.h issues its launches: set it while no other thread issues launches.
 */
#ifndef ISA_TESTING_H
#define ISA_TESTING_H

#include <stdint.h>

#include "isa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel-path switches.
 * - ISA_DEBUG_GLOBAL_TABLES makes the block-mask (flat) and Taylor kernels read
 *   their block and row tables from global memory, the path they otherwise take
 *   only when a table is too long for its LDS copy (more than 896 entries for
 *   the block mask, 2048 rows for the Taylor path).  Results are the same
 *   either way.
 * - ISA_DEBUG_4WAVE_EXACT runs the bf16 launches that read whole blocks through
 *   a block table (the exact path, the dense baseline) on the 4-wave kernel
 *   that otherwise serves only the Taylor path (a slower alternative with the
 *   same arithmetic per row, for comparison).
 * - ISA_DEBUG_PINGPONG_EXACT runs the same launches on the 8-wave ping-pong
 *   kernel, which otherwise serves only head dimension 64 and 32-token blocks.
 * Applies to launches issued after the call.  Returns ISA_ERR_INVALID_ARG (and
 * changes nothing) for unknown bits or for both exact-path switches at once. */
#define ISA_DEBUG_GLOBAL_TABLES 1u
#define ISA_DEBUG_4WAVE_EXACT 2u
#define ISA_DEBUG_PINGPONG_EXACT 4u
isa_status_t isa_debug_set_flags(uint32_t flags);

/* Failure injection for the launch wrapper: the next `skip` launches of any
 * entry point run normally, then the wrapper returns hip_error for the launch
 * after them without issuing it (so no kernel runs and the GPU is never
 * touched), and the hook disarms.  The entry point then reports ISA_ERR_HIP
 * and isa_last_hip_error() returns hip_error, exactly as for a real failed
 * launch.  hip_error 0 disarms.  Returns ISA_ERR_INVALID_ARG for skip < 0 or
 * hip_error < 0. */
isa_status_t isa_testing_fail_launch(int32_t skip, int32_t hip_error);

#ifdef __cplusplus
}
#endif

#endif /* ISA_TESTING_H */
