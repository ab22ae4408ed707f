// Test hooks of libmc2.  Exported from the library like the calls of
// include/mc2.h but not part of its interface: they exist so that tests can
// drive paths that normal inputs never reach.  Process-wide settings; not
// for production use.
#pragma once
#include <stdint.h>

#include "mc2.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Arrival emulation of mc2_allgather_matmul (mode MC2_AG_ARRIVAL): the
 * settings later calls use, process-wide.
 *   wait_ticks   -- longest wait of a GEMM wavefront for one piece of the
 *                   gathered matrix, in ticks of the GPU's 100 MHz real-time
 *                   counter; 0 restores the default of 200 ms.  A wait that
 *                   runs out reads the rest of A from the shards and is
 *                   counted by mc2_allgather_arrival_fallbacks.
 *   raised_slabs -- the copy kernel raises the ready flags of the first
 *                   raised_slabs slabs of K only (it still copies every
 *                   piece); negative restores "all".  Withheld flags make
 *                   every wait on those slabs run out, so the time-out path
 *                   runs while every kernel still exits normally.
 * Always returns MC2_OK. */
mc2_status mc2_testing_arrival(uint64_t wait_ticks, int raised_slabs);

#ifdef __cplusplus
}
#endif
