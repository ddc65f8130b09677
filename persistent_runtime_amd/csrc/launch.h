// launch.h -- host-side launchers of the device code in kernels.hip.
#pragma once
#include <hip/hip_runtime.h>

#include "mk_task.h"

namespace mk {

// One decode step as a single persistent launch: `grid` workgroups (one per
// CU) pull tickets until the task list is exhausted.  `d` is a device copy.
// mode: 0 any batch on the vector path, 1 a single slot, 2 matrix-core
// GEMVs (batches of 16..64 slots)
hipError_t launch_persistent(const DevPlan *d, const CallArgs &ca, int grid, int mode,
                             hipStream_t s);

// Scheduled executor: workgroup 0 runs the schedulers, 1..grid-1 the
// workers (d must hold the scheduled executor's queues and tables).
hipError_t launch_sched(const DevPlan *d, const CallArgs &ca, int grid, hipStream_t s);

// Kernel-per-op: tasks [first, first+count) of one launch phase, one
// workgroup per task, no counters (stream order orders the phases).
hipError_t launch_phase(const DevPlan *d, const CallArgs &ca, int first, int count,
                        hipStream_t s);

// Prefill staging: slot `slot` gets tokens[i] at position start+i, every
// other slot is marked empty.
hipError_t launch_stage(int32_t *stage_tok, int32_t *stage_pos, int B, int slot,
                        const int32_t *tokens, int i, int start, hipStream_t s);

// Prompt-chunk staging: slot j < cnt gets tokens[j] at position start + j of
// page-table row `row`; slots cnt..B-1 are empty.
hipError_t launch_stage_chunk(int32_t *stage_tok, int32_t *stage_pos, int32_t *stage_rows, int B,
                              const int32_t *tokens, int cnt, int start, int row, hipStream_t s);

// Zero n words (counter reset between epochs).
// p[0] += 1, skipping 0 (the data tag of graph-replayed steps)
hipError_t launch_bump_tag(uint32_t *p, hipStream_t s);

hipError_t launch_zero_u32(uint32_t *p, int n, hipStream_t s);

// Resource use of the persistent kernel (for reports).
int persistent_lds_bytes();

// The device's copy of the library's static scratch array (kStaticScratchBytes,
// 256-byte aligned), for plans that allocate no device memory.  `device` must
// be the current device; its address is looked up once per device.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
hipError_t static_scratch(int device, void **ptr);

}  // namespace mk
