// Host-side entry points of the kernels (called by the C ABI layer after validation).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dr {

struct Params;

// Decode: one workgroup per (sequence, head); p.S is the state updated in place.
hipError_t launch_decode(const Params& p, int64_t nheads, int dk, int dv, bool bf16, bool vec,
                         hipStream_t s);

// Prefill launch shape for a problem: value columns per workgroup and grid size.
struct PrefillPlan {
  int chunk;
  int dv_block;
  int ndvb;
  int64_t workgroups;  // padded to a multiple of 8 (XCD count)
};
PrefillPlan plan_prefill(int64_t num_pairs, int dk, int dv);

// Prefill: chunkwise-parallel forward over every (sequence, head, value block).
hipError_t launch_prefill(const Params& p, const PrefillPlan& plan, int dk, bool bf16, bool vec,
                          hipStream_t s);

}  // namespace dr
