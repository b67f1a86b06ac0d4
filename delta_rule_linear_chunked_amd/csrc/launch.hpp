// Host-side entry points of the kernels (called by the C ABI layer after validation).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dr {

struct Params;
struct BwdParams;

// Decode: one workgroup per (sequence, head); p.S is the state updated in place.
hipError_t launch_decode(const Params& p, int64_t nheads, int dk, int dv, bool bf16, bool vec,
                         hipStream_t s);
// Decode step with two KDA transitions per token (PRODUCT2).
hipError_t launch_decode2(const Params& p, int64_t nheads, int dk, int dv, bool bf16, hipStream_t s);

// Prefill launch shape for a problem.
struct PrefillPlan {
  int chunk;
  int dv_block;
  int ndvb;
  int64_t workgroups;  // state pass: padded to a multiple of 8 (XCD count)
  int64_t slots;       // chunk slots (an upper bound for packed sequences)
  int64_t rec_size;    // bytes of one (chunk slot, head) operand record
  int64_t workspace;   // bytes of workspace (records + packed-sequence tables)
};
PrefillPlan plan_prefill(int64_t num_pairs, int64_t num_seqs, int64_t batch, int64_t seqlen,
                         int64_t heads, int dk, int dv, bool packed);

// Prefill: chunk preparation over every (chunk, head), then the state pass over every
// (sequence, head, value block). `ws` is a workspace of plan.workspace bytes.
hipError_t launch_prefill(Params p, const PrefillPlan& plan, void* ws, int dk, bool bf16, bool vec,
                          hipStream_t s);

// Packed sequences: where the prefill's workspace keeps the first snapshot row of each sequence
// (filled by the prefill when snapshots are taken), followed by the sequences' longest-first order.
int32_t* prefill_snap_first(void* ws, const PrefillPlan& plan, int64_t heads, int64_t nseq);
// Packed sequences: the plan pass's clamped, non-decreasing copy of the offsets [nseq + 1], from which
// every later pass (the backward's included) takes its sequence spans.
int32_t* prefill_cu_table(void* ws, const PrefillPlan& plan, int64_t heads, int64_t nseq);

// Only the packed-sequence plan pass of a prefill (chunk slots, first snapshot rows, sequence
// order) into `ws`; nothing for fixed-length sequences.
hipError_t launch_plan_only(Params p, const PrefillPlan& plan, void* ws, hipStream_t s);

// Device address of this device's static scratch array (DR_NOALLOC_SCRATCH_BYTES bytes), looked up
// once per device.
hipError_t scratch_buffer(void** ptr);

// Backward: bwd_kernel over every (sequence, head, value block), then the reduction over the
// blocks. p.snap must hold the forward states after every 64 tokens (the prefill's snapshots);
// p.part / p.parts the per-block partial sums (ndvb = d_v / bwd_dv_block(d_v) blocks).
int bwd_dv_block(int dv);
hipError_t launch_backward(BwdParams p, int64_t pairs, int dk, int dv, bool bf16, bool vec, hipStream_t s);

}  // namespace dr
