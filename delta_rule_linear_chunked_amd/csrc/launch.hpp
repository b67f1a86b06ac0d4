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
  int64_t slots;       // chunk slots of one window (an upper bound for packed sequences)
  int64_t rec_size;    // bytes of one (chunk slot, head) operand record
  int64_t win_k;       // fixed length: chunks of every sequence per window (packed: 0, one window)
  int64_t windows;     // launches of the two passes
  int64_t carry;       // bytes of the state carried between windows (0 for one window)
  int64_t workspace;   // bytes of workspace (records of one window + packed-sequence tables + carry)
};
// Operand records of one window are kept to about this many bytes, which bounds the workspace of
// any fixed-length prefill. The default depends on the state pass's value-column block. With
// 32-column blocks (e.g. the KDA prefill, 4 x 4096 tokens, 16 heads, d = 128) one window is
// fastest: smaller windows keep the records in the 256 MB Infinity Cache, but the pass is then
// bound by its per-chunk chain and the extra launches cost 2-4 %. With 16-column blocks (few
// (sequence, head) pairs, e.g. 2 x 16384 tokens x 16 heads) every workgroup reads a whole record
// for half the matrix work, the pass is bound by those reads, and windows of about 130-170 MB of
// records measured 6.5 % faster than one or two large windows (budgets of 96 to 384 MiB tried).
constexpr int64_t PREFILL_WINDOW_BYTES = (int64_t)1 << 30;
constexpr int64_t PREFILL_WINDOW_BYTES_NARROW = (int64_t)144 << 20;  // 16-column value blocks
PrefillPlan plan_prefill(int64_t num_pairs, int64_t num_seqs, int64_t batch, int64_t seqlen,
                         int64_t heads, int dk, int dv, bool packed,
                         int64_t window_bytes = 0);  // 0: the default for the plan's value block

// Prefill: chunk preparation over every (chunk, head), then the state pass over every
// (sequence, head, value block). `ws` is a workspace of plan.workspace bytes.
hipError_t launch_prefill(Params p, const PrefillPlan& plan, void* ws, int dk, bool bf16, bool vec,
                          hipStream_t s);

// Packed sequences: where the prefill's workspace keeps the first snapshot row of each sequence
// (filled by the prefill when snapshots are taken), followed by the sequences' longest-first order.
int32_t* prefill_snap_first(void* ws, const PrefillPlan& plan, int64_t heads, int64_t nseq);
// Packed sequences: the plan pass's chunk tables: the sequence of each chunk slot (-1: unused) [slots],
// the slot's first token within its sequence [slots], each sequence's first slot [nseq + 1].
int32_t* prefill_chunk_tables(void* ws, const PrefillPlan& plan, int64_t heads);
// Packed sequences: the plan pass's clamped, non-decreasing copy of the offsets [nseq + 1], from which
// every later pass (the backward's included) takes its sequence spans.
int32_t* prefill_cu_table(void* ws, const PrefillPlan& plan, int64_t heads, int64_t nseq);
// Fixed length over several windows: the state carried from one window to the next (NULL otherwise).
float* prefill_carry(void* ws, const PrefillPlan& plan, int64_t heads);

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

// Chunked backward (backward_chunked.hip): fixed-length or packed sequences, one transition per token,
// d_k in {64, 128}, d_v a multiple of 32 up to 128. Bytes of one chunk record, then the launches:
// the flag is cleared, every (batch row, chunk, head) builds its record, the state-gradient pass
// runs over the chunks in reverse and the gradient kernel writes every output except dS0 (which
// the state-gradient pass writes). A chunk whose gates the chunked form does not take (more than 12
// gates of magnitude below 2^-4, a zero or non-finite gate, a running product outside
// [2^-110, 2^100]) sets *flag; the gradient kernel then writes nothing and the caller runs the
// exact walk.
struct CbParams;
int64_t cbwd_record_bytes(int dk, int dv);
hipError_t launch_chunked_backward(const CbParams& p, int dk, bool bf16, bool vec, hipStream_t s);

}  // namespace dr
