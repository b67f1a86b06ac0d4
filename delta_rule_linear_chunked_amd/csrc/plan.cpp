// Host-side planning of the prefill and backward launches: launch shapes, workspace sizes and the
// offsets of the workspace tables. No device code runs here; the kernels that fill the tables
// live in prefill.hip.
#include <cstdlib>

#include "prefill.hpp"

namespace dr {

static int64_t rec_size_for(int dk) {
  switch (dk) {
    case 16: case 32: return Rec<32>::SIZE;
    case 64: return Rec<64>::SIZE;
    default: return Rec<128>::SIZE;
  }
}

PrefillPlan plan_prefill(int64_t num_pairs, int64_t num_seqs, int64_t batch, int64_t seqlen,
                         int64_t heads, int dk, int dv, bool packed, int64_t window_bytes) {
  PrefillPlan pl;
  pl.chunk = CH;
  // Value columns per state workgroup: every workgroup of a head reads the head's whole
  // operand record each chunk, so wider blocks cut the load traffic per CU; narrower
  // blocks are used only when wide ones would leave CUs idle. DR_DV_BLOCK overrides
  // (16, 32 or 64) for tuning.
  pl.dv_block = (dv >= 32 && num_pairs * (dv / 32) >= 256) ? 32 : 16;
  if (const char* e = getenv("DR_DV_BLOCK")) {
    const int b = atoi(e);
    if ((b == 16 || b == 32 || b == 64) && b <= dv) pl.dv_block = b;
  }
  pl.ndvb = dv / pl.dv_block;
  const int64_t logical = num_pairs * pl.ndvb;
  // (packed: whole rows of 8 pairs, one pair per XCD, times the column blocks)
  pl.workgroups = packed ? (num_pairs + 7) / 8 * 8 * pl.ndvb : (logical + 7) / 8 * 8;
  const int64_t cps = (seqlen + CH - 1) / CH;
  pl.rec_size = rec_size_for(dk);
  pl.win_k = 0;
  pl.windows = 1;
  pl.carry = 0;
  if (packed) {
    pl.slots = cps + num_seqs;
  } else {
    // windows of equal numbers of chunks, as few as keep one window's records within the budget
    // (DR_WINDOW_BYTES overrides the budget, for tests)
    if (window_bytes <= 0) window_bytes = pl.dv_block <= 16 ? PREFILL_WINDOW_BYTES_NARROW : PREFILL_WINDOW_BYTES;
    if (const char* e = getenv("DR_WINDOW_BYTES")) {
      const long long b = atoll(e);
      if (b > 0) window_bytes = b;
    }
    const int64_t per_chunk = batch * heads * pl.rec_size;  // records of one chunk of every sequence
    int64_t kmax = per_chunk > 0 ? window_bytes / per_chunk : cps;
    if (kmax < 1) kmax = 1;
    pl.windows = cps > 0 ? (cps + kmax - 1) / kmax : 1;
    pl.win_k = cps > 0 ? (cps + pl.windows - 1) / pl.windows : 0;
    pl.slots = batch * pl.win_k;
    if (pl.windows > 1) pl.carry = num_seqs * heads * (int64_t)dk * dv * 4;
  }
  // chunk_seq, chunk_c0 [slots]; seq_first [nseq + 1]; snap_first, seq_order [nseq]; cu_ok [nseq + 1]
  const int64_t tables = packed ? ((2 * pl.slots + 4 * num_seqs + 2) * 4 + 255) / 256 * 256 : 0;
  pl.workspace = pl.slots * heads * pl.rec_size + tables + pl.carry;
  return pl;
}


int32_t* prefill_chunk_tables(void* ws, const PrefillPlan& pl, int64_t heads) {
  return reinterpret_cast<int32_t*>(static_cast<unsigned char*>(ws) + pl.slots * heads * pl.rec_size);
}

int32_t* prefill_snap_first(void* ws, const PrefillPlan& pl, int64_t heads, int64_t nseq) {
  return reinterpret_cast<int32_t*>(static_cast<unsigned char*>(ws) + pl.slots * heads * pl.rec_size) + 2 * pl.slots +
         nseq + 1;
}

int32_t* prefill_cu_table(void* ws, const PrefillPlan& pl, int64_t heads, int64_t nseq) {
  return prefill_snap_first(ws, pl, heads, nseq) + 2 * nseq;
}

float* prefill_carry(void* ws, const PrefillPlan& pl, int64_t heads) {
  // after the records (fixed length has no tables)
  return pl.carry > 0 ? reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + pl.slots * heads * pl.rec_size)
                      : nullptr;
}

int bwd_dv_block(int dv) { return dv >= 32 ? 32 : 16; }

}  // namespace dr
