// Shared pieces of the two prefill passes (prefill.hip: chunk preparation; prefill_state.hip:
// the sequential state pass): the chunk length, the operand record that passes between them,
// and its fragment accesses.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace dr {

constexpr int CH = 64;    // chunk length
constexpr int NBLK = 4;   // 16-token blocks per chunk

// Operand record of one (chunk slot, head). Every fragment is 32 bytes per lane
// (bf16 hi + lo, or eight fp32 values), stored as two 1 KiB halves (bytes 0-15 of
// every lane, then bytes 16-31), so each of a wave's two 16-byte accesses per lane
// covers one contiguous KiB.
template <int DK>
struct Rec {
  static constexpr int KS = DK / 32;
  static constexpr int64_t FR = 64 * 32;                        // bytes of one fragment
  static constexpr int64_t UT = 0;                              // Utilde  [block][ks]
  static constexpr int64_t QT = UT + NBLK * KS * FR;            // Qtilde  [block][ks]
  static constexpr int64_t KB = QT + NBLK * KS * FR;            // Kbar^T  [key tile][token step]
  static constexpr int64_t TT = KB + (DK / 16) * 2 * FR;        // T       [block][token step]
  static constexpr int64_t PP = TT + NBLK * 2 * FR;             // P       [block][token step]
  static constexpr int64_t GC = PP + NBLK * 2 * FR;             // Gamma_C [DK] fp32
  static constexpr int64_t SIZE = (GC + DK * 4 + 255) / 256 * 256;
};

// A record is addressed through a buffer descriptor of its own (base = the record,
// range = its size), so that fragment addresses are a per-lane 32-bit offset plus a
// uniform byte offset: no 64-bit address arithmetic per access, and an access outside
// the record reads zero / is dropped instead of touching other memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rec_rsrc(const unsigned char* rec, int64_t size) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(rec), 0, (int)size, 0x00020000);
}
// (Stores put the whole offset in the per-lane field and keep the scalar offset at zero:
// the compiler protects the data registers of a wide buffer store from being
// overwritten too early only in that form.)
// `nt` (uniform): non-temporal stores, for records that the state pass will read back from HBM
// anyway (one window); windows small enough for the Infinity Cache keep the default policy so
// that the records stay there until they are read.
template <class Frag>
__device__ __forceinline__ void st_frag(__amdgpu_buffer_rsrc_t rs, int off, int idx, int lane, const Frag& f,
                                        bool nt) {
  static_assert(sizeof(Frag) == 32, "fragment size");
  const u32x4* h = reinterpret_cast<const u32x4*>(&f);
  if (nt) {
    __builtin_amdgcn_raw_buffer_store_b128(h[0], rs, lane * 16 + off + idx * 2048, 0, 2);
    __builtin_amdgcn_raw_buffer_store_b128(h[1], rs, lane * 16 + 1024 + off + idx * 2048, 0, 2);
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(h[0], rs, lane * 16 + off + idx * 2048, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(h[1], rs, lane * 16 + 1024 + off + idx * 2048, 0, 0);
  }
}
template <class Frag>
__device__ __forceinline__ Frag ld_frag(__amdgpu_buffer_rsrc_t rs, int off, int idx, int lane) {
  static_assert(sizeof(Frag) == 32, "fragment size");
  Frag f;
  u32x4* h = reinterpret_cast<u32x4*>(&f);
  h[0] = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16, off + idx * 2048, 0);
  h[1] = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16 + 1024, off + idx * 2048, 0);
  return f;
}

// Orders this wave's LDS writes before its later LDS reads by other lanes of the
// same wave (LDS executes a wave's instructions in order; this stops the compiler
// from reordering across the point).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// The state pass (prefill_state.hip): one workgroup per (sequence, head, block of dvb value
// columns) over the records the preparation wrote; `workgroups` as planned.
hipError_t launch_state_pass(const Params& p, int64_t workgroups, int dk, int dvb, bool bf16, bool vec,
                             hipStream_t s);

}  // namespace dr
