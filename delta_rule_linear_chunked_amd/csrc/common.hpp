// Device-side building blocks shared by the decode and prefill kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Kernel parameter block. Pointers are device memory; sizes are element counts.
struct Params {
  const void* q;
  const void* k;
  const void* v;
  const void* alpha;    // float32, or bfloat16 when a_bf16
  const float* erase;   // beta (KDA/CKDA), e (RDA) or b (GDN-2)
  const float* write;   // == erase for KDA/CKDA, w (RDA) or w (GDN-2)
  const float* S0;      // prefill initial states (may be null); decode: unused
  const int32_t* cu;    // packed sequence offsets (may be null); past the plan pass, its clamped copy
  float* o;
  float* S;             // prefill: final states (may be null); decode: state in/out
  int64_t T;            // tokens per batch row (prefill)
  int32_t H;
  int32_t DV;           // full value width (the kernel handles a column block of it)
  int32_t num_pairs;    // sequences x heads
  int32_t ndvb;         // value-column blocks per (sequence, head)
  int32_t grid_logical; // num_pairs * ndvb
  // prefill workspace: one record of per-chunk operands per (chunk slot, head)
  unsigned char* rec;
  int64_t rec_size;
  int32_t* chunk_seq;   // packed: sequence of each chunk slot (-1: unused slot)
  int32_t* chunk_c0;    // packed: first token of the chunk within its sequence
  int32_t* seq_first;   // packed: first chunk slot of each sequence
  int32_t slots;        // chunk slots
  int32_t cps;          // fixed length: chunks per sequence
  // fixed length: one launch of the two passes covers chunks win_c0 .. win_c0 + win_nc - 1 of every
  // sequence (a window), whose records sit at slot n * win_k + (c - win_c0); the state passes from
  // one window to the next through `carry` [N, H, d_k, d_v] (read when carry_in, written instead of
  // the final state when carry_out). Packed sequences run as one window of all their chunks.
  int32_t rec_nt;       // records written with non-temporal stores (one window: read back from HBM)
  int32_t win_c0;
  int32_t win_nc;
  int32_t win_k;
  float* carry;
  int32_t carry_in;
  int32_t carry_out;
  int32_t nseq;         // sequences
  // state pools and snapshots
  const int32_t* sidx;  // slot of each sequence in the state buffers (null: slot n)
  int64_t nslots;       // slots of the state buffers when sidx is set
  float* snap;          // prefill: states after every snap_chunks chunks of each sequence (may be null)
  int32_t snap_chunks;  // chunks between snapshots
  int32_t* snap_first;  // packed: first snapshot row of each sequence
  int32_t* seq_order;   // packed: sequences by decreasing chunk count (the state pass's order)
  int32_t* cu_ok;       // packed: the plan pass's copy of the offsets, clamped to [0, tokens] and
                        // non-decreasing (the later passes read their spans from it)
  // input preparation applied while loading (all zero: inputs are used as given)
  int32_t prep_l2;      // q and k are divided by their L2 norm over d_k
  int32_t a_bf16;       // alpha is stored as bfloat16
  int32_t a_act;        // decay activation: 0 none, 1 exp(-a_scale softplus(z)), 2 tanh(z)
  int32_t g_act;        // erase / write activation: 0 none, 1 g_scale sigmoid(z)
  float a_scale;
  float g_scale;
  // transitions per token, as a power of two (0: one, 1: two). With two, a token's two
  // transitions are consecutive steps of the prefill: T, chunk positions and lengths
  // count steps (cu offsets stay in tokens and are scaled on read), q and alpha rows
  // are per token, k, v and the gates per step, and o is written after a token's last step.
  int32_t lgnh;
  // element strides of q, k and v: between consecutive tokens of a batch row (_ts) and between
  // batch rows (_bs; decode: between sequences). Within a token the heads are d apart (k and v
  // with two steps per token: a head's two steps are d apart, heads 2d apart). Dense inputs have
  // _ts = H d (x2 for k, v with two steps per token) and _bs = tokens per row x _ts.
  int64_t q_ts, q_bs, k_ts, k_bs, v_ts, v_bs;
};

// Row of step m (absolute step index) in the per-token arrays (q, alpha, o) and in the
// per-step arrays (k, v, erase, write), head h; both are m * H + h with one step per token.
__device__ __forceinline__ int64_t tok_row(const Params& p, int64_t m, int h) {
  return (m >> p.lgnh) * p.H + h;
}
__device__ __forceinline__ int64_t step_row(const Params& p, int64_t m, int h) {
  return (((m >> p.lgnh) * p.H + h) << p.lgnh) + (m & ((1 << p.lgnh) - 1));
}
// Element offsets of q (per token) and of k / v (per step) for step s of batch row b, counted
// from the start of the row, head h, with d elements per row of the input.
// (P: the prefill / decode parameters or the backward's, which carry the same stride fields)
template <class P>
__device__ __forceinline__ int64_t q_elem(const P& p, int64_t b, int64_t s, int h, int d) {
  return b * p.q_bs + (s >> p.lgnh) * p.q_ts + (int64_t)h * d;
}
template <class P>
__device__ __forceinline__ int64_t kv_elem(int64_t ts, int64_t bs, const P& p, int64_t b, int64_t s, int h,
                                           int d) {
  return b * bs + (s >> p.lgnh) * ts + ((((int64_t)h) << p.lgnh) + (s & ((1 << p.lgnh) - 1))) * d;
}
// Offset of sequence n in steps, from the packed token offsets.
__device__ __forceinline__ int64_t cu_steps(const Params& p, int n) { return (int64_t)p.cu[n] << p.lgnh; }

// Parameter block of the backward pass (gradients of a prefill).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* erase;   // beta (KDA/CKDA), e (RDA) or b (GDN-2)
  const float* write;   // == erase for KDA/CKDA, w (RDA) or w (GDN-2)
  const float* S0;      // initial states (may be null)
  const int32_t* cu;    // packed sequence offsets (may be null)
  const float* dO;      // gradient of the output
  const float* dST;     // gradient of the final states (may be null)
  float* dq;
  float* dk;
  float* dv;
  float* dalpha;
  float* derase;
  float* dwrite;        // RDA / GDN-2 only
  float* dS0;           // may be null
  const float* snap;    // forward states after every 64 tokens of each sequence
  const int32_t* snap_first;  // packed: first snapshot row of each sequence
  const int32_t* seq_order;   // packed: sequences by decreasing length (walked longest first)
  float* part;          // [ndvb][tokens * H][4][d_k] per-block row sums: dq, k-part of dk, du, dalpha
  float* parts;         // [ndvb][tokens * H] per-block v . dm
  int64_t T;
  int64_t TH;           // tokens * H
  int32_t H;
  int32_t DV;
  int32_t ndvb;
  int32_t nseq;
  int32_t variant;      // 0 KDA, 1 RDA, 2 GDN-2, 3 CKDA, 4 two KDA transitions per token
  int32_t lgnh;         // transitions per token, as a power of two (see Params); T, TH and the
                        // partial sums count steps
  int64_t q_ts, q_bs, k_ts, k_bs, v_ts, v_bs;  // element strides of q, k, v (as in Params)
  int32_t strided;      // the strides are not those of dense inputs
  const int32_t* run_flag;  // when set, the kernels run only if *run_flag is non-zero (the chunked
                            // backward hands its call over to this exact walk that way)
};

// Parameter block of the chunked backward (one transition per token).
struct CbParams {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* erase;   // beta (KDA/CKDA), e (RDA) or b (GDN-2)
  const float* write;   // == erase for KDA/CKDA, w (RDA) or w (GDN-2)
  const float* S0;      // initial states (may be null)
  const float* dO;
  const float* dST;     // may be null
  const float* snap;    // forward states after every 64 tokens of each sequence (rows as in the prefill's
                        // snapshots: fixed length b * (T / 64) + c, packed snap_first[n] + c)
  // packed sequences (cu non-null, B == 1): the prefill plan pass's clamped offsets and tables
  const int32_t* cu;
  const int32_t* chunk_seq;
  const int32_t* chunk_c0;
  const int32_t* seq_first;
  const int32_t* snap_first;
  const int32_t* seq_order;
  int32_t nseq;         // sequences (fixed length: B)
  int32_t slots;        // chunk slots (fixed length: B * nc)
  float* dq;
  float* dk;
  float* dv;
  float* dalpha;
  float* derase;
  float* dwrite;
  float* dS0;           // may be null
  unsigned char* rec;   // per (chunk slot, head): the chunk's map of the state gradient
  int64_t rec_size;
  float* dsc;           // [slots, H, d_k, d_v]: gradient reaching the state at each chunk's end
  int32_t* flag;        // set when some chunk's gates are outside the chunked form's range
  int64_t T;            // steps per batch row
  int32_t H;
  int32_t DV;
  int32_t B;
  int32_t nc;           // fixed length: 64-step chunks per sequence (chunk slot b * nc + c)
  int32_t variant;      // 0 KDA, 1 RDA, 2 GDN-2, 3 CKDA, 4 two KDA transitions per token
  int32_t lgnh;         // transitions per token, as a power of two (see Params)
  int64_t q_ts, q_bs, k_ts, k_bs, v_ts, v_bs;
};

__device__ __forceinline__ float ld_f32(const float* p) { return *p; }
__device__ __forceinline__ float ld_f32(const __bf16* p) { return (float)*p; }

// Eight consecutive elements (16-byte aligned for float pairs of f32x4, 16 bytes for bf16).
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
  x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}
__device__ __forceinline__ void load4(const float* p, float (&x)[4]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
}
__device__ __forceinline__ void store4(float* p, const f32x4& a) { *reinterpret_cast<f32x4*>(p) = a; }

// ---------------------------------------------------------------------------
// Input preparation. The activations take pre-activations z: the decay
// exp(-c softplus(z)) in (0, 1] or tanh(z) in [-1, 1], the gates c sigmoid(z). They are
// built on the hardware exp2 / log2 / reciprocal (about 1 ulp each) in forms that give the
// limits exactly: softplus(-inf) = 0 so the decay is 1, tanh(+-inf) = +-1, sigmoid(+inf) = 1,
// sigmoid(-inf) = 0.
constexpr float LOG2E = 1.4426950408889634f;
// exp(-c softplus(z)) = 2^(-c sp), sp = softplus(z) log2(e) = max(z log2 e, 0) + log2(1 + 2^(-|z| log2 e)):
// the exponent never overflows (the form 2^(-c log2(1 + 2^(z log2 e))) gave 0 for z above about 88
// whatever c was, and NaN for c = 0), and z = -inf gives exactly 1.
__device__ __forceinline__ float act_decay_softplus(float z, float c) {
  const float zl = z * LOG2E;
  const float sp = fmaxf(zl, 0.f) + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(zl)));
  return __builtin_amdgcn_exp2f(-c * sp);
}
// tanh(z): the odd Taylor polynomial through z^11 for |z| < 1/4 (truncation below 3e-10 relative),
// else sign(z) (1 - e) / (1 + e) with e = exp(-2 |z|) <= 0.61, where 1 - e has no cancellation;
// +-inf give +-1. Both forms are evaluated and one selected, so a call stays one basic block.
__device__ __forceinline__ float act_tanh(float z) {
  const float az = fabsf(z);
  const float z2 = z * z;
  float s = -1382.f / 155925.f;
  s = fmaf(s, z2, 62.f / 2835.f);
  s = fmaf(s, z2, -17.f / 315.f);
  s = fmaf(s, z2, 2.f / 15.f);
  s = fmaf(s, z2, -1.f / 3.f);
  const float poly = fmaf(s * z2, z, z);
  const float e = __builtin_amdgcn_exp2f(-2.f * LOG2E * az);
  const float big = copysignf((1.f - e) * __builtin_amdgcn_rcpf(1.f + e), z);
  return az < 0.25f ? poly : big;
}
// Both decay forms are evaluated and one is selected, so a call site stays one basic block.
__device__ __forceinline__ float prep_alpha(float z, const Params& p) {
  const float dec = act_decay_softplus(z, p.a_scale);
  const float th = act_tanh(z);
  return p.a_act == 1 ? dec : p.a_act == 2 ? th : z;
}
// One decay activation fixed at compile time (ACT 1: exp(-c softplus(z)), 2: tanh(z), 0: z),
// for kernels instantiated per activation.
template <int ACT>
__device__ __forceinline__ float prep_alpha_as(float z, float c) {
  if constexpr (ACT == 1) {
    return act_decay_softplus(z, c);
  } else if constexpr (ACT == 2) {
    return act_tanh(z);
  } else {
    return z;
  }
}
__device__ __forceinline__ float prep_gate(float z, const Params& p) {
  const float sg = p.g_scale * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-z * LOG2E));
  return p.g_act == 1 ? sg : z;
}

__device__ __forceinline__ void load8(const __bf16* p, float (&x)[8]) {
  const bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (float)a[j];
}

// Eight consecutive q / k elements as loaded (16-byte loads), converted to fp32 where used.
struct F32x8 {
  f32x4 a, b;
};
template <typename T> struct Raw8Of;
template <> struct Raw8Of<float> { using type = F32x8; };
template <> struct Raw8Of<__bf16> { using type = bf16x8; };
__device__ __forceinline__ void ld_raw8(const float* p, F32x8& r) {
  r.a = *reinterpret_cast<const f32x4*>(p);
  r.b = *reinterpret_cast<const f32x4*>(p + 4);
}
__device__ __forceinline__ void ld_raw8(const __bf16* p, bf16x8& r) { r = *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ float raw8_at(const F32x8& r, int j) { return j < 4 ? r.a[j] : r.b[j - 4]; }
__device__ __forceinline__ float raw8_at(const bf16x8& r, int j) { return (float)r[j]; }

// ---------------------------------------------------------------------------
// MFMA 16x16 tiles with a 32-deep reduction per call.
//
// Fragment convention (both precisions): lane l supplies row (A operand) or
// column (B operand) l % 16 and the eight reduction indices 8*(l/16) + j,
// j = 0..7, of the 32-deep slice. The accumulator holds column l % 16 and rows
// 4*(l/16) + i, i = 0..3. A and B use the same reduction-index assignment, so
// the sum over all four lane groups and eight items covers the slice exactly
// once.
//
// PolF32: eight v_mfma_f32_16x16x4_f32, instruction j taking item j of every
//         lane group (exact fp32 products).
// PolBF3: operands split x = hi + lo (hi = bf16(x), lo = bf16(x - hi)) and
//         hi*hi + hi*lo + lo*hi accumulated with v_mfma_f32_16x16x32_bf16;
//         the dropped lo*lo term and the rounding of lo leave a relative error
//         of about 2^-16 per product.
// ---------------------------------------------------------------------------
struct PolF32 {
  struct Frag { float v[8]; };
  static __device__ __forceinline__ Frag make(const float (&x)[8]) {
    Frag f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = x[j];
    return f;
  }
  static __device__ __forceinline__ void mma(f32x4& acc, const Frag& a, const Frag& b) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
  }
};

// Split of two fp32 values into bf16 hi (round to nearest even) and the bf16 of the remainder
// x - hi, as two packed pairs: one packed conversion for the two hi halves, their fp32 values by a
// shift and a mask, two subtractions and one packed conversion for lo (converting value by value
// leads the compiler to convert each hi twice).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
  const float ha = __builtin_bit_cast(float, hi << 16);
  const float hb = __builtin_bit_cast(float, hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a - ha, b - hb}, bf16x2));
}

struct PolBF3 {
  struct Frag { bf16x8 hi, lo; };
  static __device__ __forceinline__ Frag make(const float (&x)[8]) {
    uint32_t h[4], o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) split2(x[2 * j], x[2 * j + 1], h[j], o[j]);
    Frag f;
    f.hi = __builtin_bit_cast(bf16x8, h);
    f.lo = __builtin_bit_cast(bf16x8, o);
    return f;
  }
  static __device__ __forceinline__ void mma(f32x4& acc, const Frag& a, const Frag& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
  }
};

template <typename InT> struct PolicyFor;
template <> struct PolicyFor<float> { using type = PolF32; };
template <> struct PolicyFor<__bf16> { using type = PolBF3; };

// ---------------------------------------------------------------------------
// Scans across the 16 lanes of a DPP row (rows are lanes 0-15, 16-31, 32-47, 48-63).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_or(float old, float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, x), CTRL,
                                                               0xf, 0xf, false));
}
constexpr int ROW_SHL1 = 0x101, ROW_SHL2 = 0x102, ROW_SHL4 = 0x104, ROW_SHL8 = 0x108;
constexpr int ROW_SHR1 = 0x111, ROW_SHR2 = 0x112, ROW_SHR4 = 0x114, ROW_SHR8 = 0x118;
constexpr int ROW_BCAST15 = 0x15F;  // gfx950 row_newbcast:15: every lane reads lane 15 of its row

// Inclusive prefix product over lanes 0..r of the row (lane r receives x_0 * ... * x_r).
__device__ __forceinline__ float row_prefix_prod(float x) {
  x *= dpp_or<ROW_SHR1>(1.f, x);
  x *= dpp_or<ROW_SHR2>(1.f, x);
  x *= dpp_or<ROW_SHR4>(1.f, x);
  x *= dpp_or<ROW_SHR8>(1.f, x);
  return x;
}
// Eight independent inclusive prefix products across the row, one VOP2 DPP multiply
// per element and step: v_mul_f32_dpp x, x, x row_shr:d writes x_{r-d} * x_r, and the
// lanes r < d, whose source lies outside the row, are not written (bound_ctrl off), so
// they keep x_r. The eight chains are interleaved, so each DPP read comes 8 VALU
// instructions after the write it depends on; the s_nop pairs cover the instructions
// just before and after the block. Needs every lane of the wave active.
__device__ __forceinline__ void row_prefix_prod8(float (&x)[8]) {
#define DR_STEP(D)                                                           \
  "v_mul_f32_dpp %0, %0, %0 row_shr:" #D " row_mask:0xf bank_mask:0xf\n"    \
  "v_mul_f32_dpp %1, %1, %1 row_shr:" #D " row_mask:0xf bank_mask:0xf\n"    \
  "v_mul_f32_dpp %2, %2, %2 row_shr:" #D " row_mask:0xf bank_mask:0xf\n"    \
  "v_mul_f32_dpp %3, %3, %3 row_shr:" #D " row_mask:0xf bank_mask:0xf\n"    \
  "v_mul_f32_dpp %4, %4, %4 row_shr:" #D " row_mask:0xf bank_mask:0xf\n"    \
  "v_mul_f32_dpp %5, %5, %5 row_shr:" #D " row_mask:0xf bank_mask:0xf\n"    \
  "v_mul_f32_dpp %6, %6, %6 row_shr:" #D " row_mask:0xf bank_mask:0xf\n"    \
  "v_mul_f32_dpp %7, %7, %7 row_shr:" #D " row_mask:0xf bank_mask:0xf\n"
  asm("s_nop 1\n" DR_STEP(1) DR_STEP(2) DR_STEP(4) DR_STEP(8) "s_nop 1\n"
      : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]));
#undef DR_STEP
}

// Exclusive suffix product (lane r receives x_{r+1} * ... * x_15; lane 15 receives 1).
__device__ __forceinline__ float row_suffix_prod_excl(float x) {
  x *= dpp_or<ROW_SHL1>(1.f, x);
  x *= dpp_or<ROW_SHL2>(1.f, x);
  x *= dpp_or<ROW_SHL4>(1.f, x);
  x *= dpp_or<ROW_SHL8>(1.f, x);
  return dpp_or<ROW_SHL1>(1.f, x);
}

// Map a dispatched workgroup id to a logical work item so that consecutive
// logical items (the value-column blocks of one sequence-head pair, which read
// the same keys, queries and gates) land on the same XCD and share its L2.
// Workgroups are dispatched round-robin over the 8 XCDs.
__device__ __forceinline__ int xcd_remap(int b, int grid) {
  constexpr int NXCD = 8;
  const int per = grid / NXCD;  // grid is padded to a multiple of 8
  return (b % NXCD) * per + (b / NXCD);
}

}  // namespace dr
