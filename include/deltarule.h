/*
 * deltarule.h — C ABI of the MI355X (gfx950) gated delta-rule library.
 *
 * The library computes the recurrence
 *
 *     S_t = (I - k_t u_t^T) Diag(alpha_t) S_{t-1} + k_t m_t^T,      o_t = S_t^T q_t
 *
 * whose three instances are the KDA, RDA and GDN-2 update rules listed in the
 * Hugging Face discussion "KRAFTON/Raon-1-mini-preview" #1 (the reply giving
 * "the three state updates"), plus Complex KDA, which keeps KDA's formula with
 * alpha in [-1, 1] and beta in [0, 2] (abstract of "Complex KDA: Understanding
 * and Enhancing the Expressivity of Kimi Delta Attention", arXiv 2609.24797):
 *
 *     variant      erase gate (u_t)            write gate (m_t)
 *     DR_KDA       beta_t  [.., H]   u = beta k   write == NULL, m = beta v
 *     DR_CKDA      beta_t  [.., H]   u = beta k   write == NULL, m = beta v
 *     DR_RDA       e_t     [.., H]   u = e k      w_t [.., H],    m = w v
 *     DR_GDN2      b_t     [.., H, d_k] u = b.k   w_t [.., H, d_v], m = w.v
 *
 * DR_PRODUCT2 applies two such transitions per token, each with KDA's rule and
 * its own key, value and beta, the decay acting once before the first and the
 * readout after the second:
 *
 *     S' = (I - b_1 k_1 k_1^T) Diag(alpha_t) S_{t-1} + b_1 k_1 v_1^T
 *     S_t = (I - b_2 k_2 k_2^T) S'                    + b_2 k_2 v_2^T,   o_t = S_t^T q_t
 *
 * (the composition of two delta-rule transitions per update that the Complex KDA
 * abstract cites as prior work, DeltaProduct with two factors). Its k is
 * [.., H, 2, d_k], v [.., H, 2, d_v] and beta (erase) [.., H, 2]; q and alpha keep
 * one row per token and write is NULL; its gradients (dr_chunk_bwd) take the same
 * layouts, and its snapshot_every must be a multiple of 32.
 *
 * The state S has d_k rows (key channels) and d_v columns; Diag(alpha_t) scales
 * its rows. The readout uses the updated state and no 1/sqrt(d_k) factor.
 * Gate values are not range-checked: CKDA differs from KDA only in the values
 * the caller passes.
 *
 * Memory and layout. Every pointer argument is DEVICE memory on the current HIP
 * device, row-major and densely packed in the shapes given below, and 16-byte
 * aligned. The caller owns every argument buffer; the library keeps no pointer
 * to them after a call returns. dr_decode_step uses no other device memory.
 * dr_chunk_fwd needs a workspace between its two kernels (about 128.5 KiB per
 * 64-step chunk and head at d_k = 128 for the chunks of one window, see
 * dr_chunk_fwd_plan_ex; a step is a token, or half a token for DR_PRODUCT2); it
 * takes it stream-ordered on `stream`
 * from a per-device memory pool owned by the library, which keeps what it has
 * reserved for later calls (a larger problem grows it once). Apart from that
 * pool the library holds only a thread-local error message. Work is enqueued
 * on `stream` and runs asynchronously; outputs are valid once the stream
 * reaches that point.
 *
 * Errors. Argument errors are detected on the host before anything is launched
 * and return a negative status (nothing is written). A failed kernel launch
 * returns DR_ERR_HIP. dr_last_error() describes the most recent failure on the
 * calling thread.
 *
 * cu_seqlens. A valid cu_seqlens starts at 0, never decreases and ends at most
 * at T (rows past cu_seqlens[N] are neither read nor written). Its contents
 * live in device memory and are not read on the host by default: the kernels
 * take every sequence span from a copy clamped to [0, T] and made
 * non-decreasing, so an invalid cu_seqlens gives unspecified results (and, with
 * snapshots, snapshot rows for the clamped lengths) but no access outside the
 * token rows, the states or the workspace. With DR_DEBUG_VALIDATE set in the
 * environment (to anything but "0"), dr_chunk_fwd(_ex) and dr_chunk_bwd(_ex)
 * also copy cu_seqlens to the host (synchronising `stream`, so not inside a
 * graph capture) and return DR_ERR_SHAPE for an invalid one, with nothing
 * launched.
 */
#ifndef DELTARULE_H
#define DELTARULE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dr_variant { DR_KDA = 0, DR_RDA = 1, DR_GDN2 = 2, DR_CKDA = 3, DR_PRODUCT2 = 4 } dr_variant;

/* Element type of q, k and v. Gates, states and outputs are always float32. */
typedef enum dr_dtype { DR_F32 = 0, DR_BF16 = 1 } dr_dtype;

typedef enum dr_status {
  DR_OK = 0,
  DR_ERR_NULL = -1,        /* a required pointer is NULL */
  DR_ERR_SHAPE = -2,       /* negative or inconsistent sizes */
  DR_ERR_DTYPE = -3,       /* in_dtype is not DR_F32 / DR_BF16 */
  DR_ERR_LAYOUT = -4,      /* a pointer not 16-byte aligned, or strides the call does not take */
  DR_ERR_ALIGN = -4,       /* the same code under its earlier name */
  DR_ERR_UNSUPPORTED = -5, /* head size outside {16, 32, 64, 128}, or a size beyond the limits */
  DR_ERR_VARIANT = -6,     /* unknown variant, or gate pointers that do not fit it */
  DR_ERR_HIP = -7          /* a HIP runtime call or kernel launch failed */
} dr_status;

/* Sizes of one call.
 *   batch      B: rows of the [B, T, ...] token layout (1 when cu_seqlens is given)
 *   seqlen     T: tokens per row (the total packed length when cu_seqlens is given)
 *   num_heads  H
 *   head_dim_k d_k, head_dim_v d_v: each one of 16, 32, 64, 128
 *   num_seqs   N: number of sequences (= B without cu_seqlens, len(cu_seqlens) - 1 with it)
 *   in_dtype   element type of q, k, v (dr_dtype)
 *   version    0: q, k, v are dense as the entry points describe them; DR_DIMS_V2: the struct is
 *              the first member of a dr_dims_v2, whose strides place q, k and v
 */
typedef struct dr_dims {
  int64_t batch;
  int64_t seqlen;
  int64_t num_heads;
  int64_t head_dim_k;
  int64_t head_dim_v;
  int64_t num_seqs;
  int32_t in_dtype;
  int32_t version; /* 0 or DR_DIMS_V2 */
} dr_dims;

/* Strided q, k, v (a pointer to `base` is passed where a dr_dims is expected, with
 * base.version = DR_DIMS_V2), e.g. views of one fused [B, T, 3, H, d] projection. Each input
 * keeps its last dimension contiguous and its heads d apart within a token (d_k for q and k, d_v
 * for v; for DR_PRODUCT2, k and v keep a token's two steps d apart and heads 2 d apart), and gives
 * two element strides: between consecutive tokens of a batch row, and between batch rows (for
 * the decode step, between sequences; its token stride is unused). Dense inputs have token
 * stride H d (2 H d for DR_PRODUCT2's k and v) and batch stride T times that. Strides must be
 * non-negative and, times the element size, multiples of 16 bytes; every element the strides
 * address must lie inside the caller's buffer (not checked). alpha, the gates, the states and
 * the output stay dense (so do the gradients of the backward). Every entry point that takes q, k
 * and v takes them strided: dr_chunk_fwd, dr_chunk_fwd_ex, dr_chunk_fwd_noalloc, dr_decode_step,
 * dr_decode_step_ex, dr_chunk_bwd and dr_chunk_bwd_ex.
 */
#define DR_DIMS_V2 2
typedef struct dr_dims_v2 {
  dr_dims base;
  int64_t q_token_stride, q_batch_stride;
  int64_t k_token_stride, k_batch_stride;
  int64_t v_token_stride, v_batch_stride;
} dr_dims_v2;

/*
 * Chunkwise-parallel prefill (the "scan/chunked" form of the recurrence that the
 * course page "GDN, KDA và Mamba-2 · cập nhật state trong hybrid", section 3,
 * says must match the step recurrence in the same dtype).
 *
 *   q, k       [B, T, H, d_k]  in_dtype
 *   v          [B, T, H, d_v]  in_dtype
 *   alpha      [B, T, H, d_k]  float32, channel-wise decay
 *   erase      [B, T, H] float32 (KDA/CKDA beta, RDA e) or [B, T, H, d_k] (GDN-2 b)
 *   write      NULL (KDA/CKDA), [B, T, H] (RDA w) or [B, T, H, d_v] (GDN-2 w)
 *              (DR_PRODUCT2: k [B, T, H, 2, d_k], v [B, T, H, 2, d_v], erase [B, T, H, 2],
 *              write NULL)
 *   S0         [N, H, d_k, d_v] float32 initial states, or NULL for zero states
 *   cu_seqlens [N + 1] int32 or NULL. When given, B must be 1 and sequence n is
 *              tokens cu_seqlens[n] .. cu_seqlens[n+1]-1 of the packed row; each
 *              sequence starts from its own S0[n] and no state crosses a boundary
 *              (the same course page, section 3: document reset). Without it,
 *              sequence n is batch row n.
 *   o          [B, T, H, d_v] float32 output (written), or NULL when only the final states
 *              (or snapshots) are wanted
 *   S_T        [N, H, d_k, d_v] float32 final states, or NULL to skip; may alias S0
 *              for an in-place update.
 * o must not alias any input. Results do not depend on how the library chunks
 * the sequence, up to rounding. Returns DR_ERR_HIP, with nothing launched, when
 * the workspace cannot be reserved.
 */
int dr_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                 const float* erase, const float* write, int variant,
                 const float* S0, const int32_t* cu_seqlens,
                 float* o, float* S_T, const dr_dims* dims, hipStream_t stream);

/*
 * One recurrent decode step for N sequences x H heads, one token each: the
 * fixed-size state is read once, updated in place and the token's output
 * written (the course page above, section 1: the state's size does not grow
 * with T at decode).
 *
 *   q, k       [N, H, d_k]  in_dtype;   v [N, H, d_v] in_dtype
 *              (DR_PRODUCT2: k [N, H, 2, d_k], v [N, H, 2, d_v], erase [N, H, 2])
 *   alpha      [N, H, d_k]  float32
 *   erase      [N, H] or [N, H, d_k] (GDN-2);  write NULL, [N, H] or [N, H, d_v]
 *   S          [N, H, d_k, d_v] float32, read and overwritten with S_t
 *   o          [N, H, d_v] float32 (written)
 * dims: batch = num_seqs = N, seqlen = 1.
 */
int dr_decode_step(const void* q, const void* k, const void* v, const float* alpha,
                   const float* erase, const float* write, int variant,
                   float* S, float* o, const dr_dims* dims, hipStream_t stream);

/* Activations of the fused input preparation (dr_opts). */
typedef enum {
  DR_ACT_NONE = 0,              /* the input is used as given */
  DR_ACT_EXP_NEG_SOFTPLUS = 1,  /* decay: alpha = exp(-alpha_scale * softplus(z)), in (0, 1] */
  DR_ACT_TANH = 2,              /* decay: alpha = tanh(z), in [-1, 1] (Complex KDA) */
  DR_ACT_SIGMOID = 3            /* erase / write: gate_scale * sigmoid(z) */
} dr_act;

/*
 * Options of dr_chunk_fwd_ex / dr_decode_step_ex. A zero-filled block (or a NULL
 * pointer) means the plain call.
 *
 * Stored states, for prefix sharing and continuous batching. Section 3 of the
 * course page above keeps three things apart: padding, a document reset (each
 * sequence starts from its own state) and a state snapshot kept for prefix
 * sharing, and forbids two requests sharing a state with different content.
 *
 *   state_idx      [N] int32 (device) or NULL. When given, the state buffers
 *                  (S0 and S_T of a prefill, S of a decode step) are pools of
 *                  num_slots rows [num_slots, H, d_k, d_v] and sequence n uses
 *                  row state_idx[n]. A slot outside [0, num_slots) means the
 *                  sequence has no stored state: a prefill starts it from zero
 *                  and stores no final state; a decode step writes zeros to its
 *                  output and touches no state. Rows nobody names are left as
 *                  they are. Two sequences naming the same slot race (undefined).
 *   num_slots      rows of the pools (used only with state_idx).
 *   snapshots      prefill only: float32 [num_snapshots, H, d_k, d_v] or NULL.
 *                  Sequence n stores floor(len_n / snapshot_every) states, the
 *                  state after (j + 1) * snapshot_every of its tokens in row
 *                  first_n + j, where first_n = sum over m < n of
 *                  floor(len_m / snapshot_every). Resuming a prefill from row
 *                  first_n + j over the rest of the sequence gives the same
 *                  outputs and final state, up to rounding.
 *   snapshot_every a positive multiple of 64, or of 32 for DR_PRODUCT2 (snapshots
 *                  sit on boundaries of 64-step chunks); otherwise DR_ERR_SHAPE.
 * Snapshots cost one extra state write per snapshot (d_k * d_v * 4 bytes per head).
 *
 * Fused input preparation: the step in front of the recurrence (the course page's
 * section 2, "project and prepare q/k/v") done while the kernels load their
 * inputs, so callers pass raw projections and gate pre-activations and the
 * prepared tensors never exist in memory.
 *   l2norm_qk      1: q and k are divided by their L2 norm over d_k (per token
 *                  and head; a zero vector stays zero). 0: used as given.
 *   alpha_dtype    DR_F32 or DR_BF16: element type of alpha.
 *   alpha_act      DR_ACT_NONE, DR_ACT_EXP_NEG_SOFTPLUS or DR_ACT_TANH, applied
 *                  to alpha with alpha_scale.
 *   gate_act       DR_ACT_NONE or DR_ACT_SIGMOID, applied to erase and write
 *                  (beta for KDA / CKDA) with gate_scale (2 gives Complex KDA's
 *                  beta in [0, 2]).
 * Pre-activations of +-inf give the limits exactly (alpha = 1 or 0, tanh = +-1,
 * sigmoid = 1 or 0), so exact gates stay expressible. Other values, or a scale
 * that is not finite, are DR_ERR_UNSUPPORTED / DR_ERR_DTYPE.
 */
typedef struct dr_opts {
  /* stored states */
  const int32_t* state_idx;
  int64_t num_slots;
  float* snapshots;
  int64_t snapshot_every;
  /* input preparation */
  int32_t l2norm_qk;
  int32_t alpha_dtype;
  int32_t alpha_act;
  float alpha_scale;
  int32_t gate_act;
  float gate_scale;
} dr_opts;

/* dr_chunk_fwd with options (opts may be NULL: same as dr_chunk_fwd). alpha is
 * float32, or bfloat16 with alpha_dtype = DR_BF16. */
int dr_chunk_fwd_ex(const void* q, const void* k, const void* v, const void* alpha,
                    const float* erase, const float* write, int variant,
                    const float* S0, const int32_t* cu_seqlens,
                    float* o, float* S_T, const dr_dims* dims, const dr_opts* opts,
                    hipStream_t stream);

/* dr_decode_step with options (opts may be NULL: same as dr_decode_step;
 * snapshots must be NULL). With state_idx, S is the pool. */
int dr_decode_step_ex(const void* q, const void* k, const void* v, const void* alpha,
                      const float* erase, const float* write, int variant,
                      float* S, float* o, const dr_dims* dims, const dr_opts* opts,
                      hipStream_t stream);

/*
 * dr_chunk_fwd_ex for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation). Same arguments, semantics and results
 * (the same kernels run); the prefill's workspace is instead a static device array of
 * DR_NOALLOC_SCRATCH_BYTES bytes that the library holds on each GPU it runs on until the process
 * ends. The call allocates nothing: no hipMalloc, hipFree or pool allocation. A problem whose
 * workspace does not fit returns DR_ERR_UNSUPPORTED with nothing launched: fixed-length problems
 * run in windows small enough for the array (one chunk of every sequence at the least, so up to
 * about 2000 sequence-heads at d_k = 128), while packed sequences run as one window (about
 * 128.5 KiB per 64-step chunk and head at d_k = 128, so about 2000 chunk-heads, e.g. 8192 tokens
 * x 16 heads).
 * Every call on one GPU uses that GPU's one array, so calls that overlap on a GPU (on different
 * streams, or from different threads) race and give undefined results: serialise them.
 */
#define DR_NOALLOC_SCRATCH_BYTES (256ull << 20)
int dr_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* alpha,
                         const float* erase, const float* write, int variant,
                         const float* S0, const int32_t* cu_seqlens,
                         float* o, float* S_T, const dr_dims* dims, const dr_opts* opts,
                         hipStream_t stream);

/*
 * Gradients of dr_chunk_fwd, for training (the course page above, section 3: training needs
 * activations, checkpoints and the scan's intermediates). For a loss L with
 * dO = dL/do [B, T, H, d_v] and dS_T = dL/dS_T [N, H, d_k, d_v] (NULL: zero), writes, all
 * float32 in the shapes of the corresponding inputs:
 *   dq, dk        [B, T, H, d_k]
 *   dv            [B, T, H, d_v]
 *   dalpha        [B, T, H, d_k]
 *   derase        shape of erase: KDA / CKDA d(beta) (both of beta's uses), RDA d(e), GDN-2 d(b)
 *                 (DR_PRODUCT2: dk [B, T, H, 2, d_k], dv [B, T, H, 2, d_v], derase [B, T, H, 2])
 *   dwrite        RDA d(w) [B, T, H], GDN-2 d(w) [B, T, H, d_v]; must be NULL for KDA / CKDA
 *   dS0           [N, H, d_k, d_v], or NULL when not wanted
 * The inputs are those of the forward call (plain inputs: the fused preparation and the
 * stored-state options are forward-only; q, k, v may be strided through a dr_dims_v2, the
 * gradients are always dense). The call reruns the forward to keep the state after
 * every 64 steps (32 tokens for DR_PRODUCT2). Calls with d_k 64 or 128 and d_v a multiple of 32
 * up to 128 (fixed-length or packed, one or two transitions per token) then take the chunked form: per 64-token chunk an affine map of the
 * state gradient, a reverse pass over the chunks, and the chunk's gradients from its tile
 * products, all on MFMA. That form divides by the decays' running products and by the decays
 * themselves: up to 12 gates per chunk of magnitude below 2^-4 take their gradient from an exact
 * inner product instead, and a chunk with more of them, a zero or non-finite gate, or a running
 * product outside [2^-110, 2^100] hands the whole call, on the device and without a host
 * synchronisation, to the exact per-token walk, which every other call takes directly: it
 * walks each sequence backwards, recomputing states between the checkpoints. DR_BWD_WALK set (and
 * not "0") in the environment sends every call to the walk. The workspace (about 4 * d_k * 4
 * bytes per token-head and value block of 32 columns, plus the checkpoints; the chunked form's
 * records and chunk-end gradients, 4 * d_k * (d_k + 2 d_v) bytes per chunk-head, share it) comes from the
 * library's pool like the prefill's. Deterministic on both paths: no atomics on the results.
 */
int dr_chunk_bwd(const void* q, const void* k, const void* v, const float* alpha,
                 const float* erase, const float* write, int variant,
                 const float* S0, const int32_t* cu_seqlens,
                 const float* dO, const float* dS_T,
                 float* dq, float* dk, float* dv, float* dalpha, float* derase, float* dwrite,
                 float* dS0, const dr_dims* dims, hipStream_t stream);

/*
 * dr_chunk_bwd with the forward's checkpoints supplied by the caller, for training steps that
 * ran the forward anyway (the course page's section 3: training keeps checkpoints of the
 * forward). `checkpoints` is the `snapshots` buffer of a dr_chunk_fwd_ex call on the same
 * inputs (same S0 and cu_seqlens, no fused preparation) with snapshot_every = 64, or 32 for
 * DR_PRODUCT2: float32 [sum_n floor(len_n / snapshot_every), H, d_k, d_v]. With it the call
 * skips its own forward pass and only reads the checkpoints; NULL is dr_chunk_bwd. A buffer that
 * does not hold those states gives undefined gradients (the library cannot check its contents).
 */
int dr_chunk_bwd_ex(const void* q, const void* k, const void* v, const float* alpha,
                    const float* erase, const float* write, int variant,
                    const float* S0, const int32_t* cu_seqlens,
                    const float* dO, const float* dS_T,
                    float* dq, float* dk, float* dv, float* dalpha, float* derase, float* dwrite,
                    float* dS0, const float* checkpoints, const dr_dims* dims, hipStream_t stream);

/* Static description of a status code. Never NULL. */
const char* dr_status_string(int status);

/* Message for the last failing call on this thread ("" if none). Valid until the
 * next library call on the same thread. */
const char* dr_last_error(void);

/* Library ABI version: major * 10000 + minor * 100 + patch. */
int dr_version(void);

/*
 * Launch shape the prefill would use for `dims` (for tests and profiling):
 * chunk length, value columns per workgroup of the sequential state pass, and
 * that pass's number of workgroups (taking the sequences as packed when batch
 * is 1 and num_seqs is not). The value-column block is 32 when that gives at least 256
 * workgroups, else 16; DR_DV_BLOCK in the environment (16, 32 or 64, at most d_v) overrides it,
 * for tuning and tests (results do not depend on it beyond rounding order).
 * Returns DR_OK or an argument error.
 */
int dr_chunk_fwd_plan(const dr_dims* dims, int variant, int32_t* chunk, int32_t* dv_block,
                      int64_t* workgroups);

/*
 * The prefill's launch plan for `dims` in full (for tests, profiling and callers that size their
 * memory): the fixed-length prefill runs its two passes over windows of chunk positions (a few
 * chunks of every sequence at a time, the state carried between windows), so that one window's
 * operand records (about 128.5 KiB per chunk and head at d_k = 128) stay within 1 GiB, or
 * within 144 MiB when the state pass uses 16-column value blocks (dv_block = 16, where windows
 * that fit the Infinity Cache are faster): the workspace of a fixed-length prefill is at most
 * about 1 GiB plus the carried state (num_seqs * heads * d_k * d_v * 4 bytes) whatever its
 * length. Packed sequences run as one window. DR_WINDOW_BYTES in the environment sets another
 * budget (in bytes; windows change no arithmetic, the results stay identical bit for bit). With
 * noalloc != 0 the plan is the one dr_chunk_fwd_noalloc uses (windows small enough for its static
 * scratch). Sequences are taken as packed when batch is 1 and num_seqs is not.
 */
typedef struct dr_plan {
  int32_t chunk;          /* steps per chunk */
  int32_t dv_block;       /* value columns per workgroup of the state pass */
  int64_t workgroups;     /* workgroups of the state pass */
  int64_t window_chunks;  /* chunks of every sequence per window (0 for packed sequences) */
  int64_t windows;        /* launches of the two passes */
  int64_t workspace;      /* bytes of workspace of the call */
} dr_plan;
int dr_chunk_fwd_plan_ex(const dr_dims* dims, int variant, int noalloc, dr_plan* plan);

#ifdef __cplusplus
}
#endif

#endif /* DELTARULE_H */
