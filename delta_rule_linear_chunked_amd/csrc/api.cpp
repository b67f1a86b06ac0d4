// C ABI of the gated delta-rule library: argument validation and kernel dispatch.
// Every check runs on the host before any launch; no device memory is read here.
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/deltarule.h"
#include "common.hpp"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

bool head_dim_ok(int64_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared checks of the variant's gate pointers. scalar_lead / vector shapes are implied by the
// variant; the library cannot see extents of device buffers, so it checks presence only.
int check_variant(int variant, const float* erase, const float* write, bool has_tokens, bool* vec) {
  switch (variant) {
    case DR_KDA:
    case DR_CKDA:
    case DR_PRODUCT2:
      if (write != nullptr)
        return fail(DR_ERR_VARIANT, "variant %s takes beta as `erase` and no `write` gate",
                    variant == DR_KDA ? "KDA" : variant == DR_CKDA ? "CKDA" : "PRODUCT2");
      *vec = false;
      break;
    case DR_RDA:
      if (write == nullptr && has_tokens)
        return fail(DR_ERR_VARIANT, "variant RDA needs a per-head `write` gate");
      *vec = false;
      break;
    case DR_GDN2:
      if (write == nullptr && has_tokens)
        return fail(DR_ERR_VARIANT, "variant GDN-2 needs a channel-wise `write` gate");
      *vec = true;
      break;
    default:
      return fail(DR_ERR_VARIANT, "unknown variant %d", variant);
  }
  (void)erase;  // presence is checked with the other token pointers when there are tokens
  return DR_OK;
}

// Element strides of q, k, v: {q token, q batch, k token, k batch, v token, v batch}, the
// caller's (dr_dims_v2) or those of dense inputs with `rows` tokens per batch row (lg: log2 of
// the steps per token).
static void input_strides(const dr_dims* d, int lg, int64_t rows, int64_t st[6]) {
  if (d->version == DR_DIMS_V2) {
    const dr_dims_v2* v = reinterpret_cast<const dr_dims_v2*>(d);
    st[0] = v->q_token_stride; st[1] = v->q_batch_stride;
    st[2] = v->k_token_stride; st[3] = v->k_batch_stride;
    st[4] = v->v_token_stride; st[5] = v->v_batch_stride;
    return;
  }
  st[0] = d->num_heads * d->head_dim_k;
  st[2] = (d->num_heads * d->head_dim_k) << lg;
  st[4] = (d->num_heads * d->head_dim_v) << lg;
  st[1] = rows * st[0]; st[3] = rows * st[2]; st[5] = rows * st[4];
}

// (rows: tokens per batch row; the decode step has one)
static void set_strides(dr::Params& p, const dr_dims* d, int lg, int64_t rows) {
  int64_t st[6];
  input_strides(d, lg, rows, st);
  p.q_ts = st[0]; p.q_bs = st[1]; p.k_ts = st[2]; p.k_bs = st[3]; p.v_ts = st[4]; p.v_bs = st[5];
}

int check_dims_common(const dr_dims* d) {
  if (d == nullptr) return fail(DR_ERR_NULL, "dims is NULL");
  if (d->in_dtype != DR_F32 && d->in_dtype != DR_BF16)
    return fail(DR_ERR_DTYPE, "in_dtype %d is neither DR_F32 nor DR_BF16", d->in_dtype);
  if (d->version != 0 && d->version != DR_DIMS_V2)
    return fail(DR_ERR_SHAPE, "dims.version %d is neither 0 nor DR_DIMS_V2", d->version);
  if (d->version == DR_DIMS_V2) {
    int64_t st[6];
    input_strides(d, 0, d->seqlen, st);
    static const char* names[6] = {"q token", "q batch", "k token", "k batch", "v token", "v batch"};
    const int64_t esz = d->in_dtype == DR_BF16 ? 2 : 4;
    for (int i = 0; i < 6; ++i) {
      if (st[i] < 0) return fail(DR_ERR_SHAPE, "%s stride %lld is negative", names[i], (long long)st[i]);
      if (st[i] > ((int64_t)1 << 40) || (st[i] * esz) % 16 != 0)
        return fail(DR_ERR_LAYOUT, "%s stride %lld is not a multiple of 16 bytes (or is beyond 2^40)", names[i],
                    (long long)st[i]);
    }
  }
  if (d->batch < 0 || d->seqlen < 0 || d->num_heads < 1 || d->num_seqs < 0)
    return fail(DR_ERR_SHAPE, "bad sizes: batch=%lld seqlen=%lld heads=%lld seqs=%lld",
                (long long)d->batch, (long long)d->seqlen, (long long)d->num_heads,
                (long long)d->num_seqs);
  if (!head_dim_ok(d->head_dim_k) || !head_dim_ok(d->head_dim_v))
    return fail(DR_ERR_UNSUPPORTED, "head sizes d_k=%lld d_v=%lld: each must be 16, 32, 64 or 128",
                (long long)d->head_dim_k, (long long)d->head_dim_v);
  // Kernels index with 64-bit offsets but keep (sequence, head) and token counts in 32 bits.
  const int64_t lim = (int64_t)1 << 31;
  if (d->num_heads >= lim || d->num_seqs * d->num_heads >= lim || d->batch * d->seqlen >= lim)
    return fail(DR_ERR_SHAPE, "problem too large for 32-bit token or head counts");
  return DR_OK;
}

int check_ptrs(std::initializer_list<std::pair<const void*, const char*>> req,
               std::initializer_list<std::pair<const void*, const char*>> opt) {
  for (auto& pr : req) {
    if (pr.first == nullptr) return fail(DR_ERR_NULL, "`%s` is NULL", pr.second);
    if (!aligned16(pr.first)) return fail(DR_ERR_LAYOUT, "`%s` is not 16-byte aligned", pr.second);
  }
  for (auto& pr : opt)
    if (pr.first != nullptr && !aligned16(pr.first))
      return fail(DR_ERR_LAYOUT, "`%s` is not 16-byte aligned", pr.second);
  return DR_OK;
}

// Workspace pool of the prefill (per device): stream-ordered allocations that stay cached in
// the pool between calls, so steady-state calls do not reach the device allocator.
hipError_t workspace_alloc(size_t bytes, hipStream_t stream, void** ptr) {
  static std::mutex mu;
  static hipMemPool_t pools[256] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 256) return hipErrorInvalidDevice;
  hipMemPool_t pool;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (!pools[dev]) {
      hipMemPoolProps props = {};
      props.allocType = hipMemAllocationTypePinned;
      props.location.type = hipMemLocationTypeDevice;
      props.location.id = dev;
      e = hipMemPoolCreate(&pools[dev], &props);
      if (e != hipSuccess) {
        pools[dev] = nullptr;
        return e;
      }
      uint64_t keep = UINT64_MAX;
      e = hipMemPoolSetAttribute(pools[dev], hipMemPoolAttrReleaseThreshold, &keep);
      if (e != hipSuccess) return e;
    }
    pool = pools[dev];
  }
  return hipMallocFromPoolAsync(ptr, bytes, pool, stream);
}

// DR_DEBUG_VALIDATE set (and not "0") in the environment: the prefill and backward entry points
// also copy cu_seqlens to the host and check it.
bool debug_validate() {
  const char* e = getenv("DR_DEBUG_VALIDATE");
  return e != nullptr && e[0] != '\0' && !(e[0] == '0' && e[1] == '\0');
}

// DR_BWD_WALK set (and not "0"): the backward takes the exact per-token walk for every call (the
// chunked path is the default where it applies).
bool walk_forced() {
  const char* e = getenv("DR_BWD_WALK");
  return e != nullptr && e[0] != '\0' && !(e[0] == '0' && e[1] == '\0');
}

// cu_seqlens [nseq + 1] (device) must start at 0, never decrease and end at most at `tokens`.
// A synchronising copy on `stream`.
int check_offsets(const int32_t* cu, int64_t nseq, int64_t tokens, hipStream_t stream) {
  std::vector<int32_t> h((size_t)nseq + 1);
  hipError_t e = hipMemcpyAsync(h.data(), cu, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(DR_ERR_HIP, "DR_DEBUG_VALIDATE: reading cu_seqlens failed: %s", hipGetErrorString(e));
  if (h[0] != 0) return fail(DR_ERR_SHAPE, "cu_seqlens[0] is %d, not 0", h[0]);
  for (int64_t n = 0; n < nseq; ++n)
    if (h[n + 1] < h[n])
      return fail(DR_ERR_SHAPE, "cu_seqlens decreases at %lld (%d after %d)", (long long)(n + 1), h[n + 1], h[n]);
  if (h[nseq] > tokens)
    return fail(DR_ERR_SHAPE, "cu_seqlens ends at %d, past the %lld tokens of the row", h[nseq], (long long)tokens);
  return DR_OK;
}

}  // namespace

extern "C" {

const char* dr_status_string(int status) {
  switch (status) {
    case DR_OK: return "DR_OK";
    case DR_ERR_NULL: return "DR_ERR_NULL: a required pointer is NULL";
    case DR_ERR_SHAPE: return "DR_ERR_SHAPE: negative or inconsistent sizes";
    case DR_ERR_DTYPE: return "DR_ERR_DTYPE: unsupported input dtype";
    case DR_ERR_LAYOUT: return "DR_ERR_LAYOUT: pointer not 16-byte aligned, or strides the call does not take";
    case DR_ERR_UNSUPPORTED: return "DR_ERR_UNSUPPORTED: head size not in {16, 32, 64, 128}";
    case DR_ERR_VARIANT: return "DR_ERR_VARIANT: unknown variant or gates that do not fit it";
    case DR_ERR_HIP: return "DR_ERR_HIP: HIP runtime or launch failure";
  }
  return "unknown status";
}

const char* dr_last_error(void) { return g_last_error.c_str(); }

int dr_version(void) { return 200; }

static int prefill_checks(const dr_dims* dims, int variant, const float* erase, const float* write,
                          const int32_t* cu_seqlens, bool* vec) {
  int st = check_dims_common(dims);
  if (st) return st;
  if (variant == DR_PRODUCT2 && dims->batch * dims->seqlen >= ((int64_t)1 << 30))
    return fail(DR_ERR_SHAPE, "problem too large: two transitions per token need 2 * tokens < 2^31 steps");
  st = check_variant(variant, erase, write, dims->batch * dims->seqlen > 0, vec);
  if (st) return st;
  if (cu_seqlens != nullptr) {
    if (dims->batch != 1)
      return fail(DR_ERR_SHAPE, "packed sequences (cu_seqlens) need batch == 1, got %lld",
                  (long long)dims->batch);
  } else if (dims->num_seqs != dims->batch) {
    return fail(DR_ERR_SHAPE, "num_seqs (%lld) must equal batch (%lld) without cu_seqlens",
                (long long)dims->num_seqs, (long long)dims->batch);
  }
  return DR_OK;
}

int dr_chunk_fwd_plan(const dr_dims* dims, int variant, int32_t* chunk, int32_t* dv_block,
                      int64_t* workgroups) {
  g_last_error.clear();
  int st = check_dims_common(dims);
  if (st) return st;
  if (variant < DR_KDA || variant > DR_PRODUCT2) return fail(DR_ERR_VARIANT, "unknown variant %d", variant);
  const int lg = variant == DR_PRODUCT2 ? 1 : 0;
  const dr::PrefillPlan pl = dr::plan_prefill(dims->num_seqs * dims->num_heads, dims->num_seqs, dims->batch,
                                              dims->seqlen << lg, dims->num_heads, (int)dims->head_dim_k,
                                              (int)dims->head_dim_v, dims->batch == 1 && dims->num_seqs != 1);
  if (chunk) *chunk = pl.chunk;
  if (dv_block) *dv_block = pl.dv_block;
  if (workgroups) *workgroups = pl.workgroups;
  return DR_OK;
}

// The prefill's plan; with noalloc, windows small enough that the workspace fits the static scratch
// (when that is possible: packed sequences run as one window).
static dr::PrefillPlan make_plan(const dr_dims* dims, int lg, bool packed, bool noalloc) {
  const int64_t pairs = dims->num_seqs * dims->num_heads;
  dr::PrefillPlan pl = dr::plan_prefill(pairs, dims->num_seqs, dims->batch, dims->seqlen << lg, dims->num_heads,
                                        (int)dims->head_dim_k, (int)dims->head_dim_v, packed);
  if (noalloc && !packed && (uint64_t)pl.workspace > DR_NOALLOC_SCRATCH_BYTES) {
    // smaller windows: the records of one window and the carried state must fit the scratch
    const int64_t carry = pairs * dims->head_dim_k * dims->head_dim_v * 4;
    const int64_t room = (int64_t)DR_NOALLOC_SCRATCH_BYTES - carry;
    if (room > 0)
      pl = dr::plan_prefill(pairs, dims->num_seqs, dims->batch, dims->seqlen << lg, dims->num_heads,
                            (int)dims->head_dim_k, (int)dims->head_dim_v, packed, room);
  }
  return pl;
}

int dr_chunk_fwd_plan_ex(const dr_dims* dims, int variant, int noalloc, dr_plan* plan) {
  g_last_error.clear();
  int st = check_dims_common(dims);
  if (st) return st;
  if (variant < DR_KDA || variant > DR_PRODUCT2) return fail(DR_ERR_VARIANT, "unknown variant %d", variant);
  if (plan == nullptr) return fail(DR_ERR_NULL, "plan is NULL");
  const int lg = variant == DR_PRODUCT2 ? 1 : 0;
  const dr::PrefillPlan pl = make_plan(dims, lg, dims->batch == 1 && dims->num_seqs != 1, noalloc != 0);
  plan->chunk = pl.chunk;
  plan->dv_block = pl.dv_block;
  plan->workgroups = pl.workgroups;
  plan->window_chunks = pl.win_k;
  plan->windows = pl.windows;
  plan->workspace = pl.workspace;
  return DR_OK;
}

// Checks of the options shared by prefill and decode (lg: log2 of the transitions per token).
static int opts_checks(const dr_opts* opts, bool prefill, int lg = 0) {
  if (!opts) return DR_OK;
  if (opts->alpha_dtype != DR_F32 && opts->alpha_dtype != DR_BF16)
    return fail(DR_ERR_DTYPE, "alpha_dtype %d is not DR_F32 / DR_BF16", opts->alpha_dtype);
  if (opts->alpha_act != DR_ACT_NONE && opts->alpha_act != DR_ACT_EXP_NEG_SOFTPLUS && opts->alpha_act != DR_ACT_TANH)
    return fail(DR_ERR_UNSUPPORTED, "alpha_act %d is not a decay activation", opts->alpha_act);
  if (opts->gate_act != DR_ACT_NONE && opts->gate_act != DR_ACT_SIGMOID)
    return fail(DR_ERR_UNSUPPORTED, "gate_act %d is not a gate activation", opts->gate_act);
  if (!std::isfinite(opts->alpha_scale) || !std::isfinite(opts->gate_scale))
    return fail(DR_ERR_UNSUPPORTED, "activation scales must be finite");
  if (opts->l2norm_qk != 0 && opts->l2norm_qk != 1)
    return fail(DR_ERR_UNSUPPORTED, "l2norm_qk must be 0 or 1");
  if (opts->state_idx) {
    if (!aligned16(opts->state_idx)) return fail(DR_ERR_LAYOUT, "state_idx must be 16-byte aligned");
    if (opts->num_slots < 0) return fail(DR_ERR_SHAPE, "num_slots (%lld) is negative", (long long)opts->num_slots);
    if (opts->num_slots > INT32_MAX) return fail(DR_ERR_UNSUPPORTED, "num_slots above 2^31 - 1");
  }
  if (opts->snapshots) {
    if (!prefill) return fail(DR_ERR_SHAPE, "snapshots are a prefill option");
    if (!aligned16(opts->snapshots)) return fail(DR_ERR_LAYOUT, "snapshots must be 16-byte aligned");
    if (opts->snapshot_every <= 0 || (opts->snapshot_every << lg) % 64 != 0)
      return fail(DR_ERR_SHAPE, "snapshot_every (%lld) must be a positive multiple of %d",
                  (long long)opts->snapshot_every, 64 >> lg);
    if (opts->snapshot_every / 64 > INT32_MAX) return fail(DR_ERR_UNSUPPORTED, "snapshot_every too large");
  }
  return DR_OK;
}

// Input-preparation fields of the kernel parameters.
static void set_prep(dr::Params& p, const dr_opts* opts) {
  if (!opts) return;
  p.prep_l2 = opts->l2norm_qk;
  p.a_bf16 = opts->alpha_dtype == DR_BF16;
  p.a_act = opts->alpha_act == DR_ACT_EXP_NEG_SOFTPLUS ? 1 : opts->alpha_act == DR_ACT_TANH ? 2 : 0;
  p.a_scale = opts->alpha_scale;
  p.g_act = opts->gate_act == DR_ACT_SIGMOID ? 1 : 0;
  p.g_scale = opts->gate_scale;
}

int dr_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                 const float* erase, const float* write, int variant,
                 const float* S0, const int32_t* cu_seqlens,
                 float* o, float* S_T, const dr_dims* dims, hipStream_t stream) {
  return dr_chunk_fwd_ex(q, k, v, alpha, erase, write, variant, S0, cu_seqlens, o, S_T, dims, nullptr, stream);
}

// The prefill behind dr_chunk_fwd_ex (workspace from the pool) and dr_chunk_fwd_noalloc (workspace
// in the static scratch array).
static int chunk_fwd_impl(const void* q, const void* k, const void* v, const void* alpha,
                          const float* erase, const float* write, int variant,
                          const float* S0, const int32_t* cu_seqlens,
                          float* o, float* S_T, const dr_dims* dims, const dr_opts* opts,
                          hipStream_t stream, bool noalloc) {
  g_last_error.clear();
  bool vec = false;
  int st = prefill_checks(dims, variant, erase, write, cu_seqlens, &vec);
  if (st) return st;
  const int64_t tokens = dims->batch * dims->seqlen;
  if (tokens > 0) {
    st = check_ptrs({{q, "q"}, {k, "k"}, {v, "v"}, {alpha, "alpha"}, {erase, "erase"}},
                    {{write, "write"}, {o, "o"}});
    if (st) return st;
  }
  st = check_ptrs({}, {{S0, "S0"}, {S_T, "S_T"}, {cu_seqlens, "cu_seqlens"}});
  if (st) return st;
  // two transitions per token run as two steps of the prefill
  const int lg = variant == DR_PRODUCT2 ? 1 : 0;
  st = opts_checks(opts, true, lg);
  if (st) return st;
  if (cu_seqlens != nullptr && debug_validate()) {
    st = check_offsets(cu_seqlens, dims->num_seqs, dims->seqlen, stream);
    if (st) return st;
  }
  if (cu_seqlens == nullptr && dims->num_seqs > 0 && dims->seqlen == 0 && S_T == nullptr)
    return DR_OK;  // nothing to compute and nothing to write (no snapshot fits in zero tokens)
  if (dims->num_seqs == 0) return DR_OK;

  dr::Params p{};
  p.q = q; p.k = k; p.v = v; p.alpha = alpha;
  p.erase = erase;
  p.write = (variant == DR_RDA || variant == DR_GDN2) ? write : erase;
  p.S0 = S0; p.cu = cu_seqlens; p.o = o; p.S = S_T;
  p.lgnh = lg;
  set_strides(p, dims, lg, dims->seqlen);
  p.T = dims->seqlen << lg;
  p.H = (int32_t)dims->num_heads;
  p.DV = (int32_t)dims->head_dim_v;
  const int64_t pairs = dims->num_seqs * dims->num_heads;
  const dr::PrefillPlan pl = make_plan(dims, lg, cu_seqlens != nullptr, noalloc);
  if (pl.workgroups > INT32_MAX || pl.slots * dims->num_heads > INT32_MAX)
    return fail(DR_ERR_UNSUPPORTED, "problem too large: more than 2^31 - 1 workgroups per kernel");
  p.num_pairs = (int32_t)pairs;
  p.ndvb = pl.ndvb;
  p.grid_logical = (int32_t)(pairs * pl.ndvb);
  p.nseq = (int32_t)dims->num_seqs;
  if (opts) {
    p.sidx = opts->state_idx;
    p.nslots = opts->num_slots;
    p.snap = opts->snapshots;
    p.snap_chunks = opts->snapshots ? (int32_t)((opts->snapshot_every << lg) / 64) : 0;
  }
  set_prep(p, opts);
  void* ws = nullptr;
  hipError_t e = hipSuccess;
  if (noalloc) {
    if ((uint64_t)pl.workspace > DR_NOALLOC_SCRATCH_BYTES)
      return fail(DR_ERR_UNSUPPORTED, "dr_chunk_fwd_noalloc: this problem needs %lld bytes of workspace, above the "
                  "%llu-byte static scratch (split the call, or use dr_chunk_fwd_ex)", (long long)pl.workspace,
                  (unsigned long long)DR_NOALLOC_SCRATCH_BYTES);
    if (pl.workspace > 0) {
      e = dr::scratch_buffer(&ws);
      if (e != hipSuccess) return fail(DR_ERR_HIP, "static scratch lookup failed: %s", hipGetErrorString(e));
    }
  } else if (pl.workspace > 0) {
    e = workspace_alloc((size_t)pl.workspace, stream, &ws);
    if (e != hipSuccess)
      return fail(DR_ERR_HIP, "prefill workspace (%lld bytes) allocation failed: %s", (long long)pl.workspace,
                  hipGetErrorString(e));
  }
  e = dr::launch_prefill(p, pl, ws, (int)dims->head_dim_k, dims->in_dtype == DR_BF16, vec, stream);
  hipError_t ef = (ws && !noalloc) ? hipFreeAsync(ws, stream) : hipSuccess;
  if (e != hipSuccess) return fail(DR_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
  if (ef != hipSuccess) return fail(DR_ERR_HIP, "prefill workspace release failed: %s", hipGetErrorString(ef));
  return DR_OK;
}

int dr_chunk_fwd_ex(const void* q, const void* k, const void* v, const void* alpha,
                    const float* erase, const float* write, int variant,
                    const float* S0, const int32_t* cu_seqlens,
                    float* o, float* S_T, const dr_dims* dims, const dr_opts* opts,
                    hipStream_t stream) {
  return chunk_fwd_impl(q, k, v, alpha, erase, write, variant, S0, cu_seqlens, o, S_T, dims, opts, stream, false);
}

int dr_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* alpha,
                         const float* erase, const float* write, int variant,
                         const float* S0, const int32_t* cu_seqlens,
                         float* o, float* S_T, const dr_dims* dims, const dr_opts* opts,
                         hipStream_t stream) {
  return chunk_fwd_impl(q, k, v, alpha, erase, write, variant, S0, cu_seqlens, o, S_T, dims, opts, stream, true);
}

static int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }

int dr_chunk_bwd(const void* q, const void* k, const void* v, const float* alpha,
                 const float* erase, const float* write, int variant,
                 const float* S0, const int32_t* cu_seqlens,
                 const float* dO, const float* dS_T,
                 float* dq, float* dk, float* dv, float* dalpha, float* derase, float* dwrite,
                 float* dS0, const dr_dims* dims, hipStream_t stream) {
  return dr_chunk_bwd_ex(q, k, v, alpha, erase, write, variant, S0, cu_seqlens, dO, dS_T, dq, dk, dv, dalpha,
                         derase, dwrite, dS0, nullptr, dims, stream);
}

int dr_chunk_bwd_ex(const void* q, const void* k, const void* v, const float* alpha,
                    const float* erase, const float* write, int variant,
                    const float* S0, const int32_t* cu_seqlens,
                    const float* dO, const float* dS_T,
                    float* dq, float* dk, float* dv, float* dalpha, float* derase, float* dwrite,
                    float* dS0, const float* checkpoints, const dr_dims* dims, hipStream_t stream) {
  g_last_error.clear();
  bool vec = false;
  int st = prefill_checks(dims, variant, erase, write, cu_seqlens, &vec);
  if (st) return st;
  const bool has_write = variant == DR_RDA || variant == DR_GDN2;
  const int lg = variant == DR_PRODUCT2 ? 1 : 0;  // two transitions per token: 2T steps
  if (!has_write && dwrite != nullptr)
    return fail(DR_ERR_VARIANT, "KDA / CKDA take no dwrite (beta's whole gradient goes to derase)");
  const int64_t tokens = dims->batch * dims->seqlen;
  if (tokens > 0) {
    st = check_ptrs({{q, "q"}, {k, "k"}, {v, "v"}, {alpha, "alpha"}, {erase, "erase"}, {dO, "dO"},
                     {dq, "dq"}, {dk, "dk"}, {dv, "dv"}, {dalpha, "dalpha"}, {derase, "derase"}},
                    {{write, "write"}});
    if (st) return st;
    if (has_write && dwrite == nullptr) return fail(DR_ERR_NULL, "dwrite is required for RDA / GDN-2");
  }
  st = check_ptrs({}, {{S0, "S0"}, {dS_T, "dS_T"}, {dS0, "dS0"}, {cu_seqlens, "cu_seqlens"}, {dwrite, "dwrite"},
                       {checkpoints, "checkpoints"}});
  if (st) return st;
  if (cu_seqlens != nullptr && debug_validate()) {
    st = check_offsets(cu_seqlens, dims->num_seqs, dims->seqlen, stream);
    if (st) return st;
  }
  if (dims->num_seqs == 0) return DR_OK;
  const int dkh = (int)dims->head_dim_k, dvh = (int)dims->head_dim_v;
  const int64_t H = dims->num_heads, pairs = dims->num_seqs * H;

  // the states after every 64 steps: the caller's (a prefill's snapshots), or a forward pass
  // with no output
  dr::Params p{};
  p.q = q; p.k = k; p.v = v; p.alpha = alpha;
  p.erase = erase;
  p.write = has_write ? write : erase;
  p.S0 = S0; p.cu = cu_seqlens; p.o = nullptr; p.S = nullptr;
  p.lgnh = lg;
  set_strides(p, dims, lg, dims->seqlen);
  p.T = dims->seqlen << lg;
  p.H = (int32_t)H;
  p.DV = (int32_t)dvh;
  const dr::PrefillPlan pl = dr::plan_prefill(pairs, dims->num_seqs, dims->batch, dims->seqlen << lg, H, dkh, dvh,
                                              cu_seqlens != nullptr);
  if (pl.workgroups > INT32_MAX || pl.slots * H > INT32_MAX || pairs * (dvh / dr::bwd_dv_block(dvh)) > INT32_MAX)
    return fail(DR_ERR_UNSUPPORTED, "problem too large: more than 2^31 - 1 workgroups per kernel");
  p.num_pairs = (int32_t)pairs;
  p.ndvb = pl.ndvb;
  p.grid_logical = (int32_t)(pairs * pl.ndvb);
  p.nseq = (int32_t)dims->num_seqs;
  p.snap_chunks = 1;
  // at most floor(steps / 64) checkpoints in all (sum of floor(len_n / 64) over the sequences)
  const int64_t steps = tokens << lg;
  const int64_t nsnap = cu_seqlens ? steps / 64 : dims->batch * ((dims->seqlen << lg) / 64);
  const int ndvb = dvh / dr::bwd_dv_block(dvh);
  const int64_t TH = steps * H;
  // with the caller's checkpoints only the packed plan's tables are needed, not the records
  dr::PrefillPlan plw = pl;
  if (checkpoints) {
    plw.workspace -= pl.slots * H * pl.rec_size;
    plw.rec_size = 0;
  }
  // The chunked MFMA path (one or two transitions per token, d_k 64 or 128, d_v a multiple of 32
  // up to 128) runs first; the walk's kernels then run only if it flagged a chunk whose gates
  // it does not take. Its records and chunk-end gradients share the walk's partial-sum buffers
  // (the walk writes them only when it runs, after the chunked passes are done with them); the
  // flag sits apart.
  const bool chunked = (dkh == 64 || dkh == 128) && dvh % 32 == 0 && dvh <= 128 && dims->seqlen > 0 &&
                       !walk_forced();
  const int64_t ncpb = ((dims->seqlen << lg) + 63) / 64;  // 64-step chunks per sequence
  // chunk slots x heads: fixed length B x chunks per sequence, packed the plan's upper bound
  const int64_t cslots = (cu_seqlens ? pl.slots : dims->batch * ncpb) * H;
  const int64_t crec = chunked ? dr::cbwd_record_bytes(dkh, dvh) : 0;
  const int64_t chunk_bytes = chunked ? round256(cslots * crec) + round256(cslots * dkh * dvh * 4) : 0;
  if (chunked && cslots > INT32_MAX)
    return fail(DR_ERR_UNSUPPORTED, "problem too large: more than 2^31 - 1 workgroups per kernel");
  const int64_t off_snap = round256(plw.workspace);
  const int64_t off_part = off_snap + (checkpoints ? 0 : round256(nsnap * H * dkh * dvh * 4));
  const int64_t off_parts = off_part + round256((int64_t)ndvb * TH * 4 * dkh * 4);
  const int64_t walk_end = off_parts + round256((int64_t)ndvb * TH * 4);
  const int64_t off_flag = walk_end > off_part + chunk_bytes ? walk_end : off_part + chunk_bytes;
  const int64_t total = off_flag + 256;
  void* ws = nullptr;
  hipError_t e = workspace_alloc((size_t)total, stream, &ws);
  if (e != hipSuccess)
    return fail(DR_ERR_HIP, "backward workspace (%lld bytes) allocation failed: %s", (long long)total,
                hipGetErrorString(e));
  unsigned char* wsb = static_cast<unsigned char*>(ws);
  if (checkpoints) {
    // read only here: the plan pass uses the pointer's presence to lay out the rows
    p.snap = nsnap > 0 ? const_cast<float*>(checkpoints) : nullptr;
    if (p.snap == nullptr) p.snap_chunks = 0;
    e = dr::launch_plan_only(p, plw, ws, stream);
  } else {
    p.snap = nsnap > 0 ? reinterpret_cast<float*>(wsb + off_snap) : nullptr;
    if (p.snap == nullptr) p.snap_chunks = 0;
    e = dr::launch_prefill(p, pl, ws, dkh, dims->in_dtype == DR_BF16, vec, stream);
  }
  if (e == hipSuccess) {
    dr::BwdParams b{};
    b.q = q; b.k = k; b.v = v; b.alpha = alpha;
    b.erase = erase;
    b.write = p.write;
    b.S0 = S0; b.dO = dO; b.dST = dS_T;
    b.cu = cu_seqlens ? dr::prefill_cu_table(ws, plw, H, dims->num_seqs) : nullptr;  // the plan pass's clamped copy
    b.dq = dq; b.dk = dk; b.dv = dv; b.dalpha = dalpha; b.derase = derase; b.dwrite = dwrite; b.dS0 = dS0;
    b.snap = p.snap;
    b.snap_first = cu_seqlens ? dr::prefill_snap_first(ws, plw, H, dims->num_seqs) : nullptr;
    b.seq_order = cu_seqlens ? b.snap_first + dims->num_seqs : nullptr;  // written by the prefill's plan pass
    b.part = reinterpret_cast<float*>(wsb + off_part);
    b.parts = reinterpret_cast<float*>(wsb + off_parts);
    b.T = dims->seqlen << lg;
    b.TH = TH;
    b.lgnh = lg;
    b.H = (int32_t)H;
    b.DV = dvh;
    b.nseq = (int32_t)dims->num_seqs;
    b.variant = variant;
    b.q_ts = p.q_ts; b.q_bs = p.q_bs; b.k_ts = p.k_ts; b.k_bs = p.k_bs; b.v_ts = p.v_ts; b.v_bs = p.v_bs;
    if (dims->version == DR_DIMS_V2) {  // dense strides given as a dr_dims_v2 take the dense instance
      dr_dims dense = *dims;
      dense.version = 0;
      int64_t a[6], d[6];
      input_strides(dims, lg, dims->seqlen, a);
      input_strides(&dense, lg, dims->seqlen, d);
      for (int j = 0; j < 6; ++j)
        if (a[j] != d[j] && !(j % 2 == 1 && dims->batch <= 1)) b.strided = 1;
    }
    if (chunked) {
      dr::CbParams cb{};
      cb.q = q; cb.k = k; cb.v = v; cb.alpha = alpha;
      cb.erase = erase;
      cb.write = p.write;
      cb.S0 = S0; cb.dO = dO; cb.dST = dS_T; cb.snap = p.snap;
      cb.dq = dq; cb.dk = dk; cb.dv = dv; cb.dalpha = dalpha; cb.derase = derase; cb.dwrite = dwrite;
      cb.dS0 = dS0;
      cb.rec = wsb + off_part;
      cb.rec_size = crec;
      cb.dsc = reinterpret_cast<float*>(wsb + off_part + round256(cslots * crec));
      cb.flag = reinterpret_cast<int32_t*>(wsb + off_flag);
      cb.T = dims->seqlen << lg;
      cb.H = (int32_t)H;
      cb.DV = dvh;
      cb.B = (int32_t)dims->batch;
      cb.nc = (int32_t)ncpb;
      cb.nseq = (int32_t)dims->num_seqs;
      cb.slots = (int32_t)(cslots / H);
      if (cu_seqlens) {  // the plan pass's tables (written by the forward or by launch_plan_only above)
        int32_t* tab = dr::prefill_chunk_tables(ws, plw, H);
        cb.cu = b.cu;
        cb.chunk_seq = tab;
        cb.chunk_c0 = tab + plw.slots;
        cb.seq_first = tab + 2 * plw.slots;
        cb.snap_first = b.snap_first;
        cb.seq_order = b.seq_order;
      }
      cb.variant = variant;
      cb.lgnh = lg;
      cb.q_ts = p.q_ts; cb.q_bs = p.q_bs; cb.k_ts = p.k_ts; cb.k_bs = p.k_bs; cb.v_ts = p.v_ts; cb.v_bs = p.v_bs;
      e = dr::launch_chunked_backward(cb, dkh, dims->in_dtype == DR_BF16, vec, stream);
      b.run_flag = cb.flag;
    }
    if (e == hipSuccess) e = dr::launch_backward(b, pairs, dkh, dvh, dims->in_dtype == DR_BF16, vec, stream);
  }
  hipError_t ef = hipFreeAsync(ws, stream);
  if (e != hipSuccess) return fail(DR_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
  if (ef != hipSuccess) return fail(DR_ERR_HIP, "backward workspace release failed: %s", hipGetErrorString(ef));
  return DR_OK;
}

int dr_decode_step(const void* q, const void* k, const void* v, const float* alpha,
                   const float* erase, const float* write, int variant,
                   float* S, float* o, const dr_dims* dims, hipStream_t stream) {
  return dr_decode_step_ex(q, k, v, alpha, erase, write, variant, S, o, dims, nullptr, stream);
}

int dr_decode_step_ex(const void* q, const void* k, const void* v, const void* alpha,
                      const float* erase, const float* write, int variant,
                      float* S, float* o, const dr_dims* dims, const dr_opts* opts,
                      hipStream_t stream) {
  g_last_error.clear();
  int st = check_dims_common(dims);
  if (st) return st;
  bool vec = false;
  st = check_variant(variant, erase, write, dims->num_seqs > 0, &vec);
  if (st) return st;
  if (dims->num_seqs != dims->batch)
    return fail(DR_ERR_SHAPE, "decode: num_seqs (%lld) must equal batch (%lld)",
                (long long)dims->num_seqs, (long long)dims->batch);
  const int64_t nheads = dims->num_seqs * dims->num_heads;
  if (nheads == 0) return DR_OK;
  st = check_ptrs({{q, "q"}, {k, "k"}, {v, "v"}, {alpha, "alpha"}, {erase, "erase"}, {S, "S"}, {o, "o"}},
                  {{write, "write"}});
  if (st) return st;
  st = opts_checks(opts, false);
  if (st) return st;
  dr::Params p{};
  if (opts) {
    p.sidx = opts->state_idx;
    p.nslots = opts->num_slots;
  }
  set_prep(p, opts);
  p.q = q; p.k = k; p.v = v; p.alpha = alpha;
  p.erase = erase;
  p.write = (variant == DR_RDA || variant == DR_GDN2) ? write : erase;
  p.o = o; p.S = S;
  p.H = (int32_t)dims->num_heads;
  p.DV = (int32_t)dims->head_dim_v;
  set_strides(p, dims, variant == DR_PRODUCT2 ? 1 : 0, 1);
  hipError_t e = variant == DR_PRODUCT2
                     ? dr::launch_decode2(p, nheads, (int)dims->head_dim_k, (int)dims->head_dim_v,
                                          dims->in_dtype == DR_BF16, stream)
                     : dr::launch_decode(p, nheads, (int)dims->head_dim_k, (int)dims->head_dim_v,
                                         dims->in_dtype == DR_BF16, vec, stream);
  if (e != hipSuccess) return fail(DR_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return DR_OK;
}

}  // extern "C"
