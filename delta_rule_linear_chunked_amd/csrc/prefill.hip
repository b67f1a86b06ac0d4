// Chunkwise-parallel prefill of the gated delta rule on gfx950.
//
// The recurrence S_t = Diag(alpha_t) S_{t-1} + k_t delta_t^T with
// delta_t = m_t - S_{t-1}^T (alpha_t . u_t) and o_t = S_t^T q_t (the KDA, RDA and
// GDN-2 rules of the Hugging Face discussion "KRAFTON/Raon-1-mini-preview" #1,
// with the erase/write vectors u, m of each rule; Complex KDA uses KDA's rule
// with signed gates) is evaluated 64 tokens at a time. Inside a chunk with
// start state S0 and ratio(r, s) = prod_{j=s+1..r} alpha_j:
//
//   A[r,s] = sum_i u_ri k_si ratio(r,s)_i   (s < r)        P[r,s] likewise with q (s <= r)
//   T      = (I + A)^-1
//   delta  = T (M - Utilde S0),              Utilde_r = Gamma_r . u_r
//   O      = Qtilde S0 + P delta,            Qtilde_r = Gamma_r . q_r
//   S_C    = Diag(Gamma_C) S0 + Kbar^T delta, Kbar_s = ratio(C, s) . k_s
//
// (derived by unrolling the step rule; the course page "GDN, KDA và Mamba-2",
// section 3, asks for such a chunked kernel to be checked against the step
// recurrence).
//
// Two passes. chunk_prep_kernel (one workgroup per chunk and head, all chunks in
// parallel) computes everything that does not depend on the state — gate
// products, A, P, T, Utilde, Qtilde, Kbar, Gamma_C — and writes it to a
// workspace record as MFMA operand fragments. chunk_state_kernel (prefill_state.hip; one workgroup
// per sequence, head and block of value columns) then walks the chunks in order
// with the state held in registers, doing only the state-dependent products.
//
// Gate preparation uses signed products, never logarithms, because Complex KDA
// gates may be negative or zero. Each chunk is split into four 16-token blocks;
// per key channel the kernel forms, with DPP scans across the 16 lanes that hold
// a block's rows:
//   f_r = prod of alpha from the block start to r (inclusive)
//   g_s = prod of alpha from s+1 to the block end
//   t_J = total product of block J
// so that for r in block I and s in block J < I
//   ratio(r, s) = f_r * (prod_{J<J'<I} t_J') * g_s     (every factor in [-1, 1] when |alpha| <= 1)
// and inside a block ratio(r, s) = f_r * (1 / f_s), g_s = t_J / f_s. The in-block
// factorisation is used only while every |f| of the block lies in [2^-100, 2^100];
// otherwise (gates at or extremely close to zero) the block's diagonal tiles and
// g come from running products, which are exact for any gate value.
#include <type_traits>

#include "prefill.hpp"

namespace dr {

constexpr int LDT = 68;   // padded row stride of 64-wide fp32 tiles
constexpr float FAST_LO = 0x1p-100f;
constexpr float FAST_HI = 0x1p100f;

// Sequence, first token, length and record slot of the chunk that workgroup slot `slot` prepares.
// Returns false for an unused slot.
__device__ __forceinline__ bool resolve_slot(const Params& p, int slot, int& n, int64_t& bos, int64_t& len,
                                             int64_t& c0, int& rslot) {
  if (p.cu) {
    n = p.chunk_seq[slot];
    if (n < 0) return false;
    bos = cu_steps(p, n);
    len = cu_steps(p, n + 1) - bos;
    c0 = p.chunk_c0[slot];
    rslot = slot;
  } else {  // chunk win_c0 + slot % win_nc of sequence slot / win_nc
    n = slot / p.win_nc;
    const int cw = slot % p.win_nc;
    bos = (int64_t)n * p.T;
    len = p.T;
    c0 = (int64_t)(p.win_c0 + cw) * CH;
    rslot = n * p.win_k + cw;
  }
  return true;
}

// ============================================================================ pass 0
// Packed sequences: first chunk slot of each sequence (exclusive scan of the chunk
// counts), first snapshot row of each sequence, the sequences in order of decreasing
// chunk count (the state pass's order), and, for every slot, its sequence and first
// token. One workgroup.
__global__ __launch_bounds__(256) void chunk_plan_kernel(Params p) {
  __shared__ int s_scan[256];
  __shared__ int s_carry;
  const int tid = threadIdx.x;
  // The offsets, clamped to [0, tokens] and made non-decreasing by a running maximum, into
  // cu_ok; this pass and the later ones take every span from that copy, so a malformed
  // cu_seqlens gives wrong spans but no access outside the token rows, the chunk slots or the
  // snapshot rows those spans imply.
  {
    const int32_t ntok = (int32_t)(p.T >> p.lgnh);
    if (tid == 0) s_carry = 0;
    __syncthreads();
    for (int base = 0; base <= p.nseq; base += 256) {
      const int n = base + tid;
      int x = n <= p.nseq ? min(max(p.cu[n], 0), ntok) : 0;
      s_scan[tid] = x;
      __syncthreads();
      for (int d = 1; d < 256; d <<= 1) {
        const int y = tid >= d ? s_scan[tid - d] : 0;
        __syncthreads();
        s_scan[tid] = max(s_scan[tid], y);
        __syncthreads();
      }
      if (n <= p.nseq) p.cu_ok[n] = max(s_scan[tid], s_carry);
      __syncthreads();
      if (tid == 255) s_carry = max(s_carry, s_scan[255]);
      __syncthreads();
    }
    p.cu = p.cu_ok;  // (the workgroup-scope fence of the barriers above covers global memory)
  }
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < p.nseq; base += 256) {
    const int n = base + tid;
    const int nc = n < p.nseq ? (int)((cu_steps(p, n + 1) - cu_steps(p, n) + CH - 1) / CH) : 0;
    s_scan[tid] = nc;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
      const int x = tid >= d ? s_scan[tid - d] : 0;
      __syncthreads();
      s_scan[tid] += x;
      __syncthreads();
    }
    if (n < p.nseq) p.seq_first[n] = s_carry + s_scan[tid] - nc;
    __syncthreads();
    if (tid == 255) s_carry += s_scan[255];
    __syncthreads();
  }
  const int total = s_carry;
  if (tid == 0) p.seq_first[p.nseq] = total;
  __syncthreads();  // seq_first complete (the workgroup-scope fence covers global memory)
  if (p.snap) {  // first snapshot row of each sequence: exclusive scan of floor(len / stride)
    if (tid == 0) s_carry = 0;
    __syncthreads();
    const int stride = p.snap_chunks * CH;
    for (int base = 0; base < p.nseq; base += 256) {
      const int n = base + tid;
      const int ns = n < p.nseq ? (int)((cu_steps(p, n + 1) - cu_steps(p, n)) / stride) : 0;
      s_scan[tid] = ns;
      __syncthreads();
      for (int d = 1; d < 256; d <<= 1) {
        const int x = tid >= d ? s_scan[tid - d] : 0;
        __syncthreads();
        s_scan[tid] += x;
        __syncthreads();
      }
      if (n < p.nseq) p.snap_first[n] = s_carry + s_scan[tid] - ns;
      __syncthreads();
      if (tid == 255) s_carry += s_scan[255];
      __syncthreads();
    }
  }
  // sequences by decreasing chunk count (ties by index): the state pass starts the longest
  // chains first. Ranked by comparison for up to 1024 sequences, else kept in index order.
  {
    __shared__ int s_nc[1024];
    if (p.nseq <= 1024) {
      for (int n = tid; n < p.nseq; n += 256) s_nc[n] = (int)((cu_steps(p, n + 1) - cu_steps(p, n) + CH - 1) / CH);
      __syncthreads();
      for (int n = tid; n < p.nseq; n += 256) {
        const int c = s_nc[n];
        int r = 0;
        for (int m = 0; m < p.nseq; ++m) {
          const int cm = s_nc[m];
          r += (cm > c || (cm == c && m < n)) ? 1 : 0;
        }
        p.seq_order[r] = n;
      }
    } else {
      for (int n = tid; n < p.nseq; n += 256) p.seq_order[n] = n;
    }
  }
  for (int slot = tid; slot < p.slots; slot += 256) {
    int n = -1, c0 = 0;
    if (slot < total) {
      int lo = 0, hi = p.nseq;  // last sequence whose first slot is <= slot
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.seq_first[mid] <= slot) lo = mid; else hi = mid;
      }
      n = lo;
      c0 = (slot - p.seq_first[lo]) * CH;
    }
    p.chunk_seq[slot] = n;
    p.chunk_c0[slot] = c0;
  }
}

// ============================================================================ pass 1
template <int DK>
struct PrepSmem {
  float tot[NBLK][DK];      // t_J
  float A[CH][LDT];         // A (strictly lower)
  float Td[NBLK][16][20];   // (I + A_JJ)^-1
  union { float P[CH][LDT]; float At[CH][LDT]; } u1;      // P, later T_II A_IK
  union { float kg[CH][DK + 4]; float T[CH][LDT]; } u2;   // k . g, later T
};

// Eight decay values at element `i` of alpha for alpha mode AM: 0 float32 as given,
// 1 float32 pre-activations, 2 bfloat16 pre-activations (activated here); 3 and 4 return
// the bfloat16 / float32 pre-activations themselves.
template <int AM, int ACT = 0>
__device__ __forceinline__ void load_alpha(const Params& p, int64_t i, float (&a)[8]) {
  if constexpr (AM == 2 || AM == 3) load8(static_cast<const __bf16*>(p.alpha) + i, a);
  else load8(static_cast<const float*>(p.alpha) + i, a);
  if constexpr (AM == 1 || AM == 2) {
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = prep_alpha_as<ACT>(a[j], p.a_scale);
  }
}

// A block with a gate at or extremely near zero (rare): k . g from exact suffix products and
// the diagonal tiles of A and P from running products of the gates, exact for any gate value.
template <int DKR, int DK, typename InT, bool VEC, int AM, int ACT>
__device__ __forceinline__ void exact_block(const Params& p, PrepSmem<DK>& sm, int64_t thq, int64_t thk, int64_t qo,
                                         int64_t ko, bool unit_a, bool valid, float esc,
                                         float rq, float rk, int w, int r, int g) {
  constexpr int KS = DK / 32;
  const int row = 16 * w + r;
  const InT* qp = static_cast<const InT*>(p.q);
  const InT* kp = static_cast<const InT*>(p.k);
  auto alpha8 = [&](int64_t i, float (&a)[8]) { load_alpha<AM, ACT>(p, i, a); };
  auto gate = [&](float z) {
    if constexpr (AM != 0) return prep_gate(z, p);
    else return z;
  };
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int ch0 = 32 * ks + 8 * g;
    const bool live = valid && ch0 < DKR;
    float a8[8], k8[8];
    alpha8(thq * DKR + (live ? ch0 : 0), a8);
    load8(kp + ko + (live ? ch0 : 0), k8);
    float kgv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) kgv[j] = (live ? k8[j] * rk : 0.f) * row_suffix_prod_excl(live && !unit_a ? a8[j] : 1.f);
    store4(&sm.u2.kg[row][ch0], f32x4{kgv[0], kgv[1], kgv[2], kgv[3]});
    store4(&sm.u2.kg[row][ch0 + 4], f32x4{kgv[4], kgv[5], kgv[6], kgv[7]});
  }
  for (int s = 0; s < 16; ++s) {
    float ap = 0.f, pp = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch0 = 32 * ks + 8 * g;
      const bool live = valid && ch0 < DKR;
      float a2[8], k2[8], q2[8], b2[8];
      load_alpha<AM == 0 ? 0 : AM == 2 ? 3 : 4>(p, thq * DKR + (live ? ch0 : 0), a2);  // raw
      load8(kp + ko + (live ? ch0 : 0), k2);
      load8(qp + qo + (live ? ch0 : 0), q2);
      if constexpr (VEC) load8(p.erase + thk * DKR + (live ? ch0 : 0), b2);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float a = 1.f;
        if (live && !unit_a) {
          if constexpr (AM != 0) a = prep_alpha_as<ACT>(a2[j], p.a_scale);  // one element at a time
          else a = a2[j];
        }
        const float kk = live ? k2[j] * rk : 0.f;
        const float qq = live ? q2[j] * rq : 0.f;
        const float uu = (VEC ? gate(b2[j]) : esc) * kk;
        const float rho = row_prefix_prod(r > s ? a : 1.f);
        const float kv = __shfl(kk, 16 * g + s);
        ap = fmaf(uu * kv, rho, ap);
        pp = fmaf(qq * kv, rho, pp);
      }
    }
    ap += __shfl_xor(ap, 16);
    ap += __shfl_xor(ap, 32);
    pp += __shfl_xor(pp, 16);
    pp += __shfl_xor(pp, 32);
    if (g == 0) {
      sm.A[16 * w + r][16 * w + s] = (r > s) ? ap : 0.f;
      sm.u1.P[16 * w + r][16 * w + s] = (r >= s) ? pp : 0.f;
    }
  }
}
template <int DKR, typename InT, bool VEC, int AM, int ACT>
__global__ __launch_bounds__(256, 2) void chunk_prep_kernel(const Params p) {
  using Pol = typename PolicyFor<InT>::type;
  using Frag = typename Pol::Frag;
  constexpr int DK = DKR < 32 ? 32 : DKR;  // key width padded to the 32-deep MFMA slice
  constexpr int KS = DK / 32;
  using R = Rec<DK>;

  __shared__ __align__(16) PrepSmem<DK> sm;

  const int slot = blockIdx.x / p.H;
  const int h = blockIdx.x % p.H;
  int n, rslot;
  int64_t bos, len, c0;
  if (!resolve_slot(p, slot, n, bos, len, c0, rslot)) return;
  unsigned char* rec = p.rec + ((int64_t)h * p.slots + rslot) * p.rec_size;  // a head's chunks are adjacent
  const __amdgpu_buffer_rsrc_t rs = rec_rsrc(rec, p.rec_size);
  const int wu = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // the wave index, uniform
  const int H = p.H;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, r = l & 15, g = l >> 4;
  const InT* qp = static_cast<const InT*>(p.q);
  const InT* kp = static_cast<const InT*>(p.k);
  // decay and gate loads, with the fused activations unless AM == 0
  auto alpha8 = [&](int64_t i, float (&a)[8]) { load_alpha<AM, ACT>(p, i, a); };
  auto gate = [&](float z) {
    if constexpr (AM != 0) return prep_gate(z, p);
    else return z;
  };

  // upper blocks of P are read (as zeros) by the state pass's 32-deep steps
  for (int i = tid; i < CH * LDT; i += 256) (&sm.u1.P[0][0])[i] = 0.f;

  const int row = 16 * w + r;
  const bool valid = c0 + row < len;
  // rows of this lane's step in the per-token (q, alpha) and per-step (k, gates) arrays; the
  // decay acts on the first step of a token only
  const int64_t mstep = bos + c0 + (valid ? row : 0);
  const int64_t thq = tok_row(p, mstep, h), thk = step_row(p, mstep, h);
  // q and k through their strides (alpha and the gates are dense: rows thq, thk)
  const int64_t brow = p.cu ? 0 : n, srow = p.cu ? mstep : mstep - bos;
  const int64_t qo = q_elem(p, brow, srow, h, DKR), ko = kv_elem(p.k_ts, p.k_bs, p, brow, srow, h, DKR);
  const bool unit_a = (mstep & ((1 << p.lgnh) - 1)) != 0;

  // ---------------------------------------------------------------- input preparation
  // With fused preparation the row's decay pre-activations are loaded first, so that their
  // latency overlaps the q/k norm pass, and activated as independent chains afterwards.
  float av[AM != 0 ? KS : 1][8];
  if constexpr (AM != 0) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch0 = 32 * ks + 8 * g;
      load_alpha<AM == 2 ? 3 : 4>(p, thq * DKR + (valid && ch0 < DKR ? ch0 : 0), av[ks]);  // raw
    }
  }
  // inverse L2 norms of this row's q and k over d_k (1 when the inputs come normalised): the
  // row's channels are spread over the four lanes l, l^16, l^32, l^48
  float rq = 1.f, rk = 1.f;
  if (AM != 0 && p.prep_l2) {
    float sq = 0.f, sk = 0.f;
    typename Raw8Of<InT>::type kn[KS], qn[KS];  // every slice's loads issued first (see below)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch0 = 32 * ks + 8 * g, cl = ch0 < DKR ? ch0 : 0;
      ld_raw8(kp + ko + cl, kn[ks]);
      ld_raw8(qp + qo + cl, qn[ks]);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bool live = valid && 32 * ks + 8 * g < DKR;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float qv = live ? raw8_at(qn[ks], j) : 0.f, kv = live ? raw8_at(kn[ks], j) : 0.f;
        sq = fmaf(qv, qv, sq);
        sk = fmaf(kv, kv, sk);
      }
    }
    sq += __shfl_xor(sq, 16);
    sq += __shfl_xor(sq, 32);
    sk += __shfl_xor(sk, 16);
    sk += __shfl_xor(sk, 32);
    rq = sq > 0.f ? __builtin_amdgcn_rsqf(sq) : 0.f;
    rk = sk > 0.f ? __builtin_amdgcn_rsqf(sk) : 0.f;
  }
  if constexpr (AM != 0) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int j = 0; j < 8; ++j) av[ks][j] = unit_a ? 1.f : prep_alpha_as<ACT>(av[ks][j], p.a_scale);
    }
  }

  // ---------------------------------------------------------------- gate preparation
  float uf[KS][8], qf[KS][8];  // u . f and q . f of this lane's row
  {
    bool ok = true;
    f32x4 ad = f32x4{0.f, 0.f, 0.f, 0.f}, pd = ad;
    const float esc = (!VEC && valid) ? gate(p.erase[thk]) : 0.f;
    // All slices' loads are issued before any is used: every lane loads (rows past the sequence
    // end read the chunk's first row, channels past d_k channel 0) and the values are selected
    // afterwards. Loads under the condition, slice by slice, were each waited for before the next
    // slice's were issued.
    typename Raw8Of<InT>::type kr[KS], qr[KS];
    float ar[AM != 0 ? 1 : KS][8], br[VEC ? KS : 1][8];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch0 = 32 * ks + 8 * g, cl = ch0 < DKR ? ch0 : 0;
      ld_raw8(kp + ko + cl, kr[ks]);
      ld_raw8(qp + qo + cl, qr[ks]);
      if constexpr (AM == 0) alpha8(thq * DKR + cl, ar[ks]);
      if constexpr (VEC) load8(p.erase + thk * DKR + cl, br[ks]);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch0 = 32 * ks + 8 * g;
      const bool live = valid && ch0 < DKR;
      float a8[8], k8[8], q8[8], b8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        k8[j] = raw8_at(kr[ks], j);
        q8[j] = raw8_at(qr[ks], j);
        if constexpr (AM != 0) a8[j] = av[ks][j];
        else a8[j] = ar[ks][j];
        if constexpr (VEC) b8[j] = br[ks][j];
        else b8[j] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (AM != 0) {
          k8[j] *= rk;
          q8[j] *= rq;
          if constexpr (VEC) b8[j] = gate(b8[j]);
        } else {
          a8[j] = unit_a ? 1.f : a8[j];
        }
        k8[j] = live ? k8[j] : 0.f;
        q8[j] = live ? q8[j] : 0.f;
        a8[j] = live ? a8[j] : 1.f;
        if constexpr (VEC) b8[j] = live ? b8[j] : 0.f;
        else b8[j] = 0.f;
      }
      float f8[8], kd[8], kgv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) f8[j] = a8[j];
      row_prefix_prod8(f8);
      if (r == 15) {
        store4(&sm.tot[w][ch0], f32x4{f8[0], f8[1], f8[2], f8[3]});
        store4(&sm.tot[w][ch0 + 4], f32x4{f8[4], f8[5], f8[6], f8[7]});
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float f = f8[j];
        const float af = fabsf(f);
        ok = ok && (af >= FAST_LO) && (af <= FAST_HI);
        const float rf = __builtin_amdgcn_rcpf(f);
        uf[ks][j] = (VEC ? b8[j] : esc) * k8[j] * f;
        qf[ks][j] = q8[j] * f;
        kd[j] = k8[j] * rf;
        // k_s . g_s with g_s = t / f_s (replaced below if some |f| is out of range)
        kgv[j] = k8[j] * (dpp_or<ROW_BCAST15>(0.f, f) * rf);
      }
      const Frag KD = Pol::make(kd);
      Pol::mma(ad, Pol::make(uf[ks]), KD);
      Pol::mma(pd, Pol::make(qf[ks]), KD);
      store4(&sm.u2.kg[row][ch0], f32x4{kgv[0], kgv[1], kgv[2], kgv[3]});
      store4(&sm.u2.kg[row][ch0 + 4], f32x4{kgv[4], kgv[5], kgv[6], kgv[7]});
    }
    if (__all(ok)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 4 * g + i;  // row within the block; r is the column
        sm.A[16 * w + rr][16 * w + r] = (r < rr) ? ad[i] : 0.f;
        sm.u1.P[16 * w + rr][16 * w + r] = (r <= rr) ? pd[i] : 0.f;
      }
    } else {
      // Some gate of this block is zero or nearly so: exact block path (out of line).
      exact_block<DKR, DK, InT, VEC, AM, ACT>(p, sm, thq, thk, qo, ko, unit_a, valid, esc, rq, rk, w, r, g);
    }
  }
  wave_lds_sync();
  // (I + A_ww)^-1 by forward substitution, one lane per column
  if (l < 16) {
    float t[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      float ar[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) load4(&sm.A[16 * w + rr][16 * w + 4 * q4], *reinterpret_cast<float(*)[4]>(&ar[4 * q4]));
      float acc = (rr == l) ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < rr; ++s) acc = fmaf(-ar[s], t[s], acc);
      t[rr] = acc;
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) sm.Td[w][rr][l] = t[rr];
  }
  __syncthreads();

  // ---------------------------------------------------------------- off-diagonal tiles, Utilde, Qtilde
  {
    f32x4 accA[NBLK - 1], accP[NBLK - 1];
#pragma unroll
    for (int J = 0; J < NBLK - 1; ++J) { accA[J] = f32x4{0.f, 0.f, 0.f, 0.f}; accP[J] = accA[J]; }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch0 = 32 * ks + 8 * g;
      // mid[J] = prod_{J<J'<w} t_J', run = prod_{J<w} t_J (Gamma at the block start)
      float run[8], mid[NBLK - 1][8];
#pragma unroll
      for (int j = 0; j < 8; ++j) run[j] = 1.f;
#pragma unroll
      for (int J = NBLK - 2; J >= 0; --J) {
        if (J < w) {
#pragma unroll
          for (int j = 0; j < 8; ++j) mid[J][j] = run[j];
          float t8[8];
          load8(&sm.tot[J][ch0], t8);
#pragma unroll
          for (int j = 0; j < 8; ++j) run[j] *= t8[j];
        }
      }
      const Frag UF = Pol::make(uf[ks]);
      const Frag QF = Pol::make(qf[ks]);
#pragma unroll
      for (int J = 0; J < NBLK - 1; ++J) {
        if (J < w) {
          float x[8];
          load8(&sm.u2.kg[16 * J + r][ch0], x);
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] *= mid[J][j];
          const Frag B = Pol::make(x);
          Pol::mma(accA[J], UF, B);
          Pol::mma(accP[J], QF, B);
        }
      }
      float ut[8], qt[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) { ut[j] = uf[ks][j] * run[j]; qt[j] = qf[ks][j] * run[j]; }
      st_frag(rs, R::UT, wu * KS + ks, l, Pol::make(ut), p.rec_nt);
      // Qtilde and P serve the output only: a call without output (states and snapshots only)
      // leaves them out of the record, and its state pass does not read them
      if (p.o) st_frag(rs, R::QT, wu * KS + ks, l, Pol::make(qt), p.rec_nt);
    }
#pragma unroll
    for (int J = 0; J < NBLK - 1; ++J) {
      if (J < w) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sm.A[16 * w + 4 * g + i][16 * J + r] = accA[J][i];
          sm.u1.P[16 * w + 4 * g + i][16 * J + r] = accP[J][i];
        }
      }
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- P, Kbar^T and Gamma_C out
  // (rows of blocks 0 and 1 are zero in tokens 32..63: that step is never read, nor written)
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    if (p.o && (st == 0 || w >= 2)) {
      float a8[8];
      load8(&sm.u1.P[16 * w + r][32 * st + 8 * g], a8);
      st_frag(rs, R::PP, wu * 2 + st, l, Pol::make(a8), p.rec_nt);
    }
  }
  for (int rt = wu; rt < DK / 16; rt += 4) {
    const int chA = 16 * rt + r;
    float tA[NBLK];
#pragma unroll
    for (int J = 0; J < NBLK; ++J) tA[J] = sm.tot[J][chA];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int k0 = 32 * st + 8 * g;
      const int blk = 2 * st + (g >> 1);
      float suf = 1.f;
#pragma unroll
      for (int J = 1; J < NBLK; ++J) suf *= (J > blk) ? tA[J] : 1.f;
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = sm.u2.kg[k0 + j][chA] * suf;
      st_frag(rs, R::KB, rt * 2 + st, l, Pol::make(x), p.rec_nt);
    }
  }
  if (tid < DK) {
    reinterpret_cast<float*>(rec + R::GC)[tid] = sm.tot[0][tid] * sm.tot[1][tid] * sm.tot[2][tid] * sm.tot[3][tid];
  }
  __syncthreads();

  // ---------------------------------------------------------------- T = (I + A)^-1
  for (int i = tid; i < CH * LDT; i += 256) {
    const int rr = i / LDT, cc = i % LDT;
    (&sm.u2.T[0][0])[i] = (cc < CH && (rr >> 4) == (cc >> 4)) ? sm.Td[rr >> 4][rr & 15][cc & 15] : 0.f;
  }
  {  // At_IK = T_II A_IK (K < I)
    float x[8];
    if (g < 2) {
      load8(&sm.Td[w][r][8 * g], x);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = 0.f;
    }
    const Frag Tii = Pol::make(x);
#pragma unroll
    for (int K = 0; K < NBLK - 1; ++K) {
      if (K < w) {
        float y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = (g < 2) ? sm.A[16 * w + 8 * g + j][16 * K + r] : 0.f;
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        Pol::mma(acc, Tii, Pol::make(y));
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.u1.At[16 * w + 4 * g + i][16 * K + r] = acc[i];
      }
    }
  }
  __syncthreads();
  // T_IJ = -sum_{K=J..I-1} At_IK T_KJ, by increasing distance I - J
#pragma unroll
  for (int d = 1; d < NBLK; ++d) {
    if (w >= d) {
      const int J = w - d;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if (st < (d + 1) / 2) {
          const int k0 = 16 * J + 32 * st + 8 * g;
          float a8[8], b8[8];
          if (k0 < 16 * w) {
            load8(&sm.u1.At[16 * w + r][k0], a8);
#pragma unroll
            for (int j = 0; j < 8; ++j) b8[j] = sm.u2.T[k0 + j][16 * J + r];
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) { a8[j] = 0.f; b8[j] = 0.f; }
          }
          Pol::mma(acc, Pol::make(a8), Pol::make(b8));
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.u2.T[16 * w + 4 * g + i][16 * J + r] = -acc[i];
    }
    __syncthreads();
  }
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    if (st == 0 || w >= 2) {
      float a8[8];
      load8(&sm.u2.T[16 * w + r][32 * st + 8 * g], a8);
      st_frag(rs, R::TT, wu * 2 + st, l, Pol::make(a8), p.rec_nt);
    }
  }
}

// ============================================================================ host
template <int DKR, typename InT, bool VEC>
static hipError_t launch_window_t(Params p, const PrefillPlan& pl, int64_t wi, hipStream_t s);

template <int DKR, typename InT, bool VEC>
static hipError_t launch_t(const Params& p0, const PrefillPlan& pl, hipStream_t s) {
  if (p0.cu) {
    hipLaunchKernelGGL(chunk_plan_kernel, dim3(1), dim3(256), 0, s, p0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  Params p = p0;
  if (p.cu) p.cu = p.cu_ok;  // every later pass reads the plan's clamped offsets
  for (int64_t wi = 0; wi < pl.windows; ++wi) {
    const hipError_t e = launch_window_t<DKR, InT, VEC>(p, pl, wi, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// One window: the chunk preparation of its chunks, then the state pass over them.
template <int DKR, typename InT, bool VEC>
static hipError_t launch_window_t(Params p, const PrefillPlan& pl, int64_t wi, hipStream_t s) {
  const bool prep = p.prep_l2 || p.a_bf16 || p.a_act || p.g_act;
  int64_t prep_slots = pl.slots;
  if (!p.cu) {
    const int64_t cps = p.cps;
    p.win_c0 = (int32_t)(wi * pl.win_k);
    p.win_nc = (int32_t)(cps - p.win_c0 < pl.win_k ? cps - p.win_c0 : pl.win_k);
    p.win_k = (int32_t)pl.win_k;
    p.carry_in = wi > 0;
    p.carry_out = wi + 1 < pl.windows;
    prep_slots = pl.win_k > 0 ? (pl.slots / pl.win_k) * p.win_nc : 0;  // batch rows x this window's chunks
  }
  if (prep_slots > 0) {
    const dim3 grid((unsigned)(prep_slots * p.H));
    // the decay's storage type and activation are template arguments: each instance evaluates
    // only its own activation
    if (!prep)
      hipLaunchKernelGGL((chunk_prep_kernel<DKR, InT, VEC, 0, 0>), grid, dim3(256), 0, s, p);
    else if (!p.a_bf16 && p.a_act == 1)
      hipLaunchKernelGGL((chunk_prep_kernel<DKR, InT, VEC, 1, 1>), grid, dim3(256), 0, s, p);
    else if (!p.a_bf16 && p.a_act == 2)
      hipLaunchKernelGGL((chunk_prep_kernel<DKR, InT, VEC, 1, 2>), grid, dim3(256), 0, s, p);
    else if (!p.a_bf16)
      hipLaunchKernelGGL((chunk_prep_kernel<DKR, InT, VEC, 1, 0>), grid, dim3(256), 0, s, p);
    else if (p.a_act == 1)
      hipLaunchKernelGGL((chunk_prep_kernel<DKR, InT, VEC, 2, 1>), grid, dim3(256), 0, s, p);
    else if (p.a_act == 2)
      hipLaunchKernelGGL((chunk_prep_kernel<DKR, InT, VEC, 2, 2>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((chunk_prep_kernel<DKR, InT, VEC, 2, 0>), grid, dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_state_pass(p, pl.workgroups, DKR, pl.dv_block, std::is_same<InT, __bf16>::value, VEC, s);
}

template <int DKR>
static hipError_t launch_dk(const Params& p, const PrefillPlan& pl, bool bf16, bool vec, hipStream_t s) {
  if (bf16) return vec ? launch_t<DKR, __bf16, true>(p, pl, s) : launch_t<DKR, __bf16, false>(p, pl, s);
  return vec ? launch_t<DKR, float, true>(p, pl, s) : launch_t<DKR, float, false>(p, pl, s);
}

// Workspace pointers of a call: the records, then (packed sequences) the plan's tables.
static void set_workspace(Params& p, const PrefillPlan& pl, void* ws) {
  p.rec = static_cast<unsigned char*>(ws);
  p.rec_size = pl.rec_size;
  p.slots = (int32_t)pl.slots;
  p.cps = (int32_t)((p.T + CH - 1) / CH);
  p.win_c0 = 0;
  p.win_nc = p.cps;
  p.win_k = (int32_t)pl.win_k;
  p.carry = prefill_carry(ws, pl, p.H);
  p.carry_in = p.carry_out = 0;
  // Records of a window larger than the 256 MB Infinity Cache come back from HBM whatever the
  // store policy: non-temporal stores then make the call faster (KDA prefill, 4 x 4096 tokens x
  // 16 heads: 0.393 -> 0.381 ms per call). Smaller records, and windows sized for the cache, keep
  // the default policy, under which they are still cached when read.
  p.rec_nt = (pl.slots * p.H * pl.rec_size > ((int64_t)256 << 20)) ? 1 : 0;
  if (p.cu) {
    int32_t* tables = reinterpret_cast<int32_t*>(p.rec + pl.slots * p.H * pl.rec_size);
    p.chunk_seq = tables;
    p.chunk_c0 = tables + pl.slots;
    p.seq_first = tables + 2 * pl.slots;
    p.snap_first = prefill_snap_first(ws, pl, p.H, p.nseq);
    p.seq_order = p.snap_first + p.nseq;
    p.cu_ok = prefill_cu_table(ws, pl, p.H, p.nseq);
  }
}

hipError_t launch_plan_only(Params p, const PrefillPlan& pl, void* ws, hipStream_t s) {
  if (!p.cu || pl.workgroups == 0) return hipSuccess;
  set_workspace(p, pl, ws);
  hipLaunchKernelGGL(chunk_plan_kernel, dim3(1), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_prefill(Params p, const PrefillPlan& pl, void* ws, int dk, bool bf16, bool vec,
                          hipStream_t s) {
  if (pl.workgroups == 0) return hipSuccess;
  set_workspace(p, pl, ws);
  switch (dk) {
    case 16: return launch_dk<16>(p, pl, bf16, vec, s);
    case 32: return launch_dk<32>(p, pl, bf16, vec, s);
    case 64: return launch_dk<64>(p, pl, bf16, vec, s);
    case 128: return launch_dk<128>(p, pl, bf16, vec, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dr
