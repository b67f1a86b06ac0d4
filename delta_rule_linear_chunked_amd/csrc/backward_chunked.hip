// Chunked backward of the gated delta-rule prefill on gfx950: the gradients of a prefill with one
// transition per token (fixed-length or packed sequences), in three MFMA passes after the
// checkpointing forward (the course page "GDN, KDA và Mamba-2 · cập nhật state trong hybrid",
// section 3: training keeps checkpoints and the chunked form's intermediates).
//
// Inside a chunk with start state S0, end-state gradient dS (the gradient reaching the state
// after the chunk's last token from later tokens) and output gradient dO, with Gamma_r the
// running product of the decays and the chunk algebra of prefill.hip (T = (I + A)^-1,
// Utilde = Gamma . u, Qtilde = Gamma . q, Kbar_s = Gamma_C / Gamma_s . k_s, P, delta):
//
//   eps    = T^T (P^T dO + Kbar dS)                  the gradient of delta (= dm)
//   dS0    = Diag(Gamma_C) dS + Qtilde^T dO - Utilde^T eps
//          = M dS + N,  M = Diag(Gamma_C) - W^T Kbar,  N = Z^T dO,  W = T Utilde,  Z = Qtilde - P W
//   dQtilde = dO S0^T,  dUtilde = -eps S0^T,  dKbar = delta dS^T,
//   dP = tril(dO delta^T),  dA = -strict_tril(eps delta^T)
//
// and, with the decay ratios written through the chunk's running product (Kd_s = k_s / Gamma_s),
//   dq = Gamma . (dQtilde + dP Kd),  du = Gamma . (dUtilde + dA Kd),
//   dk (as the key) = (Gamma_C . dKbar + dP^T Qtilde + dA^T Utilde) / Gamma.
// Every decay product in a chunk runs over a token range, and alpha_t times its derivative is that
// product, so alpha_t dL/dalpha_t (per channel) is the reverse cumulative sum over the chunk of
// q . dq + u . du - k . dk plus the end state's term rowsum(dS . S_C); dividing by alpha_t gives
// the gate gradient.
//
// The divisions by Gamma_s and by alpha_t are what limit this form. A gate of magnitude below 2^-4
// takes its gate gradient from an exact inner product instead (up to 12 such gates per chunk);
// a chunk with more of them, a zero or non-finite gate, or a running product outside
// [2^-110, 2^100] raises a flag, and the whole call then takes the exact per-token reverse walk
// (backward.hip), which divides by nothing. (KDA, RDA and GDN-2 decays exp(-c softplus(z)) close
// to 1 never raise it; Complex KDA gates, a few percent of them near zero, do.)
//
// Passes (chunks of 64 tokens from each sequence's start; packed sequences take their chunk slots
// from the prefill's plan pass):
//   cbwd_prep_kernel   one workgroup per (chunk, head): M as MFMA operand fragments
//                      and N in fp32 into the chunk's record;
//   cbwd_state_kernel  one workgroup per (sequence, head, 32 value columns): walks the chunks in
//                      reverse with dS in registers, stores dS at every chunk end, dS <- M dS + N;
//   cbwd_grad_kernel   one workgroup per (chunk, head): recomputes the chunk algebra,
//                      loops over 32-column value blocks for delta, eps and the tile gradients,
//                      then forms dq, dk, dv, dalpha and the gate gradients.
#include "prefill.hpp"

namespace dr {

namespace {

// Gates of magnitude below CB_TAU take the exact gate gradient: the cumulative sum's rounding,
// divided by alpha, measured up to 2.5e-5 (split bf16) and 2e-6 (fp32) of the gradient's RMS over
// |alpha| with Complex KDA gates, so below 2^-4 the division would exceed the parity bars' margin.
constexpr float CB_TAU = 0x1p-4f;
constexpr int CB_NE = 12;            // at most this many such (token, channel) entries per chunk
constexpr float CB_LO = 0x1p-110f;   // range of the running products the chunked form takes
constexpr float CB_HI = 0x1p100f;
constexpr int L68 = CH + 4;          // row stride of 64-column fp32 tiles
constexpr int L36 = 36;              // row stride of 32-column fp32 tiles

// Record of one (batch row, chunk, head): M's fragments as A operands (row tiles of output
// channels x 32-deep steps over input channels), then N [d_k][d_v] in fp32.
template <int DK>
struct CRec {
  static constexpr int KS = DK / 32;
  static constexpr int64_t MF = 0;
  static constexpr int64_t NN = (int64_t)(DK / 16) * KS * 2048;
  static int64_t size(int dv) { return (NN + (int64_t)DK * dv * 4 + 255) / 256 * 256; }
};

// LDS of the two per-chunk kernels. r0: Gamma (then, by pass, Utilde / Qtilde / Z, or dP and dA);
// r1: Kd (then dO in the preparation); r2: A, At, P, T of the chunk algebra, then the value-block
// buffers of the gradient kernel, then Qtilde / Utilde and the gate-gradient sums, or W and M in the
// preparation.
template <int DK>
struct CbSmem {
  static constexpr int LG = DK + 4;
  static constexpr int R0 = (CH * LG > 2 * CH * L68) ? CH * LG : 2 * CH * L68;
  static constexpr int R1 = CH * (128 + 4);
  static constexpr int RB = 2 * DK * L36 + 3 * CH * L36 + 2 * 32 * L68;  // value-block buffers
  static constexpr int RM = DK * LG;                                   // M in the preparation
  static constexpr int R2a = RB > 4 * CH * L68 ? RB : 4 * CH * L68;
  static constexpr int R2b = 2 * CH * LG > RM ? 2 * CH * LG : RM;
  static constexpr int R2 = R2a > R2b ? R2a : R2b;
  float r0[R0];
  float r1[R1];
  float r2[R2];
  float gc[DK];     // Gamma_C
  float ddp[512];   // per-thread partial sums of rowsum(S0 . dS)
  float ecs[4][DK]; // per-row-block column sums of Kbar . dKbar
  float red[2][2][CH];  // per-half token sums: k . du, v . dm
  // gates of magnitude below CB_TAU: their count, (token, channel), and for the gradient kernel
  // Qtilde and Utilde down the entry's channel and the entry's inner product
  int ne;
  int ent[CB_NE];
  float eq[CB_NE][CH], eu[CB_NE][CH];
  float eacc[CB_NE];
};
// offsets in r2 during the chunk algebra
constexpr int OA = 0, OAT = CH * L68, OP = 2 * CH * L68, OT = 3 * CH * L68;

template <class Pol>
__device__ __forceinline__ typename Pol::Frag frag_c(const float* p) {
  float x[8];
  load8(p, x);
  return Pol::make(x);
}
template <class Pol>
__device__ __forceinline__ typename Pol::Frag frag_s(const float* p, int stride) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = p[j * stride];
  return Pol::make(x);
}

// Step m of batch row b (fixed length; packed sequences: b = 0 and m the absolute step), head h:
// its row in the per-token arrays (q, alpha, dO, dq, dalpha) and in the per-step arrays (k, v, the
// gates and their gradients), and whether it is a token's first or last step. With one transition
// per token both rows are (b T + m) H + h; with two (lgnh = 1) a token's steps are consecutive.
__device__ __forceinline__ int64_t cb_tok(const CbParams& p, int b, int64_t m, int h) {
  return ((((int64_t)b * p.T + m) >> p.lgnh) * p.H + h);
}
__device__ __forceinline__ int64_t cb_step(const CbParams& p, int b, int64_t m, int h) {
  const int64_t a = (int64_t)b * p.T + m;
  return ((((a >> p.lgnh) * p.H + h) << p.lgnh) + (a & ((1 << p.lgnh) - 1)));
}
__device__ __forceinline__ bool cb_first(const CbParams& p, int64_t m) { return (m & ((1 << p.lgnh) - 1)) == 0; }
__device__ __forceinline__ bool cb_last(const CbParams& p, int64_t m) {
  return (m & ((1 << p.lgnh) - 1)) == (1 << p.lgnh) - 1;
}

// The chunk algebra shared by the preparation and the gradient kernel (the chunk's rows are tokens
// m0 .. m0 + 63 of batch row b): Gamma in r0, Kd in r1,
// A, P and T in r2, Gamma_C in gc; ut / qt receive this thread's row of Utilde / Qtilde (token
// 16 w + lane % 16, channels 32 ks + 8 (lane / 16) + j). With set_flag, a chunk outside the
// chunked form's range sets *p.flag.
template <int DK, typename InT, bool VEC>
__device__ __forceinline__ void chunk_algebra(const CbParams& p, CbSmem<DK>& sm, int b, int64_t m0, int h, int nvalid,
                                              float (&ut)[DK / 32][8], float (&qt)[DK / 32][8], bool set_flag) {
  using Pol = typename PolicyFor<InT>::type;
  using Frag = typename Pol::Frag;
  constexpr int KS = DK / 32, LG = CbSmem<DK>::LG;
  // (with 512 threads, waves w and w + 4 share row block w; the second half only builds its ut / qt)
  const int tid = threadIdx.x, w = (tid >> 6) & 3, hf = tid >> 8, l = tid & 63, r = l & 15, g = l >> 4;

  // This thread's row of q, k (and the erase gates) is loaded first, so that these loads are in
  // flight while Gamma is formed: every lane loads (rows past the sequence end read the chunk's
  // first row) and the values are selected where used. Loads under that condition were each
  // waited for inside it, one slice after the other.
  const int row = 16 * w + r;
  const bool valid = row < nvalid;
  const int64_t mrow = m0 + (valid ? row : 0);
  const int64_t th = cb_step(p, b, mrow, h);
  const int64_t qo = q_elem(p, b, mrow, h, DK), ko = kv_elem(p.k_ts, p.k_bs, p, b, mrow, h, DK);
  typename Raw8Of<InT>::type qr[KS], kr[KS];
  float br[VEC ? KS : 1][8];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int ch0 = 32 * ks + 8 * g;
    ld_raw8(static_cast<const InT*>(p.q) + qo + ch0, qr[ks]);
    ld_raw8(static_cast<const InT*>(p.k) + ko + ch0, kr[ks]);
    if constexpr (VEC) load8(p.erase + th * DK + ch0, br[ks]);
  }
  const float esr = VEC ? 0.f : p.erase[th];

  // Gamma: running products down the chunk per channel (tokens past the sequence end take decay
  // 1), in segments of SEG tokens: every thread loads its segment, multiplies it out, and the
  // segments' totals are chained through LDS. Gates of magnitude below CB_TAU are listed.
  if (tid == 0) sm.ne = 0;
  __syncthreads();
  {
    constexpr int NSEG = 4, SEG = CH / NSEG;
    const int nthr = blockDim.x;
    for (int it = tid; it < DK * NSEG; it += nthr) {
      const int ch = it % DK, sg = it / DK;
      float a[SEG];
#pragma unroll
      for (int t = 0; t < SEG; ++t) {
        const int tt = sg * SEG + t;
        a[t] = tt < nvalid && cb_first(p, m0 + tt) ? p.alpha[cb_tok(p, b, m0 + tt, h) * DK + ch] : 1.f;
      }
      float gm = 1.f;
      bool bad = false;
#pragma unroll
      for (int t = 0; t < SEG; ++t) {
        const float aa = fabsf(a[t]);
        bad = bad || !(aa > 0.f && aa <= CB_HI);  // zero, not finite (NaN included) or too large
        if (aa < CB_TAU && aa > 0.f) {
          const int e = atomicAdd(&sm.ne, 1);
          if (e < CB_NE) sm.ent[e] = (sg * SEG + t) * DK + ch;
        }
        gm *= a[t];
        sm.r0[(sg * SEG + t) * LG + ch] = gm;
      }
      sm.ddp[sg * DK + ch] = gm;  // the segment's total
      if (set_flag && bad) atomicOr(p.flag, 1);
    }
    __syncthreads();
    for (int it = tid; it < DK * NSEG; it += nthr) {
      const int ch = it % DK, sg = it / DK;
      float pre = 1.f;
      for (int q = 0; q < sg; ++q) pre *= sm.ddp[q * DK + ch];
      bool bad = false;
#pragma unroll
      for (int t = 0; t < SEG; ++t) {
        float* x = &sm.r0[(sg * SEG + t) * LG + ch];
        const float gm = pre * *x;
        bad = bad || !(fabsf(gm) >= CB_LO && fabsf(gm) <= CB_HI);
        *x = gm;
      }
      if (sg == NSEG - 1) sm.gc[ch] = pre * sm.ddp[sg * DK + ch];
      if (set_flag && bad) atomicOr(p.flag, 1);
    }
  }
  __syncthreads();
  if (set_flag && tid == 0 && sm.ne > CB_NE) atomicOr(p.flag, 1);

  // this thread's row: Utilde, Qtilde (registers) and Kd (LDS)
  {
    const float esc = valid ? esr : 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch0 = 32 * ks + 8 * g;
      float q8[8], k8[8], b8[8], g8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        q8[j] = valid ? raw8_at(qr[ks], j) : 0.f;
        k8[j] = valid ? raw8_at(kr[ks], j) : 0.f;
        if constexpr (VEC) b8[j] = valid ? br[ks][j] : 0.f;
        else b8[j] = 0.f;
      }
      load8(&sm.r0[row * LG + ch0], g8);
      float kd[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        qt[ks][j] = q8[j] * g8[j];
        ut[ks][j] = (VEC ? b8[j] : esc) * k8[j] * g8[j];
        kd[j] = k8[j] * __builtin_amdgcn_rcpf(g8[j]);  // Gamma lies in [2^-110, 2^100] here
      }
      if (hf == 0) {
        store4(&sm.r1[row * LG + ch0], f32x4{kd[0], kd[1], kd[2], kd[3]});
        store4(&sm.r1[row * LG + ch0 + 4], f32x4{kd[4], kd[5], kd[6], kd[7]});
      }
    }
  }
  __syncthreads();

  // A = strict_tril(Utilde Kd^T), P = tril(Qtilde Kd^T) for row block w; T zeroed in row block w
  if (hf == 0) {
    f32x4 accA[NBLK], accP[NBLK];
#pragma unroll
    for (int J = 0; J < NBLK; ++J) { accA[J] = f32x4{0.f, 0.f, 0.f, 0.f}; accP[J] = accA[J]; }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const Frag UF = Pol::make(ut[ks]);
      const Frag QF = Pol::make(qt[ks]);
#pragma unroll
      for (int J = 0; J < NBLK; ++J) {
        if (J <= w) {
          const Frag KF = frag_c<Pol>(&sm.r1[(16 * J + r) * LG + 32 * ks + 8 * g]);
          Pol::mma(accA[J], UF, KF);
          Pol::mma(accP[J], QF, KF);
        }
      }
    }
#pragma unroll
    for (int J = 0; J < NBLK; ++J) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * w + 4 * g + i, col = 16 * J + r;
        sm.r2[OA + row * L68 + col] = (J <= w && col < row) ? accA[J][i] : 0.f;
        sm.r2[OP + row * L68 + col] = (J <= w && col <= row) ? accP[J][i] : 0.f;
        sm.r2[OT + row * L68 + col] = 0.f;
      }
    }
  }
  __syncthreads();
  float* A = sm.r2 + OA;
  float* At = sm.r2 + OAT;
  float* Tm = sm.r2 + OT;
  // diagonal blocks of T = (I + A)^-1 by forward substitution, one lane per column of block w
  if (hf == 0 && l < 16) {
    float t[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      float acc = (rr == l) ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < rr; ++s) acc = fmaf(-A[(16 * w + rr) * L68 + 16 * w + s], t[s], acc);
      t[rr] = acc;
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) Tm[(16 * w + rr) * L68 + 16 * w + l] = t[rr];
  }
  __syncthreads();
  // At_wK = T_ww A_wK for K < w (16-deep products, the upper half of the 32-deep slice zero)
  if (hf == 0) {
    float x[8];
    if (g < 2) {
      load8(&Tm[(16 * w + r) * L68 + 16 * w + 8 * g], x);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = 0.f;
    }
    const Frag Tww = Pol::make(x);
#pragma unroll
    for (int K = 0; K < NBLK - 1; ++K) {
      if (K < w) {
        float y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = g < 2 ? A[(16 * w + 8 * g + j) * L68 + 16 * K + r] : 0.f;
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        Pol::mma(acc, Tww, Pol::make(y));
#pragma unroll
        for (int i = 0; i < 4; ++i) At[(16 * w + 4 * g + i) * L68 + 16 * K + r] = acc[i];
      }
    }
  }
  __syncthreads();
  // T_wJ = -sum_{K = J}^{w - 1} At_wK T_KJ, by increasing distance d = w - J
#pragma unroll
  for (int d = 1; d < NBLK; ++d) {
    if (hf == 0 && w >= d) {
      const int J = w - d;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if (st < (d + 1) / 2) {
          const int k0 = 16 * J + 32 * st + 8 * g;
          float a8[8], b8[8];
          if (k0 < 16 * w) {
            load8(&At[(16 * w + r) * L68 + k0], a8);
#pragma unroll
            for (int j = 0; j < 8; ++j) b8[j] = Tm[(k0 + j) * L68 + 16 * J + r];
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) { a8[j] = 0.f; b8[j] = 0.f; }
          }
          Pol::mma(acc, Pol::make(a8), Pol::make(b8));
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) Tm[(16 * w + 4 * g + i) * L68 + 16 * J + r] = -acc[i];
    }
    __syncthreads();
  }
}

// The chunk a workgroup of the per-chunk kernels takes (blockIdx.x = chunk slot * H + head): its
// sequence n and chunk index c within it, the batch row b and first token m0 through which its
// rows are addressed, and its valid tokens. False for an unused slot of packed sequences.
struct CbChunk {
  int n, c, h, b, nvalid;
  int64_t m0;
};
__device__ __forceinline__ bool cb_chunk(const CbParams& p, CbChunk& k) {
  const int slot = blockIdx.x / p.H;
  k.h = blockIdx.x % p.H;
  if (p.cu) {
    k.n = p.chunk_seq[slot];
    if (k.n < 0) return false;
    const int64_t bos = (int64_t)p.cu[k.n] << p.lgnh, len = ((int64_t)p.cu[k.n + 1] << p.lgnh) - bos;
    const int64_t c0 = p.chunk_c0[slot];
    k.c = (int)(c0 / CH);
    k.b = 0;
    k.m0 = bos + c0;
    k.nvalid = len - c0 < CH ? (int)(len - c0) : CH;
  } else {
    k.n = slot / p.nc;
    k.c = slot % p.nc;
    k.b = k.n;
    k.m0 = (int64_t)k.c * CH;
    const int64_t left = p.T - k.m0;
    k.nvalid = left < CH ? (int)left : CH;
  }
  return true;
}

// State at the start of chunk k (null: zero): the initial state, or the forward's snapshot after
// the previous chunk.
__device__ __forceinline__ const float* cb_start_state(const CbParams& p, const CbChunk& k, int64_t SS) {
  if (k.c == 0) return p.S0 ? p.S0 + ((int64_t)k.n * p.H + k.h) * SS : nullptr;
  const int64_t row = (p.cu ? (int64_t)p.snap_first[k.n] : (int64_t)k.n * (p.T / CH)) + k.c - 1;
  return p.snap + (row * p.H + k.h) * SS;
}

}  // namespace

// The entries' <L, R> over one value block's columns, for wave w8's entries w8, w8 + 8, ...: lane
// (c, half) takes column c and every second token of the sums, the halves meet by a lane swap.
// Out of line, so that the gradient kernel's registers are not sized for it on the path without
// such entries.
template <int DK>
__device__ __attribute__((noinline)) void cb_entries(CbSmem<DK>& sm, int ne, int w8, int l, const float* S0b,
                                                      const float* dSb, const float* dOb, const float* Dl,
                                                      const float* El) {
  constexpr int LG = CbSmem<DK>::LG;
  for (int e = w8; e < ne; e += 8) {
    const int te = sm.ent[e] / DK, ie = sm.ent[e] % DK, c = l & 31, hv = l >> 5;
    float Lv = hv == 0 ? S0b[ie * L36 + c] : 0.f;
    for (int s2 = hv; s2 < te; s2 += 2) Lv = fmaf(sm.r1[s2 * LG + ie], Dl[s2 * L36 + c], Lv);
    float Rv = hv == 0 ? sm.gc[ie] * dSb[ie * L36 + c] : 0.f;
    for (int r2 = te + ((te ^ hv) & 1); r2 < CH; r2 += 2)
      Rv = fmaf(sm.eq[e][r2], dOb[r2 * L36 + c], fmaf(-sm.eu[e][r2], El[r2 * L36 + c], Rv));
    Lv += __shfl_xor(Lv, 32);
    Rv += __shfl_xor(Rv, 32);
    float prod = hv == 0 ? Lv * Rv : 0.f;
#pragma unroll
    for (int d = 1; d < 32; d <<= 1) prod += __shfl_xor(prod, d);
    if (l == 0) sm.eacc[e] += prod;
  }
}

// ============================================================================ pass 1
__global__ void cbwd_flag_clear_kernel(int32_t* flag) {
  if (threadIdx.x == 0) *flag = 0;
}

// Eight waves: waves w and w + 4 share row block w of the 64-token products (W, Z) and take half of
// the channel tiles each; in the products over channels (M, N) wave v takes output-channel tile
// v % (d_k / 16) and, for d_k = 64, every second column tile.
template <int DK, typename InT, bool VEC>
__global__ __launch_bounds__(512, 1) void cbwd_prep_kernel(const CbParams p) {
  using Pol = typename PolicyFor<InT>::type;
  using Frag = typename Pol::Frag;
  constexpr int KS = DK / 32, LG = CbSmem<DK>::LG, NCT = DK / 16, NCH = NCT / 2;
  constexpr int RT = DK / 16, WPR = 8 / RT;  // output-channel tiles; waves per tile
  using R = CRec<DK>;
  __shared__ __align__(16) CbSmem<DK> sm;
  CbChunk ck;
  if (!cb_chunk(p, ck)) return;
  const int b = ck.b, h = ck.h, nvalid = ck.nvalid;
  const int64_t m0 = ck.m0;
  const int tid = threadIdx.x, w8 = tid >> 6, w = w8 & 3, hf = w8 >> 2, l = tid & 63, r = l & 15, g = l >> 4;
  const int rt = w8 % RT, part = w8 / RT;
  float ut[KS][8], qt[KS][8];
  chunk_algebra<DK, InT, VEC>(p, sm, b, m0, h, nvalid, ut, qt, true);
  // dO of the chunk (zero past the sequence end), loaded here so that its latency overlaps W, Z
  // and M, and put in LDS once M is done with Kd: DV / 32 16-byte pieces per thread (d_v <= 128).
  // Every load is issued, pieces that do not count reading the chunk's first row, and zeroed at
  // the store: loads under a condition each got a wait for their data right behind them.
  const int DV = p.DV, LV = DV + 4, NQ = DV / 32;
  f32x4 dOr[4];
  unsigned dOk = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = tid + 512 * k, t = idx / (DV / 4), v4 = idx % (DV / 4);
    const bool ok = k < NQ && t < nvalid && cb_last(p, m0 + t);
    dOk |= ok ? 1u << k : 0u;
    dOr[k] = *reinterpret_cast<const f32x4*>(p.dO + cb_tok(p, b, m0 + (ok ? t : 0), h) * DV + 4 * (ok ? v4 : 0));
  }
  const float* Tm = sm.r2 + OT;
  const float* Pm = sm.r2 + OP;
  float* Wm = sm.r2;  // W over A and At (no longer read)

  // Utilde -> r0 (Gamma is not read past the chunk algebra)
  auto put_rows = [&](const float (&x)[KS][8]) {
    if (hf == 0) {
      const int row = 16 * w + r;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int ch0 = 32 * ks + 8 * g;
        store4(&sm.r0[row * LG + ch0], f32x4{x[ks][0], x[ks][1], x[ks][2], x[ks][3]});
        store4(&sm.r0[row * LG + ch0 + 4], f32x4{x[ks][4], x[ks][5], x[ks][6], x[ks][7]});
      }
    }
  };
  put_rows(ut);
  __syncthreads();
  // W = T Utilde, row block w, this half's channel tiles
  {
    f32x4 acc[NCH];
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) acc[cc] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      if (st == 0 || w >= 2) {
        const Frag TF = frag_c<Pol>(&Tm[(16 * w + r) * L68 + 32 * st + 8 * g]);
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc)
          Pol::mma(acc[cc], TF, frag_s<Pol>(&sm.r0[(32 * st + 8 * g) * LG + 16 * (hf * NCH + cc) + r], LG));
      }
    }
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
#pragma unroll
      for (int i = 0; i < 4; ++i) Wm[(16 * w + 4 * g + i) * LG + 16 * (hf * NCH + cc) + r] = acc[cc][i];
    }
  }
  __syncthreads();
  // Qtilde -> r0, then Z = Qtilde - P W in place (row block w, this half's channel tiles)
  put_rows(qt);
  __syncthreads();
  {
    f32x4 acc[NCH];
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) acc[cc] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      if (st == 0 || w >= 2) {
        const Frag PF = frag_c<Pol>(&Pm[(16 * w + r) * L68 + 32 * st + 8 * g]);
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc)
          Pol::mma(acc[cc], PF, frag_s<Pol>(&Wm[(32 * st + 8 * g) * LG + 16 * (hf * NCH + cc) + r], LG));
      }
    }
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float* z = &sm.r0[(16 * w + 4 * g + i) * LG + 16 * (hf * NCH + cc) + r];
        *z = *z - acc[cc][i];
      }
    }
  }
  __syncthreads();
  // M = Diag(Gamma_C) - W^T Kbar: output-channel tile rt, column tiles part, part + WPR, ...
  {
    constexpr int NM = NCT / WPR;
    f32x4 acc[NM];
#pragma unroll
    for (int u = 0; u < NM; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const Frag AF = frag_s<Pol>(&Wm[(32 * st + 8 * g) * LG + 16 * rt + r], LG);
#pragma unroll
      for (int u = 0; u < NM; ++u) {
        const int ct = part + WPR * u;
        const float gcc = sm.gc[16 * ct + r];
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = sm.r1[(32 * st + 8 * g + j) * LG + 16 * ct + r] * gcc;
        Pol::mma(acc[u], AF, Pol::make(x));
      }
    }
    __syncthreads();  // W and Kd read by every wave
    float* Mm = sm.r2;
#pragma unroll
    for (int u = 0; u < NM; ++u) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra = 16 * rt + 4 * g + i, cb = 16 * (part + WPR * u) + r;
        Mm[ra * LG + cb] = (ra == cb ? sm.gc[cb] : 0.f) - acc[u][i];
      }
    }
  }
  // dO -> r1 [64][d_v + 4]
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = tid + 512 * k;
    if (k < NQ)
      store4(&sm.r1[(idx / (DV / 4)) * LV + 4 * (idx % (DV / 4))], (dOk >> k) & 1u ? dOr[k] : f32x4{0.f, 0.f, 0.f, 0.f});
  }
  __syncthreads();
  const int64_t slot = blockIdx.x;
  unsigned char* rec = p.rec + slot * p.rec_size;
  const __amdgpu_buffer_rsrc_t rs = rec_rsrc(rec, p.rec_size);
  // M's fragments: row tile rt, step kb: row 16 rt + lane % 16, columns 32 kb + 8 (lane / 16) + j
  if (part == 0) {
#pragma unroll
    for (int kb = 0; kb < KS; ++kb) {
      float x[8];
      load8(&sm.r2[(16 * rt + r) * LG + 32 * kb + 8 * g], x);
      st_frag(rs, (int)R::MF, rt * KS + kb, l, Pol::make(x), true);
    }
  }
  // N = Z^T dO: output-channel tile rt, column tiles part, part + WPR, ..., stored row-major in fp32
  float* Nrec = reinterpret_cast<float*>(rec + R::NN);
  const int NV = DV / 16;
  Frag AZ[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) AZ[st] = frag_s<Pol>(&sm.r0[(32 * st + 8 * g) * LG + 16 * rt + r], LG);
  for (int ct0 = part; ct0 < NV; ct0 += 4 * WPR) {
    f32x4 acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int ct = ct0 + WPR * u;
        if (ct < NV) Pol::mma(acc[u], AZ[st], frag_s<Pol>(&sm.r1[(32 * st + 8 * g) * LV + 16 * ct + r], LV));
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ct = ct0 + WPR * u;
      if (ct < NV) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __builtin_nontemporal_store(acc[u][i], &Nrec[(16 * rt + 4 * g + i) * DV + 16 * ct + r]);
      }
    }
  }
}

// ============================================================================ pass 2
// dS, transposed ([value column][channel]), as split MFMA B operands: hi / lo bf16 planes (bf16
// inputs) or fp32, written four channels at a time from the accumulators
template <class Pol, int DK> struct GTile;
template <int DK> struct GTile<PolBF3, DK> {
  __bf16 hi[32][DK + 8], lo[32][DK + 8];
  __device__ __forceinline__ void put4(int v, int ch, const f32x4& x) {
    uint32_t hh[2], ll[2];
    split2(x[0], x[1], hh[0], ll[0]);
    split2(x[2], x[3], hh[1], ll[1]);
    *reinterpret_cast<bf16x4*>(&hi[v][ch]) = __builtin_bit_cast(bf16x4, hh);
    *reinterpret_cast<bf16x4*>(&lo[v][ch]) = __builtin_bit_cast(bf16x4, ll);
  }
  __device__ __forceinline__ PolBF3::Frag get8(int v, int ch) const {
    PolBF3::Frag f;
    f.hi = *reinterpret_cast<const bf16x8*>(&hi[v][ch]);
    f.lo = *reinterpret_cast<const bf16x8*>(&lo[v][ch]);
    return f;
  }
};
template <int DK> struct GTile<PolF32, DK> {
  float x[32][DK + 4];
  __device__ __forceinline__ void put4(int v, int ch, const f32x4& a) { store4(&x[v][ch], a); }
  __device__ __forceinline__ PolF32::Frag get8(int v, int ch) const {
    PolF32::Frag f;
    load8(&x[v][ch], f.v);
    return f;
  }
};

// dS walks the chunks in reverse, one workgroup per (sequence, head, 32 value columns); wave w
// holds output-channel tiles w + 4 m. The next chunk's M_c fragments and N_c values are loaded a
// chunk ahead, and dS alternates between two LDS tiles, so each chunk takes one barrier.
template <int DK, typename InT>
__global__ __launch_bounds__(256, 1) void cbwd_state_kernel(const CbParams p) {
  using Pol = typename PolicyFor<InT>::type;
  using Frag = typename Pol::Frag;
  constexpr int KS = DK / 32, NRT = DK / 64, NCT = 2, DVB = 32;
  using R = CRec<DK>;
  __shared__ __align__(16) GTile<Pol, DK> Gt[2];
  const int ndvb = p.DV / DVB;
  const int logical = p.nseq * p.H * ndvb;
  const int lid = (gridDim.x % 8 == 0) ? xcd_remap(blockIdx.x, gridDim.x) : blockIdx.x;
  if (lid >= logical) return;
  // (sequence, head) pairs, packed sequences longest first; a pair's value blocks are adjacent
  const int pair = lid / ndvb, dv0 = (lid % ndvb) * DVB;
  const int b = p.cu ? p.seq_order[pair / p.H] : pair / p.H, h = pair % p.H;
  // the sequence's chunk slots: first .. first + nch - 1
  const int first = p.cu ? p.seq_first[b] : b * p.nc;
  const int nch = p.cu ? (int)(((((int64_t)p.cu[b + 1] - p.cu[b]) << p.lgnh) + CH - 1) / CH) : p.nc;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = l & 15, g = l >> 4;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int DV = p.DV;
  const int64_t SS = (int64_t)DK * DV;

  f32x4 G[NRT][NCT];
#pragma unroll
  for (int m = 0; m < NRT; ++m) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ch = 16 * (w + 4 * m) + 4 * g + i;
        G[m][ct][i] = p.dST ? p.dST[((int64_t)b * p.H + h) * SS + (int64_t)ch * DV + dv0 + 16 * ct + r] : 0.f;
      }
    }
  }
  Frag MF[NRT][KS];
  f32x4 NV[NRT][NCT];
  auto load_chunk = [&](int c) {
    const int64_t slot = ((int64_t)first + c) * p.H + h;
    const unsigned char* rec = p.rec + slot * p.rec_size;
    const __amdgpu_buffer_rsrc_t rs = rec_rsrc(rec, p.rec_size);
    const float* Nrec = reinterpret_cast<const float*>(rec + R::NN);
#pragma unroll
    for (int m = 0; m < NRT; ++m) {
#pragma unroll
      for (int kb = 0; kb < KS; ++kb) MF[m][kb] = ld_frag<Frag>(rs, (int)R::MF, (wu + 4 * m) * KS + kb, l);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          NV[m][ct][i] = Nrec[(int64_t)(16 * (w + 4 * m) + 4 * g + i) * DV + dv0 + 16 * ct + r];
      }
    }
  };
  if (nch > 0) load_chunk(nch - 1);
  for (int c = nch - 1; c >= 0; --c) {
    GTile<Pol, DK>& T = Gt[c & 1];
    float* dsc = p.dsc + (((int64_t)first + c) * p.H + h) * SS;
    f32x4 acc[NRT][NCT];
    Frag A[NRT][KS];
#pragma unroll
    for (int m = 0; m < NRT; ++m) {
#pragma unroll
      for (int kb = 0; kb < KS; ++kb) A[m][kb] = MF[m][kb];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        acc[m][ct] = NV[m][ct];
        const int ch0 = 16 * (w + 4 * m) + 4 * g;
        T.put4(16 * ct + r, ch0, G[m][ct]);
#pragma unroll
        for (int i = 0; i < 4; ++i) dsc[(int64_t)(ch0 + i) * DV + dv0 + 16 * ct + r] = G[m][ct][i];
      }
    }
    if (c > 0) load_chunk(c - 1);
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < KS; ++kb) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const Frag BF = T.get8(16 * ct + r, 32 * kb + 8 * g);
#pragma unroll
        for (int m = 0; m < NRT; ++m) Pol::mma(acc[m][ct], A[m][kb], BF);
      }
    }
#pragma unroll
    for (int m = 0; m < NRT; ++m) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) G[m][ct] = acc[m][ct];
    }
  }
  if (p.dS0) {
#pragma unroll
    for (int m = 0; m < NRT; ++m) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ch = 16 * (w + 4 * m) + 4 * g + i;
          p.dS0[((int64_t)b * p.H + h) * SS + (int64_t)ch * DV + dv0 + 16 * ct + r] = G[m][ct][i];
        }
      }
    }
  }
}

// ============================================================================ pass 3
// Eight waves, two per SIMD so that each covers the other's LDS and memory waits. Waves w and w + 4
// share the 16-token row block w and split the products by role: the first half (waves 0-3) those
// with S0 (X = Utilde S0, delta = T R, dQtilde, dUtilde, then dq and du), the second half those with
// dS (Y = Kbar dS + P^T dO, eps = T^T Y, dKbar, dP, dA, then dk).
template <int DK, typename InT, bool VEC>
__global__ __launch_bounds__(512, 1) void cbwd_grad_kernel(const CbParams p) {
  using Pol = typename PolicyFor<InT>::type;
  using Frag = typename Pol::Frag;
  constexpr int KS = DK / 32, LG = CbSmem<DK>::LG, NCT = DK / 16, KH = KS / 2;
  constexpr int NA2 = NCT > 8 ? NCT : 8;
  constexpr int PARTS = 512 / DK, CPP = 32 / PARTS;  // rowsum partials: threads per channel, columns each
  __shared__ __align__(16) CbSmem<DK> sm;
  if (*p.flag) return;  // the exact walk takes the call
  CbChunk ck;
  if (!cb_chunk(p, ck)) return;
  const int b = ck.b, h = ck.h, nvalid = ck.nvalid;
  const int64_t m0 = ck.m0;
  const int tid = threadIdx.x, w = (tid >> 6) & 3, hf = tid >> 8, l = tid & 63, r = l & 15, g = l >> 4;
  const int DV = p.DV;
  const int64_t SS = (int64_t)DK * DV;
  const bool kda = p.variant == 0 || p.variant == 3 || p.variant == 4;  // beta for both uses
  const InT* qp = static_cast<const InT*>(p.q);
  const InT* kp = static_cast<const InT*>(p.k);
  const InT* vp = static_cast<const InT*>(p.v);

  // A operands of row block w: first half Utilde (F1) and T (F2); second half Kbar (F1), T^T (F2)
  // and P^T (F3)
  Frag F1[KS], F2[2], F3[2];
  {
    float ut[KS][8], qt[KS][8];
    chunk_algebra<DK, InT, VEC>(p, sm, b, m0, h, nvalid, ut, qt, false);
    const float* Tm = sm.r2 + OT;
    const float* Pm = sm.r2 + OP;
    if (hf == 0) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) F1[ks] = Pol::make(ut[ks]);
#pragma unroll
      for (int st = 0; st < 2; ++st) F2[st] = frag_c<Pol>(&Tm[(16 * w + r) * L68 + 32 * st + 8 * g]);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = sm.r1[(16 * w + r) * LG + 32 * ks + 8 * g + j] * sm.gc[32 * ks + 8 * g + j];
        F1[ks] = Pol::make(x);
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        F2[st] = frag_s<Pol>(&Tm[(32 * st + 8 * g) * L68 + 16 * w + r], L68);
        F3[st] = frag_s<Pol>(&Pm[(32 * st + 8 * g) * L68 + 16 * w + r], L68);
      }
    }
  }
  // Gates of magnitude below CB_TAU (at most CB_NE; more hand the call to the walk): their gate
  // gradient is formed exactly, without the cumulative sum's cancelling terms, as
  // alpha_t dalpha_t = <L, R> with L = S0_i + sum_{s<t} Kd_si delta_s (S_{t-1}'s row i over Gamma_{t-1})
  // and R = Gamma_C,i dS_i + sum_{r>=t} (Qtilde_ri dO_r - Utilde_ri eps_r) (Gamma_t times the
  // gradient reaching X_t's row i): every term of R holds alpha_t as a factor, so the division by
  // alpha_t at the end loses nothing. Wave w8 takes entries w8, w8 + 8, ...; here Qtilde and
  // Utilde down each entry's channel.
  const int ne = sm.ne < CB_NE ? sm.ne : CB_NE;
  const int w8 = tid >> 6;
  for (int idx = tid; idx < ne * CH; idx += 512) {
    const int e = idx / CH, rr = idx % CH;
    const int te = sm.ent[e] / DK, ie = sm.ent[e] % DK;
    float qv = 0.f, uv = 0.f;
    if (rr >= te && rr < nvalid) {
      const int64_t m = m0 + rr;
      const float gm = sm.r0[rr * LG + ie];
      const int64_t th = cb_step(p, b, m, h);
      qv = gm * ld_f32(qp + q_elem(p, b, m, h, DK) + ie);
      uv = gm * (VEC ? p.erase[th * DK + ie] : p.erase[th]) * ld_f32(kp + kv_elem(p.k_ts, p.k_bs, p, b, m, h, DK) + ie);
    }
    sm.eq[e][rr] = qv;
    sm.eu[e][rr] = uv;
    if (rr == 0) sm.eacc[e] = 0.f;
  }
  __syncthreads();

  // ---- value blocks of 32 columns: delta, eps, dv and the tile gradients
  float* S0b = sm.r2;
  float* dSb = S0b + DK * L36;
  float* dOb = dSb + DK * L36;
  float* Dl = dOb + CH * L36;
  float* El = Dl + CH * L36;
  float* Rt = El + CH * L36;
  float* Yt = Rt + 32 * L68;
  const float* S0p = cb_start_state(p, ck, SS);
  const float* dSp = p.dsc + (int64_t)blockIdx.x * SS;
  // accumulators: first half dQtilde (A1) and dUtilde (A2) over the channel tiles; second half
  // dKbar (A1), dP over the token blocks (A2[0..3]) and dA (A2[4..7])
  f32x4 A1[NCT], A2[NA2];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) A1[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ct = 0; ct < NA2; ++ct) A2[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dpart = 0.f;
  float vdm[4] = {0.f, 0.f, 0.f, 0.f};  // second half: v . dm of rows 16 w + 4 g + i, this lane's columns
  for (int dv0 = 0; dv0 < DV; dv0 += 32) {
    // the block's S0, dS and dO, every load issued before the first store (a dO row that does not
    // count reads the chunk's first row and is zeroed at the store; loads under a condition were
    // each waited for inside it)
    constexpr int NSR = DK * 8 / 512;  // 16-byte pieces of S0 and of dS per thread
    f32x4 s0v[NSR], dsv[NSR];
    const float* S0q = S0p ? S0p : dSp;
#pragma unroll
    for (int k = 0; k < NSR; ++k) {
      const int idx = tid + 512 * k;
      const int64_t o = (int64_t)(idx >> 3) * DV + dv0 + 4 * (idx & 7);
      s0v[k] = *reinterpret_cast<const f32x4*>(S0q + o);
      dsv[k] = *reinterpret_cast<const f32x4*>(dSp + o);
    }
    const int td = tid >> 3, q4d = tid & 7;  // CH * 8 = 512 pieces of dO, one per thread
    const bool dok = td < nvalid && cb_last(p, m0 + td);
    const f32x4 dov = *reinterpret_cast<const f32x4*>(p.dO + cb_tok(p, b, m0 + (dok ? td : 0), h) * DV + dv0 + 4 * q4d);
#pragma unroll
    for (int k = 0; k < NSR; ++k) {
      const int idx = tid + 512 * k, row = idx >> 3, q4 = idx & 7;
      store4(&S0b[row * L36 + 4 * q4], S0p ? s0v[k] : f32x4{0.f, 0.f, 0.f, 0.f});
      store4(&dSb[row * L36 + 4 * q4], dsv[k]);
    }
    store4(&dOb[td * L36 + 4 * q4d], dok ? dov : f32x4{0.f, 0.f, 0.f, 0.f});
    // rows 16 w + 4 g + i, columns 16 ct + r of the block: first half m = write . v, second half v
    // (ev) and the write gate (wv)
    float ev[2][4], wv[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // the row index is made opaque so that its 64-bit offsets are formed again in each value
      // block instead of being hoisted out of the loop: held across it they pushed accumulators
      // to scratch (91 spilled registers; 10 now, none reloaded inside the loop's tile phase)
      int t = 16 * w + 4 * g + i;
      asm volatile("" : "+v"(t));
      const bool ok = t < nvalid;
      const int64_t m = m0 + (ok ? t : 0);
      const int64_t th = cb_step(p, b, m, h);
      const int64_t vo = kv_elem(p.v_ts, p.v_bs, p, b, m, h, DV);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int col = dv0 + 16 * ct + r;
        // loaded whatever ok (the row is clamped to the chunk's first) and selected after
        const float vr = ld_f32(vp + vo + col);
        const float wr = VEC ? p.write[th * DV + col] : p.write[th];
        const float vx = ok ? vr : 0.f;
        const float wg = ok ? wr : 0.f;
        ev[ct][i] = hf == 0 ? wg * vx : vx;
        wv[ct][i] = wg;
      }
    }
    __syncthreads();
    {  // rowsum(S0 . dS) partials: channel tid % DK, columns CPP * (tid / DK) ..
      const int ch = tid % DK, c0 = CPP * (tid / DK);
#pragma unroll
      for (int j = 0; j < CPP; ++j) dpart = fmaf(S0b[ch * L36 + c0 + j], dSb[ch * L36 + c0 + j], dpart);
    }
    {
      f32x4 acc[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (hf == 0) {  // X = Utilde S0 -> R = M - X, transposed into Rt
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
          for (int ct = 0; ct < 2; ++ct)
            Pol::mma(acc[ct], F1[ks], frag_s<Pol>(&S0b[(32 * ks + 8 * g) * L36 + 16 * ct + r], L36));
        }
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
          for (int i = 0; i < 4; ++i) Rt[(16 * ct + r) * L68 + 16 * w + 4 * g + i] = ev[ct][i] - acc[ct][i];
        }
      } else {  // Y = Kbar dS + P^T dO, transposed into Yt
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
          for (int ct = 0; ct < 2; ++ct)
            Pol::mma(acc[ct], F1[ks], frag_s<Pol>(&dSb[(32 * ks + 8 * g) * L36 + 16 * ct + r], L36));
        }
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          if (st == 1 || w < 2) {  // P^T's rows of block w are zero before token 16 w
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
              Pol::mma(acc[ct], F3[st], frag_s<Pol>(&dOb[(32 * st + 8 * g) * L36 + 16 * ct + r], L36));
          }
        }
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
          for (int i = 0; i < 4; ++i) Yt[(16 * ct + r) * L68 + 16 * w + 4 * g + i] = acc[ct][i];
        }
      }
    }
    __syncthreads();
    {  // delta = T R (first half), eps = T^T Y (second half; dm = eps goes to dv and the write gate)
      f32x4 acc[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      const float* src = hf == 0 ? Rt : Yt;
      // T's rows of block w are zero past token 16 w + 15, T^T's before token 16 w: skip the
      // 32-token step that is all zero
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if (hf == 0 ? (st == 0 || w >= 2) : (st == 1 || w < 2)) {
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) Pol::mma(acc[ct], F2[st], frag_c<Pol>(&src[(16 * ct + r) * L68 + 32 * st + 8 * g]));
        }
      }
      float* dst = hf == 0 ? Dl : El;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * w + 4 * g + i;
          dst[t * L36 + 16 * ct + r] = acc[ct][i];
          if (hf == 1 && t < nvalid) {
            int to = t;  // opaque, as above
            asm volatile("" : "+v"(to));
            const int64_t th = cb_step(p, b, m0 + to, h);
            const int col = dv0 + 16 * ct + r;
            const float e = acc[ct][i];
            p.dv[th * DV + col] = wv[ct][i] * e;
            if constexpr (VEC) p.dwrite[th * DV + col] = ev[ct][i] * e;
            else vdm[i] = fmaf(ev[ct][i], e, vdm[i]);
          }
        }
      }
    }
    __syncthreads();
    if (w8 < ne) cb_entries<DK>(sm, ne, w8, l, S0b, dSb, dOb, Dl, El);
    // tile gradients of row block w
    {
      const Frag AO = frag_c<Pol>(&dOb[(16 * w + r) * L36 + 8 * g]);
      float xe[8];
      load8(&El[(16 * w + r) * L36 + 8 * g], xe);
#pragma unroll
      for (int j = 0; j < 8; ++j) xe[j] = -xe[j];
      const Frag AE = Pol::make(xe);
      if (hf == 0) {  // dQtilde += dO S0^T, dUtilde -= eps S0^T
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const Frag BS = frag_c<Pol>(&S0b[(16 * ct + r) * L36 + 8 * g]);
          Pol::mma(A1[ct], AO, BS);
          Pol::mma(A2[ct], AE, BS);
        }
      } else {  // dKbar += delta dS^T, dP += dO delta^T, dA -= eps delta^T
        const Frag AD = frag_c<Pol>(&Dl[(16 * w + r) * L36 + 8 * g]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) Pol::mma(A1[ct], AD, frag_c<Pol>(&dSb[(16 * ct + r) * L36 + 8 * g]));
#pragma unroll
        for (int J = 0; J < NBLK; ++J) {
          if (J <= w) {
            const Frag BD = frag_c<Pol>(&Dl[(16 * J + r) * L36 + 8 * g]);
            Pol::mma(A2[J], AO, BD);
            Pol::mma(A2[NBLK + J], AE, BD);
          }
        }
      }
    }
    __syncthreads();
  }
  sm.ddp[tid] = dpart;
  // values read back at the end (loaded before any of this phase's stores, so that their loads
  // overlap the work in between): the decay at the positions whose gate gradient this lane writes,
  // and the erase gate
  float al[4][NCT / 2], esr[4], evr[VEC ? NCT : 1][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 16 * w + 4 * g + i;
    const int64_t mt = m0 + (t < nvalid ? t : 0);
    const int64_t th = cb_step(p, b, mt, h), tq = cb_tok(p, b, mt, h);
#pragma unroll
    for (int cc = 0; cc < NCT / 2; ++cc) al[i][cc] = p.alpha[tq * DK + 16 * (hf * (NCT / 2) + cc) + r];
    if constexpr (VEC) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) evr[ct][i] = hf == 0 ? p.erase[th * DK + 16 * ct + r] : 0.f;
      esr[i] = 0.f;
    } else {
      esr[i] = p.erase[th];
    }
  }

  // ---- Qtilde and Utilde -> r2 (recomputed from Gamma; each half takes half the channels),
  // Gamma at this lane's positions
  float* Ql = sm.r2;
  float* Ul = sm.r2 + CH * LG;
  {
    const int row = 16 * w + r;
    const bool valid = row < nvalid;
    const int64_t m = m0 + (valid ? row : 0);
    const int64_t th = cb_step(p, b, m, h);
    const int64_t qo = q_elem(p, b, m, h, DK), ko = kv_elem(p.k_ts, p.k_bs, p, b, m, h, DK);
    const float esr = VEC ? 0.f : p.erase[th];
    const float esc = valid ? esr : 0.f;
    // both slices' loads issued first, selected after (as in the chunk algebra)
    typename Raw8Of<InT>::type qr[KH], kr[KH];
    float br[VEC ? KH : 1][8];
#pragma unroll
    for (int kh = 0; kh < KH; ++kh) {
      const int ch0 = 32 * (hf * KH + kh) + 8 * g;
      ld_raw8(qp + qo + ch0, qr[kh]);
      ld_raw8(kp + ko + ch0, kr[kh]);
      if constexpr (VEC) load8(p.erase + th * DK + ch0, br[kh]);
    }
#pragma unroll
    for (int kh = 0; kh < KH; ++kh) {
      const int ch0 = 32 * (hf * KH + kh) + 8 * g;
      float q8[8], k8[8], b8[8], g8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        q8[j] = valid ? raw8_at(qr[kh], j) : 0.f;
        k8[j] = valid ? raw8_at(kr[kh], j) : 0.f;
        if constexpr (VEC) b8[j] = valid ? br[kh][j] : 0.f;
        else b8[j] = 0.f;
      }
      load8(&sm.r0[row * LG + ch0], g8);
      float a[8], u[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) { a[j] = q8[j] * g8[j]; u[j] = (VEC ? b8[j] : esc) * k8[j] * g8[j]; }
      store4(&Ql[row * LG + ch0], f32x4{a[0], a[1], a[2], a[3]});
      store4(&Ql[row * LG + ch0 + 4], f32x4{a[4], a[5], a[6], a[7]});
      store4(&Ul[row * LG + ch0], f32x4{u[0], u[1], u[2], u[3]});
      store4(&Ul[row * LG + ch0 + 4], f32x4{u[4], u[5], u[6], u[7]});
    }
  }
  float gam[NCT][4];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
    for (int i = 0; i < 4; ++i) gam[ct][i] = sm.r0[(16 * w + 4 * g + i) * LG + 16 * ct + r];
  }
  __syncthreads();
  float* dPl = sm.r0;
  float* dAl = sm.r0 + CH * L68;
  if (hf == 1) {
    // dP (lower triangle) and dA (strict lower triangle) -> r0
#pragma unroll
    for (int J = 0; J < NBLK; ++J) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * w + 4 * g + i, col = 16 * J + r;
        dPl[row * L68 + col] = (J <= w && col <= row) ? A2[J][i] : 0.f;
        dAl[row * L68 + col] = (J <= w && col < row) ? A2[NBLK + J][i] : 0.f;
      }
    }
    // Gamma_C . dKbar, and the column sums of Kbar . dKbar (= Kd . (Gamma_C . dKbar))
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int ch = 16 * ct + r;
      const float gcc = sm.gc[ch];
      float e = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        A1[ct][i] *= gcc;
        e = fmaf(sm.r1[(16 * w + 4 * g + i) * LG + ch], A1[ct][i], e);
      }
      e += __shfl_xor(e, 16);
      e += __shfl_xor(e, 32);
      if (g == 0) sm.ecs[w][ch] = e;
    }
  }
  __syncthreads();
  if (hf == 0) {  // dq' = dQtilde + dP Kd, du' = dUtilde + dA Kd
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      if (st == 0 || w >= 2) {
        const Frag AP = frag_c<Pol>(&dPl[(16 * w + r) * L68 + 32 * st + 8 * g]);
        const Frag AA = frag_c<Pol>(&dAl[(16 * w + r) * L68 + 32 * st + 8 * g]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const Frag BK = frag_s<Pol>(&sm.r1[(32 * st + 8 * g) * LG + 16 * ct + r], LG);
          Pol::mma(A1[ct], AP, BK);
          Pol::mma(A2[ct], AA, BK);
        }
      }
    }
  } else {  // dk' = Gamma_C . dKbar + dP^T Qtilde + dA^T Utilde
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      if (st == 1 || w < 2) {  // dP^T's and dA^T's rows of block w are zero before token 16 w
        const Frag APt = frag_s<Pol>(&dPl[(32 * st + 8 * g) * L68 + 16 * w + r], L68);
        const Frag AAt = frag_s<Pol>(&dAl[(32 * st + 8 * g) * L68 + 16 * w + r], L68);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          Pol::mma(A1[ct], APt, frag_s<Pol>(&Ql[(32 * st + 8 * g) * LG + 16 * ct + r], LG));
          Pol::mma(A1[ct], AAt, frag_s<Pol>(&Ul[(32 * st + 8 * g) * LG + 16 * ct + r], LG));
        }
      }
    }
  }
  __syncthreads();
  // dk as the key (second half) -> r0 (dP and dA are no longer read); then the first half forms
  // everything per (token 16 w + 4 g + i, channel 16 ct + r) from the LDS copies of Qtilde, Utilde
  // and Kd (q dq = Qtilde dq', u du = Utilde du', k = Gamma Kd), with x = q dq + u du - k dk -> X
  // in Qtilde's place
  float* X = sm.r2;
  float* Kk = sm.r0;
  if (hf == 1) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int i = 0; i < 4; ++i)  // Gamma in [2^-110, 2^100]: the reciprocal is exact to an ulp
        Kk[(16 * w + 4 * g + i) * LG + 16 * ct + r] = A1[ct][i] * __builtin_amdgcn_rcpf(gam[ct][i]);
    }
  }
  __syncthreads();
  if (hf == 0) {
    float kdu[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * w + 4 * g + i;
      const bool ok = t < nvalid;
      const int64_t mt = m0 + (ok ? t : 0);
      const int64_t th = cb_step(p, b, mt, h), tq = cb_tok(p, b, mt, h);
      const bool lastq = cb_last(p, mt);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int ch = 16 * ct + r, o = t * LG + ch;
        const float gm = gam[ct][i];
        const float dqv = gm * A1[ct][i];
        const float duv = gm * A2[ct][i];
        const float dkk = Kk[o];
        const float kv = sm.r1[o] * gm;
        const float evv = VEC ? evr[ct][i] : esr[i];
        X[o] = Ql[o] * A1[ct][i] + Ul[o] * A2[ct][i] - kv * dkk;
        if (ok) {
          if (lastq) p.dq[tq * DK + ch] = dqv;
          p.dk[th * DK + ch] = fmaf(evv, duv, dkk);
          if constexpr (VEC) p.derase[th * DK + ch] = kv * duv;
        }
        kdu[i] = fmaf(kv, duv, kdu[i]);
      }
    }
    if constexpr (!VEC) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float a = kdu[i];
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) a += __shfl_xor(a, d);
        if (r == 0) sm.red[0][0][16 * w + 4 * g + i] = a;
      }
    }
  } else if constexpr (!VEC) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = vdm[i];
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) v += __shfl_xor(v, d);
      if (r == 0) sm.red[0][1][16 * w + 4 * g + i] = v;
    }
  }
  __syncthreads();
  if constexpr (!VEC) {
    // per token: k . du over the channels, v . dm over the value columns
    if (tid < nvalid) {
      const int64_t th = cb_step(p, b, m0 + tid, h);
      const float a = sm.red[0][0][tid], v = sm.red[0][1][tid];
      if (kda) {
        p.derase[th] = a + v;
      } else {
        p.derase[th] = a;
        p.dwrite[th] = v;
      }
    }
  }
  // alpha_t dalpha_t = reverse cumulative sum of x + Gamma_C rowsum(S0 . dS) + sum_s Kbar . dKbar,
  // over PARTS segments of SEG tokens per channel: segment sums, then each segment's scan from the
  // sum of everything after it
  {
    constexpr int SEG = CH / PARTS;
    const int ch = tid % DK, sg = tid / DK;
    float xs[SEG], tot = 0.f;
#pragma unroll
    for (int j = 0; j < SEG; ++j) {
      xs[j] = X[(SEG * sg + j) * LG + ch];
      tot += xs[j];
    }
    float base = 0.f;
    if (sg == 0) {
#pragma unroll
      for (int q = 0; q < PARTS; ++q) base += sm.ddp[q * DK + ch];
      base *= sm.gc[ch];
#pragma unroll
      for (int q = 0; q < 4; ++q) base += sm.ecs[q][ch];
    }
    __syncthreads();
    sm.ddp[sg * DK + ch] = tot;
    if (sg == 0) sm.ecs[0][ch] = base;
    __syncthreads();
    float s = sm.ecs[0][ch];
    for (int q = PARTS - 1; q > sg; --q) s += sm.ddp[q * DK + ch];
#pragma unroll
    for (int j = SEG - 1; j >= 0; --j) {
      s += xs[j];
      X[(SEG * sg + j) * LG + ch] = s;
    }
  }
  __syncthreads();
  if (tid < ne) X[(sm.ent[tid] / DK) * LG + sm.ent[tid] % DK] = sm.eacc[tid];  // the entries' exact values
  __syncthreads();
  // each half writes half of the channel tiles
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 16 * w + 4 * g + i;
    if (t < nvalid && cb_first(p, m0 + t)) {  // the decay acts on a token's first step
      const int64_t tq = cb_tok(p, b, m0 + t, h);
#pragma unroll
      for (int cc = 0; cc < NCT / 2; ++cc) {
        const int ch = 16 * (hf * (NCT / 2) + cc) + r;
        p.dalpha[tq * DK + ch] = X[t * LG + ch] / al[i][cc];
      }
    }
  }
}

// ============================================================================ host
int64_t cbwd_record_bytes(int dk, int dv) { return dk == 64 ? CRec<64>::size(dv) : CRec<128>::size(dv); }

template <int DK, typename InT, bool VEC>
static hipError_t launch_cb_t(const CbParams& p, hipStream_t s) {
  const int64_t slots = (int64_t)p.slots * p.H;
  hipLaunchKernelGGL(cbwd_flag_clear_kernel, dim3(1), dim3(64), 0, s, p.flag);
  hipLaunchKernelGGL((cbwd_prep_kernel<DK, InT, VEC>), dim3((unsigned)slots), dim3(512), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t wg = (int64_t)p.nseq * p.H * (p.DV / 32);
  wg = (wg + 7) / 8 * 8;
  hipLaunchKernelGGL((cbwd_state_kernel<DK, InT>), dim3((unsigned)wg), dim3(256), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((cbwd_grad_kernel<DK, InT, VEC>), dim3((unsigned)slots), dim3(512), 0, s, p);
  return hipGetLastError();
}

template <int DK>
static hipError_t launch_cb_dk(const CbParams& p, bool bf16, bool vec, hipStream_t s) {
  if (bf16) return vec ? launch_cb_t<DK, __bf16, true>(p, s) : launch_cb_t<DK, __bf16, false>(p, s);
  return vec ? launch_cb_t<DK, float, true>(p, s) : launch_cb_t<DK, float, false>(p, s);
}

hipError_t launch_chunked_backward(const CbParams& p, int dk, bool bf16, bool vec, hipStream_t s) {
  if (p.nseq == 0 || p.H == 0) return hipSuccess;
  if (dk == 64) return launch_cb_dk<64>(p, bf16, vec, s);
  if (dk == 128) return launch_cb_dk<128>(p, bf16, vec, s);
  return hipErrorInvalidValue;
}

}  // namespace dr
