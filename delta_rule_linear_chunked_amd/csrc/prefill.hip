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
//   delta  = (I + A)^-1 (M - Utilde S0),     Utilde_r = Gamma_r . u_r
//   O      = Qtilde S0 + P delta,            Qtilde_r = Gamma_r . q_r
//   S_C    = Diag(Gamma_C) S0 + Kbar^T delta, Kbar_s = ratio(C, s) . k_s
//
// (derived by unrolling the step rule; the course page "GDN, KDA và Mamba-2",
// section 3, asks for such a chunked kernel to be checked against the step
// recurrence).
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
// and inside a block ratio(r, s) = f_r * (1 / f_s). The in-block factorisation
// is used only while every |f| of the block lies in [2^-100, 2^100]; otherwise
// (gates at or extremely close to zero) the block's diagonal tile is computed
// directly from running products, which is exact for any gate value.
//
// Work split: one workgroup of four waves per (sequence, head, block of value
// columns); the d_k x DVB state block stays in LDS across the whole sequence.
// Wave w owns token rows 16w..16w+15 of each chunk.
#include "common.hpp"
#include "launch.hpp"

namespace dr {

constexpr int CH = 64;    // chunk length
constexpr int NBLK = 4;   // 16-token blocks per chunk
constexpr int LDT = 68;   // padded row stride of 64-wide tiles (floats)
constexpr float FAST_LO = 0x1p-100f;
constexpr float FAST_HI = 0x1p100f;

template <int DK, int DVB>
struct PrefillSmem {
  float kg[CH][DK + 4];     // k_s . g_s
  float tot[NBLK][DK];      // t_J
  float A[CH][LDT];         // A: strictly lower diagonal blocks and the blocks below them
  float P[CH][LDT];         // P: lower blocks; blocks above the diagonal stay zero
  float Td[NBLK][16][20];   // (I + A_JJ)^-1 of each diagonal block
  float S[DVB][DK + 4];     // state block, transposed: [value column][key channel]
  float D[DVB][LDT];        // delta^T
};

// Orders this wave's LDS writes before its later LDS reads by other lanes of the
// same wave (LDS executes a wave's instructions in order; this stops the compiler
// from reordering across the point).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <int DKR, int DVB, typename InT, bool VEC>
__global__ __launch_bounds__(256, 1) void chunk_fwd_kernel(const Params p) {
  using Pol = typename PolicyFor<InT>::type;
  using Frag = typename Pol::Frag;
  using Frag4 = typename Pol::Frag4;
  constexpr int DK = DKR < 32 ? 32 : DKR;  // key width padded to the 32-deep MFMA slice
  constexpr int KS = DK / 32;              // reduction slices over key channels
  constexpr int NCT = DVB / 16;            // 16-wide value-column tiles
  static_assert(DVB % 16 == 0 && DVB <= 64, "value block");

  __shared__ __align__(16) PrefillSmem<DK, DVB> sm;

  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  if (lid >= p.grid_logical) return;
  const int pair = lid / p.ndvb;
  const int dv0 = (lid % p.ndvb) * DVB;
  const int H = p.H;
  const int n = pair / H, h = pair % H;
  int64_t bos, len;
  if (p.cu) {
    bos = p.cu[n];
    len = (int64_t)p.cu[n + 1] - bos;
  } else {
    bos = (int64_t)n * p.T;
    len = p.T;
  }

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, r = l & 15, g = l >> 4;
  const InT* qp = static_cast<const InT*>(p.q);
  const InT* kp = static_cast<const InT*>(p.k);
  const InT* vp = static_cast<const InT*>(p.v);
  const int DV = p.DV;

  // ---- state block in; P's upper blocks zeroed once (never written)
  for (int i = tid; i < CH * LDT; i += 256) (&sm.P[0][0])[i] = 0.f;
  for (int i = tid; i < DK * DVB; i += 256) {
    const int ch = i / DVB, c = i % DVB;
    float s0 = 0.f;
    if (p.S0 && ch < DKR) s0 = p.S0[(((int64_t)n * H + h) * DKR + ch) * DV + dv0 + c];
    sm.S[c][ch] = s0;
  }

  // ---- prefetch registers: this lane's token row of the next chunk (lane layout of the
  // 32-deep fragments: row r of block w, channels 32*ks + 8*g + j), and the value/write
  // entries it needs in accumulator layout (rows 4*g + i of block w, column 16*ct + r).
  Raw8<InT> pk[KS], pq[KS];
  float pa[KS][8], pb[VEC ? KS : 1][8];
  float pe = 0.f;
  InT pv[NCT][4];  // raw: converting at load time would make the load synchronous
  float pw[VEC ? NCT : 1][4];
  auto prefetch = [&](int64_t c0n) {
    const int64_t last = bos + len - 1;  // a valid token: rows past the end are clamped, then masked
    int64_t tk = bos + c0n + 16 * w + r;
    tk = tk > last ? last : tk;
    const int64_t th = tk * H + h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch0 = (32 * ks + 8 * g) < DKR ? (32 * ks + 8 * g) : 0;
      pk[ks].load(kp + th * DKR + ch0);
      pq[ks].load(qp + th * DKR + ch0);
      load8(p.alpha + th * DKR + ch0, pa[ks]);
      if constexpr (VEC) load8(p.erase + th * DKR + ch0, pb[ks]);
    }
    if constexpr (!VEC) pe = p.erase[th];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int64_t tv = bos + c0n + 16 * w + 4 * g + i;
      tv = tv > last ? last : tv;
      const int64_t thv = tv * H + h;
      if constexpr (!VEC) pw[0][i] = p.write[thv];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int col = dv0 + 16 * ct + r;
        pv[ct][i] = vp[thv * DV + col];
        if constexpr (VEC) pw[ct][i] = p.write[thv * DV + col];
      }
    }
  };
  if (len > 0) prefetch(0);
  __syncthreads();

  for (int64_t c0 = 0; c0 < len; c0 += CH) {
    const int row = 16 * w + r;
    const bool valid = c0 + row < len;

    // ================= gate preparation, operands and the diagonal tiles of block w
    Frag UF[KS], QF[KS];
    float mv[NCT][4];  // write vectors m of rows 4g+i (accumulator layout)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool vi = c0 + 16 * w + 4 * g + i < len;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        mv[ct][i] = vi ? pw[VEC ? ct : 0][i] * (float)pv[ct][i] : 0.f;
        // Materialise here: if the product sinks past the next prefetch, the old and new
        // prefetch registers overlap and the compiler copies them with waiting moves.
        asm volatile("" : "+v"(mv[ct][i]));
      }
    }
    {
      bool ok = true;
      f32x4 ad = f32x4{0.f, 0.f, 0.f, 0.f}, pd = ad;
      float fr[KS][8], rf[KS][8];  // f_r and 1 / f_r of this lane's row
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int ch0 = 32 * ks + 8 * g;
        const bool live = valid && ch0 < DKR;
        float uf[8], qf[8], kd[8], f8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) f8[j] = live ? pa[ks][j] : 1.f;
        row_prefix_prod8(f8);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float kk = live ? pk[ks].get(j) : 0.f;
          const float qq = live ? pq[ks].get(j) : 0.f;
          const float ee = VEC ? pb[VEC ? ks : 0][j] : pe;
          const float f = f8[j];
          const float af = fabsf(f);
          ok = ok && (af >= FAST_LO) && (af <= FAST_HI);
          fr[ks][j] = f;
          rf[ks][j] = __builtin_amdgcn_rcpf(f);
          uf[j] = ee * kk * f;
          qf[j] = qq * f;
          kd[j] = kk * rf[ks][j];
        }
        if (r == 15) {
          store4(&sm.tot[w][ch0], f32x4{fr[ks][0], fr[ks][1], fr[ks][2], fr[ks][3]});
          store4(&sm.tot[w][ch0 + 4], f32x4{fr[ks][4], fr[ks][5], fr[ks][6], fr[ks][7]});
        }
        UF[ks] = Pol::make(uf);
        QF[ks] = Pol::make(qf);
        const Frag KD = Pol::make(kd);
        Pol::mma(ad, UF[ks], KD);
        Pol::mma(pd, QF[ks], KD);
      }
      const bool fast = __all(ok);
      // k_s . g_s, g_s = prod of alpha over s+1 .. block end: t / f_s while every |f| is in
      // range, else an exact suffix scan.
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int ch0 = 32 * ks + 8 * g;
        const bool live = valid && ch0 < DKR;
        float kgv[8];
        if (fast) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float t = dpp_or<ROW_BCAST15>(0.f, fr[ks][j]);
            kgv[j] = (live ? pk[ks].get(j) : 0.f) * (t * rf[ks][j]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float a = live ? pa[ks][j] : 1.f;
            kgv[j] = (live ? pk[ks].get(j) : 0.f) * row_suffix_prod_excl(a);
          }
        }
        store4(&sm.kg[row][ch0], f32x4{kgv[0], kgv[1], kgv[2], kgv[3]});
        store4(&sm.kg[row][ch0 + 4], f32x4{kgv[4], kgv[5], kgv[6], kgv[7]});
      }
      if (fast) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 4 * g + i;  // row within the block; r is the column
          sm.A[16 * w + rr][16 * w + r] = (r < rr) ? ad[i] : 0.f;
          sm.P[16 * w + rr][16 * w + r] = (r <= rr) ? pd[i] : 0.f;
        }
      } else {
        // Diagonal tile from running products of the gates (exact for any gate value,
        // including zero), reloading this lane's row of the chunk.
        const int64_t last = bos + len - 1;
        int64_t tk = bos + c0 + row;
        tk = tk > last ? last : tk;
        const int64_t th = tk * H + h;
        for (int s = 0; s < 16; ++s) {
          float ap = 0.f, pp = 0.f;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const int ch0 = 32 * ks + 8 * g;
            const bool live = valid && ch0 < DKR;
            float a2[8], k2[8], q2[8], b2[8];
            load8(p.alpha + th * DKR + (live ? ch0 : 0), a2);
            load8(kp + th * DKR + (live ? ch0 : 0), k2);
            load8(qp + th * DKR + (live ? ch0 : 0), q2);
            if constexpr (VEC) load8(p.erase + th * DKR + (live ? ch0 : 0), b2);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float a = live ? a2[j] : 1.f;
              const float kk = live ? k2[j] : 0.f;
              const float qq = live ? q2[j] : 0.f;
              const float uu = (VEC ? b2[j] : pe) * kk;
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
            sm.P[16 * w + r][16 * w + s] = (r >= s) ? pp : 0.f;
          }
        }
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
    // Unconditional (rows past the end are clamped): a conditional prefetch makes the
    // compiler copy the in-flight registers at the loop latch, which waits for the loads.
    prefetch(c0 + CH);
    __syncthreads();

    // ================= off-diagonal tiles of block row w, and X = Utilde S0, Y = Qtilde S0
    f32x4 accY[NCT], Rm[NCT];
    {
      f32x4 accA[NBLK - 1], accP[NBLK - 1], accX[NCT];
#pragma unroll
      for (int J = 0; J < NBLK - 1; ++J) { accA[J] = f32x4{0.f, 0.f, 0.f, 0.f}; accP[J] = accA[J]; }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) { accX[ct] = f32x4{0.f, 0.f, 0.f, 0.f}; accY[ct] = accX[ct]; }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int ch0 = 32 * ks + 8 * g;
        // running product over earlier blocks: mid[J] = prod_{J<J'<w} t_J', pre = prod_{J<w} t_J
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
#pragma unroll
        for (int J = 0; J < NBLK - 1; ++J) {
          if (J < w) {
            float x[8];
            load8(&sm.kg[16 * J + r][ch0], x);
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] *= mid[J][j];
            const Frag B = Pol::make(x);
            Pol::mma(accA[J], UF[ks], B);
            Pol::mma(accP[J], QF[ks], B);
          }
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          float x[8];
          load8(&sm.S[16 * ct + r][ch0], x);
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] *= run[j];
          const Frag B = Pol::make(x);
          Pol::mma(accX[ct], UF[ks], B);
          Pol::mma(accY[ct], QF[ks], B);
        }
      }
#pragma unroll
      for (int J = 0; J < NBLK - 1; ++J) {
        if (J < w) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sm.A[16 * w + 4 * g + i][16 * J + r] = accA[J][i];
            sm.P[16 * w + 4 * g + i][16 * J + r] = accP[J][i];
          }
        }
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
        for (int i = 0; i < 4; ++i) Rm[ct][i] = mv[ct][i] - accX[ct][i];
      }
    }
    __syncthreads();

    // ================= delta by blocked forward substitution:
    //   delta_J = (I + A_JJ)^-1 (R_J - sum_{K<J} A_JK delta_K)
#pragma unroll
    for (int J = 0; J < NBLK; ++J) {
      if (w == J) {
#pragma unroll
        for (int K = 0; K < NBLK - 1; ++K) {
          if (K < J) {
            float a4[4];
            load4(&sm.A[16 * J + r][16 * K + 4 * g], a4);
#pragma unroll
            for (int j = 0; j < 4; ++j) a4[j] = -a4[j];
            const Frag4 Af = Pol::make4(a4);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
              float b4[4];
              load4(&sm.D[16 * ct + r][16 * K + 4 * g], b4);
              Pol::mma16(Rm[ct], Af, Pol::make4(b4));
            }
          }
        }
        float t4[4];
        load4(&sm.Td[J][r][4 * g], t4);
        const Frag4 Tf = Pol::make4(t4);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          float b4[4] = {Rm[ct][0], Rm[ct][1], Rm[ct][2], Rm[ct][3]};
          f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
          Pol::mma16(d, Tf, Pol::make4(b4));
          store4(&sm.D[16 * ct + r][16 * J + 4 * g], d);
        }
      }
      __syncthreads();
    }

    // ================= O = Y + P delta   (block row w)
    const int nst = (w + 2) / 2;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      if (st < nst) {
        const int k0 = 32 * st + 8 * g;
        float a8[8];
        load8(&sm.P[16 * w + r][k0], a8);
        const Frag Af = Pol::make(a8);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          float b8[8];
          load8(&sm.D[16 * ct + r][k0], b8);
          Pol::mma(accY[ct], Af, Pol::make(b8));
        }
      }
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rw = 16 * w + 4 * g + i;
        if (c0 + rw < len) p.o[((bos + c0 + rw) * H + h) * DV + dv0 + 16 * ct + r] = accY[ct][i];
      }
    }

    // ================= S <- Diag(Gamma_C) S0 + Kbar^T delta   (key-channel tiles of this wave)
    {
      Frag DF[NCT][2];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          float b8[8];
          load8(&sm.D[16 * ct + r][32 * st + 8 * g], b8);
          DF[ct][st] = Pol::make(b8);
        }
      }
      for (int rt = w; rt < DK / 16; rt += 4) {
        const int chA = 16 * rt + r;
        float tA[NBLK];
#pragma unroll
        for (int J = 0; J < NBLK; ++J) tA[J] = sm.tot[J][chA];
        Frag KB[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int k0 = 32 * st + 8 * g;
          const int blk = 2 * st + (g >> 1);
          float suf = 1.f;
#pragma unroll
          for (int J = 1; J < NBLK; ++J) suf *= (J > blk) ? tA[J] : 1.f;
          float x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = sm.kg[k0 + j][chA] * suf;
          KB[st] = Pol::make(x);
        }
        float tt[NBLK][4];
#pragma unroll
        for (int J = 0; J < NBLK; ++J) load4(&sm.tot[J][16 * rt + 4 * g], tt[J]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          float s4[4];
          load4(&sm.S[16 * ct + r][16 * rt + 4 * g], s4);
          f32x4 acc;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = tt[0][i] * tt[1][i] * tt[2][i] * tt[3][i] * s4[i];
#pragma unroll
          for (int st = 0; st < 2; ++st) Pol::mma(acc, KB[st], DF[ct][st]);
          store4(&sm.S[16 * ct + r][16 * rt + 4 * g], acc);
        }
      }
    }
    __syncthreads();
  }

  // ---- final state out
  if (p.S) {
    for (int i = tid; i < DKR * DVB; i += 256) {
      const int ch = i / DVB, c = i % DVB;
      p.S[(((int64_t)n * H + h) * DKR + ch) * DV + dv0 + c] = sm.S[c][ch];
    }
  }
}

PrefillPlan plan_prefill(int64_t num_pairs, int dk, int dv) {
  (void)dk;
  PrefillPlan pl;
  pl.chunk = CH;
  pl.dv_block = (dv >= 32 && num_pairs * (dv / 32) >= 256) ? 32 : 16;
  pl.ndvb = dv / pl.dv_block;
  const int64_t logical = num_pairs * pl.ndvb;
  pl.workgroups = (logical + 7) / 8 * 8;
  return pl;
}

template <int DKR, int DVB, typename InT, bool VEC>
static hipError_t launch_t(const Params& p, const PrefillPlan& pl, hipStream_t s) {
  hipLaunchKernelGGL((chunk_fwd_kernel<DKR, DVB, InT, VEC>), dim3((unsigned)pl.workgroups), dim3(256),
                     0, s, p);
  return hipGetLastError();
}

template <int DKR, int DVB>
static hipError_t launch_gate(const Params& p, const PrefillPlan& pl, bool bf16, bool vec, hipStream_t s) {
  if (bf16) return vec ? launch_t<DKR, DVB, __bf16, true>(p, pl, s) : launch_t<DKR, DVB, __bf16, false>(p, pl, s);
  return vec ? launch_t<DKR, DVB, float, true>(p, pl, s) : launch_t<DKR, DVB, float, false>(p, pl, s);
}

template <int DKR>
static hipError_t launch_dvb(const Params& p, const PrefillPlan& pl, bool bf16, bool vec, hipStream_t s) {
  if (pl.dv_block == 32) return launch_gate<DKR, 32>(p, pl, bf16, vec, s);
  return launch_gate<DKR, 16>(p, pl, bf16, vec, s);
}

hipError_t launch_prefill(const Params& p, const PrefillPlan& pl, int dk, bool bf16, bool vec,
                          hipStream_t s) {
  if (pl.workgroups == 0) return hipSuccess;
  switch (dk) {
    case 16: return launch_dvb<16>(p, pl, bf16, vec, s);
    case 32: return launch_dvb<32>(p, pl, bf16, vec, s);
    case 64: return launch_dvb<64>(p, pl, bf16, vec, s);
    case 128: return launch_dvb<128>(p, pl, bf16, vec, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dr
