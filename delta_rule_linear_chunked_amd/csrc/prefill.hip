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
  float A[CH][LDT];         // strictly lower A
  float At[CH][LDT];        // T_II A_IK for K < I
  float Ti[CH][LDT];        // T = (I + A)^-1, lower blocks; upper blocks stay zero
  float P[CH][LDT];         // lower P; upper blocks stay zero
  float S[DVB][DK + 4];     // state block, transposed: [value column][key channel]
  float R[DVB][LDT];        // (M - Utilde S0)^T
  float D[DVB][LDT];        // delta^T
};

template <int N>
__device__ __forceinline__ void mul8(float (&x)[8], const float* p) {
  float t[8];
  load8(p, t);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] *= t[j];
}

template <int DKR, int DVB, typename InT, bool VEC>
__global__ __launch_bounds__(256, 1) void chunk_fwd_kernel(const Params p) {
  using Pol = typename PolicyFor<InT>::type;
  using Frag = typename Pol::Frag;
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
  const int I = w;  // this wave's 16-token block
  const InT* qp = static_cast<const InT*>(p.q);
  const InT* kp = static_cast<const InT*>(p.k);
  const InT* vp = static_cast<const InT*>(p.v);
  const int DV = p.DV;

  // ---- state block in, upper tiles of P and T zeroed
  for (int i = tid; i < CH * LDT; i += 256) {
    (&sm.P[0][0])[i] = 0.f;
    (&sm.Ti[0][0])[i] = 0.f;
  }
  for (int i = tid; i < DK * DVB; i += 256) {
    const int ch = i / DVB, c = i % DVB;
    float s0 = 0.f;
    if (p.S0 && ch < DKR) s0 = p.S0[(((int64_t)n * H + h) * DKR + ch) * DV + dv0 + c];
    sm.S[c][ch] = s0;
  }
  __syncthreads();

  for (int64_t c0 = 0; c0 < len; c0 += CH) {
    const int nrows = (int)((len - c0) < CH ? (len - c0) : CH);
    const int row = 16 * I + r;
    const bool valid = row < nrows;
    const int64_t th = (bos + c0 + row) * H + h;  // token-head index of this lane's row

    // ================= gate preparation and operands of this wave's rows
    Frag UF[KS], QF[KS], KD[KS];
    bool ok = true;
    {
      const float esc = (!VEC && valid) ? p.erase[th] : 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int ch0 = 32 * ks + 8 * g;
        float a8[8], k8[8], q8[8], b8[8];
        if (valid && ch0 < DKR) {
          load8(kp + th * DKR + ch0, k8);
          load8(qp + th * DKR + ch0, q8);
          load8(p.alpha + th * DKR + ch0, a8);
          if (VEC) load8(p.erase + th * DKR + ch0, b8);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) { k8[j] = 0.f; q8[j] = 0.f; a8[j] = 1.f; b8[j] = 0.f; }
        }
        float uf[8], qf[8], kd[8], kgv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float f = row_prefix_prod(a8[j]);
          const float gx = row_suffix_prod_excl(a8[j]);
          const float u = (VEC ? b8[j] : esc) * k8[j];
          const float af = fabsf(f);
          ok = ok && (af >= FAST_LO) && (af <= FAST_HI);
          uf[j] = u * f;
          qf[j] = q8[j] * f;
          kd[j] = k8[j] * __builtin_amdgcn_rcpf(f);
          kgv[j] = k8[j] * gx;
          if (r == 15) sm.tot[I][ch0 + j] = f;
        }
        *reinterpret_cast<f32x4*>(&sm.kg[row][ch0]) = f32x4{kgv[0], kgv[1], kgv[2], kgv[3]};
        *reinterpret_cast<f32x4*>(&sm.kg[row][ch0 + 4]) = f32x4{kgv[4], kgv[5], kgv[6], kgv[7]};
        UF[ks] = Pol::make(uf);
        QF[ks] = Pol::make(qf);
        KD[ks] = Pol::make(kd);
      }
    }
    const bool fast = __all(ok);
    __syncthreads();

    // ================= A and P tiles of block row I
    {
      f32x4 accA[NBLK], accP[NBLK];
#pragma unroll
      for (int J = 0; J < NBLK; ++J) { accA[J] = f32x4{0.f, 0.f, 0.f, 0.f}; accP[J] = accA[J]; }
#pragma unroll
      for (int J = 0; J < NBLK - 1; ++J) {
        if (J < I) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const int ch0 = 32 * ks + 8 * g;
            float x[8];
            load8(&sm.kg[16 * J + r][ch0], x);
            for (int Jp = J + 1; Jp < I; ++Jp) mul8<8>(x, &sm.tot[Jp][ch0]);
            const Frag B = Pol::make(x);
            Pol::mma(accA[J], UF[ks], B);
            Pol::mma(accP[J], QF[ks], B);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sm.A[16 * I + 4 * g + i][16 * J + r] = accA[J][i];
            sm.P[16 * I + 4 * g + i][16 * J + r] = accP[J][i];
          }
        }
      }
      if (fast) {
        f32x4 ad = f32x4{0.f, 0.f, 0.f, 0.f}, pd = ad;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          Pol::mma(ad, UF[ks], KD[ks]);
          Pol::mma(pd, QF[ks], KD[ks]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 4 * g + i;  // row within the block; r is the column
          sm.A[16 * I + rr][16 * I + r] = (r < rr) ? ad[i] : 0.f;
          sm.P[16 * I + rr][16 * I + r] = (r <= rr) ? pd[i] : 0.f;
        }
      } else {
        // Diagonal tile from running products of the gates (exact for any gate value).
        const float esc = (!VEC && valid) ? p.erase[th] : 0.f;
        float a2[KS][8], k2[KS][8], q2[KS][8], u2[KS][8];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int ch0 = 32 * ks + 8 * g;
          float b8[8];
          if (valid && ch0 < DKR) {
            load8(kp + th * DKR + ch0, k2[ks]);
            load8(qp + th * DKR + ch0, q2[ks]);
            load8(p.alpha + th * DKR + ch0, a2[ks]);
            if (VEC) load8(p.erase + th * DKR + ch0, b8);
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) { k2[ks][j] = 0.f; q2[ks][j] = 0.f; a2[ks][j] = 1.f; b8[j] = 0.f; }
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) u2[ks][j] = (VEC ? b8[j] : esc) * k2[ks][j];
        }
        for (int s = 0; s < 16; ++s) {
          float ap = 0.f, pp = 0.f;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float rho = row_prefix_prod(r > s ? a2[ks][j] : 1.f);
              const float kv = __shfl(k2[ks][j], 16 * g + s);
              ap = fmaf(u2[ks][j] * kv, rho, ap);
              pp = fmaf(q2[ks][j] * kv, rho, pp);
            }
          }
          ap += __shfl_xor(ap, 16);
          ap += __shfl_xor(ap, 32);
          pp += __shfl_xor(pp, 16);
          pp += __shfl_xor(pp, 32);
          if (g == 0) {
            sm.A[16 * I + r][16 * I + s] = (r > s) ? ap : 0.f;
            sm.P[16 * I + r][16 * I + s] = (r >= s) ? pp : 0.f;
          }
        }
      }
    }
    __syncthreads();

    // ================= T = (I + A)^-1
    // (a) diagonal blocks by forward substitution, one lane per column
    if (l < 16) {
      float t[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        float acc = (rr == l) ? 1.f : 0.f;
#pragma unroll
        for (int s = 0; s < rr; ++s) acc = fmaf(-sm.A[16 * I + rr][16 * I + s], t[s], acc);
        t[rr] = acc;
      }
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sm.Ti[16 * I + rr][16 * I + l] = t[rr];
    }
    __syncthreads();
    // (b) At_IK = T_II A_IK
    {
      float x[8];
      if (g < 2) load8(&sm.Ti[16 * I + r][16 * I + 8 * g], x);
      else {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = 0.f;
      }
      const Frag Tii = Pol::make(x);
#pragma unroll
      for (int K = 0; K < NBLK - 1; ++K) {
        if (K < I) {
          float y[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) y[j] = (g < 2) ? sm.A[16 * I + 8 * g + j][16 * K + r] : 0.f;
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
          Pol::mma(acc, Tii, Pol::make(y));
#pragma unroll
          for (int i = 0; i < 4; ++i) sm.At[16 * I + 4 * g + i][16 * K + r] = acc[i];
        }
      }
    }
    __syncthreads();
    // (c) T_IJ = -sum_{K=J..I-1} At_IK T_KJ, by increasing distance I - J
#pragma unroll
    for (int d = 1; d < NBLK; ++d) {
      if (I >= d) {
        const int J = I - d;
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          if (st < (d + 1) / 2) {
            const int k0 = 16 * J + 32 * st + 8 * g;
            float a8[8], b8[8];
            if (k0 < 16 * I) {
              load8(&sm.At[16 * I + r][k0], a8);
#pragma unroll
              for (int j = 0; j < 8; ++j) b8[j] = sm.Ti[k0 + j][16 * J + r];
            } else {
#pragma unroll
              for (int j = 0; j < 8; ++j) { a8[j] = 0.f; b8[j] = 0.f; }
            }
            Pol::mma(acc, Pol::make(a8), Pol::make(b8));
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.Ti[16 * I + 4 * g + i][16 * J + r] = -acc[i];
      }
      __syncthreads();
    }

    // ================= X = Utilde S0, Y = Qtilde S0, R = M - X   (block row I)
    f32x4 accY[NCT];
    {
      f32x4 accX[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) { accX[ct] = f32x4{0.f, 0.f, 0.f, 0.f}; accY[ct] = accX[ct]; }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int ch0 = 32 * ks + 8 * g;
        float pre[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pre[j] = 1.f;
        for (int Jp = 0; Jp < I; ++Jp) mul8<8>(pre, &sm.tot[Jp][ch0]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          float x[8];
          load8(&sm.S[16 * ct + r][ch0], x);
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] *= pre[j];
          const Frag B = Pol::make(x);
          Pol::mma(accX[ct], UF[ks], B);
          Pol::mma(accY[ct], QF[ks], B);
        }
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int col = dv0 + 16 * ct + r;
        f32x4 rv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rw = 16 * I + 4 * g + i;
          float m = 0.f;
          if (rw < nrows) {
            const int64_t tht = (bos + c0 + rw) * H + h;
            const float wg = VEC ? p.write[tht * DV + col] : p.write[tht];
            m = wg * ld_f32(vp + tht * DV + col);
          }
          rv[i] = m - accX[ct][i];
        }
        *reinterpret_cast<f32x4*>(&sm.R[16 * ct + r][16 * I + 4 * g]) = rv;
      }
    }
    __syncthreads();

    // ================= delta = T R   (block row I)
    const int nst = (I + 2) / 2;
    {
      f32x4 accD[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) accD[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if (st < nst) {
          const int k0 = 32 * st + 8 * g;
          float a8[8];
          load8(&sm.Ti[16 * I + r][k0], a8);
          const Frag Af = Pol::make(a8);
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            float b8[8];
            load8(&sm.R[16 * ct + r][k0], b8);
            Pol::mma(accD[ct], Af, Pol::make(b8));
          }
        }
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        *reinterpret_cast<f32x4*>(&sm.D[16 * ct + r][16 * I + 4 * g]) = accD[ct];
    }
    __syncthreads();

    // ================= O = Y + P delta   (block row I)
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      if (st < nst) {
        const int k0 = 32 * st + 8 * g;
        float a8[8];
        load8(&sm.P[16 * I + r][k0], a8);
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
        const int rw = 16 * I + 4 * g + i;
        if (rw < nrows) p.o[((bos + c0 + rw) * H + h) * DV + dv0 + 16 * ct + r] = accY[ct][i];
      }
    }

    // ================= S <- Diag(Gamma_C) S0 + Kbar^T delta   (key-channel tiles of this wave)
    for (int rt = w; rt < DK / 16; rt += 4) {
      const int chA = 16 * rt + r;
      Frag KB[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int k0 = 32 * st + 8 * g;
        const int blk = k0 >> 4;
        float suf = 1.f;
        for (int Jp = blk + 1; Jp < NBLK; ++Jp) suf *= sm.tot[Jp][chA];
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = sm.kg[k0 + j][chA] * suf;
        KB[st] = Pol::make(x);
      }
      float gC[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ch = 16 * rt + 4 * g + i;
        gC[i] = sm.tot[0][ch] * sm.tot[1][ch] * sm.tot[2][ch] * sm.tot[3][ch];
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 s4 = *reinterpret_cast<const f32x4*>(&sm.S[16 * ct + r][16 * rt + 4 * g]);
        f32x4 acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = gC[i] * s4[i];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          float b8[8];
          load8(&sm.D[16 * ct + r][32 * st + 8 * g], b8);
          Pol::mma(acc, KB[st], Pol::make(b8));
        }
        *reinterpret_cast<f32x4*>(&sm.S[16 * ct + r][16 * rt + 4 * g]) = acc;
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
