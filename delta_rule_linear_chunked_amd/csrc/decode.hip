// Single-token decode step of the gated delta rule on gfx950.
//
// One workgroup per (sequence, head, slice of DVS value columns): every value
// column of the update is independent (delta_j needs only column j of S), so a
// head splits into d_v / DVS workgroups with no exchange between them. The slice
// of the fp32 state is streamed from HBM once with 128-bit non-temporal loads,
// kept in registers, reduced over key rows, updated and streamed back in place,
// so each state byte is read once and written once:
//
//   r_u = S^T (alpha . u),   r_q = S^T (alpha . q)        (one pass over S)
//   delta = m - r_u                                        (delta-rule error)
//   S <- Diag(alpha) S + k delta^T                         (in place)
//   o = S_new^T q = r_q + (q . k) delta
//
// The update is the rule S_t = (I - k u^T) Diag(alpha) S + k m^T with the
// erase/write vectors u, m of the KDA, RDA and GDN-2 rules (Hugging Face
// discussion "KRAFTON/Raon-1-mini-preview" #1, the three state updates); the
// last identity follows from S_new^T q = Diag(alpha)S^T q + delta (k . q).
#include "common.hpp"
#include "launch.hpp"

#ifndef DECODE_DVS
#define DECODE_DVS 128
#endif
#ifndef DECODE_NT
#define DECODE_NT 256
#endif

namespace dr {

template <int DK, int DV>
struct DecodeShape {
  static constexpr int DVS = DECODE_DVS < DV ? DECODE_DVS : DV;       // value columns per workgroup
  static constexpr int NSPLIT = DV / DVS;
  static constexpr int COLS4 = DVS / 4;                                // float4 columns
  static constexpr int RG = (DK < DECODE_NT / COLS4) ? DK : DECODE_NT / COLS4;  // row groups
  static constexpr int RPT = DK / RG;                                  // rows per thread
  static constexpr int NT = RG * COLS4;                                // threads
  static_assert(RG * RPT == DK, "row split");
  static_assert(NT <= 512 && NT % 64 == 0, "thread count");
};

template <int DK, int DV, typename InT, bool VEC>
__global__ __launch_bounds__((DecodeShape<DK, DV>::NT)) void decode_kernel(const Params p) {
  using Sh = DecodeShape<DK, DV>;
  constexpr int DVS = Sh::DVS, COLS4 = Sh::COLS4, RG = Sh::RG, RPT = Sh::RPT, NT = Sh::NT;
  __shared__ float s_q[DK], s_k[DK], s_au[DK], s_aq[DK], s_a[DK], s_m[DVS];
  __shared__ float s_red[2][RG][DVS + 4];
  __shared__ float s_qk[RG];
  __shared__ float s_delta[DVS];
  __shared__ float s_norm[2];

  const int tid = threadIdx.x;
  const int c4 = tid % COLS4;
  const int rg = tid / COLS4;
  const int64_t nh = blockIdx.x / Sh::NSPLIT;          // sequence * H + head
  const int col0 = (blockIdx.x % Sh::NSPLIT) * DVS;    // first value column of the slice
  // state row: the sequence's own, or slot state_idx[n] of a pool; a slot outside the
  // pool has no state: the output is zero and nothing is read or written
  int64_t srow = nh;
  if (p.sidx) {
    const int64_t n = nh / p.H;
    const int32_t sl = p.sidx[n];
    if (sl < 0 || sl >= p.nslots) {
      for (int j = tid; j < DVS; j += NT) p.o[nh * DV + col0 + j] = 0.f;
      return;
    }
    srow = (int64_t)sl * p.H + (nh - n * p.H);
  }
  float* S = p.S + srow * (int64_t)DK * DV + col0;

  // The token's vectors first (one element per thread; they are small and the staging below
  // needs them), then the state: memory returns in issue order, so the staging does not wait
  // for the state to arrive.
  const int64_t sn = nh / p.H, sh = nh - sn * p.H;  // sequence and head (inputs through their strides)
  const InT* q = static_cast<const InT*>(p.q) + sn * p.q_bs + sh * DK;
  const InT* k = static_cast<const InT*>(p.k) + sn * p.k_bs + sh * DK;
  const InT* v = static_cast<const InT*>(p.v) + sn * p.v_bs + sh * DV + col0;
  static_assert(DK <= NT && DVS <= NT, "one token element per thread");
  const bool prep = p.a_act || p.g_act || p.a_bf16;  // fused activations (uniform)
  float qi = 0.f, ki = 0.f, az = 0.f, e = 0.f, vj = 0.f, wr = 0.f;
  if (tid < DK) {
    qi = ld_f32(q + tid);
    ki = ld_f32(k + tid);
    az = p.a_bf16 ? (float)static_cast<const __bf16*>(p.alpha)[nh * DK + tid]
                  : static_cast<const float*>(p.alpha)[nh * DK + tid];
    e = VEC ? p.erase[nh * DK + tid] : p.erase[nh];
  }
  if (tid < DVS) {
    vj = ld_f32(v + tid);
    wr = VEC ? p.write[nh * DV + col0 + tid] : p.write[nh];
  }
  f32x4 st[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + RG * i;
    st[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + row * DV) + c4);
  }

  // inverse L2 norms of q and k over d_k (1 when the inputs come normalised)
  float nq = 1.f, nk = 1.f;
  if (p.prep_l2) {
    float sq = qi * qi, sk = ki * ki;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      sq += __shfl_xor(sq, o);
      sk += __shfl_xor(sk, o);
    }
    if ((tid & 63) == 0 && tid < DK) {
      s_red[0][0][tid >> 6] = sq;
      s_red[1][0][tid >> 6] = sk;
    }
    __syncthreads();
    if (tid == 0) {
      float tq = 0.f, tk = 0.f;
      for (int wv = 0; wv < (DK + 63) / 64; ++wv) {
        tq += s_red[0][0][wv];
        tk += s_red[1][0][wv];
      }
      s_norm[0] = tq > 0.f ? __builtin_amdgcn_rsqf(tq) : 0.f;
      s_norm[1] = tk > 0.f ? __builtin_amdgcn_rsqf(tk) : 0.f;
    }
    __syncthreads();
    nq = s_norm[0];
    nk = s_norm[1];
  }
  if (tid < DK) {
    const float a = prep ? prep_alpha(az, p) : az;
    const float ug = prep ? prep_gate(e, p) : e;
    qi *= nq;
    ki *= nk;
    s_q[tid] = qi;
    s_k[tid] = ki;
    s_a[tid] = a;
    s_au[tid] = a * (ug * ki);
    s_aq[tid] = a * qi;
  }
  if (tid < DVS) s_m[tid] = (prep ? prep_gate(wr, p) : wr) * vj;
  __syncthreads();

  // Partial reductions over this thread's rows.
  float ru[4] = {0.f, 0.f, 0.f, 0.f}, rq[4] = {0.f, 0.f, 0.f, 0.f}, qk = 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + RG * i;
    const float au = s_au[row], aq = s_aq[row];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      ru[c] = fmaf(st[i][c], au, ru[c]);
      rq[c] = fmaf(st[i][c], aq, rq[c]);
    }
    qk = fmaf(s_q[row], s_k[row], qk);
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    s_red[0][rg][4 * c4 + c] = ru[c];
    s_red[1][rg][4 * c4 + c] = rq[c];
  }
  if (c4 == 0) s_qk[rg] = qk;
  __syncthreads();

  if (tid < DVS) {
    float u_sum = 0.f, q_sum = 0.f, qk_sum = 0.f;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      u_sum += s_red[0][g][tid];
      q_sum += s_red[1][g][tid];
      qk_sum += s_qk[g];
    }
    const float delta = s_m[tid] - u_sum;
    s_delta[tid] = delta;
    p.o[nh * DV + col0 + tid] = fmaf(qk_sum, delta, q_sum);
  }
  __syncthreads();

  float d[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) d[c] = s_delta[4 * c4 + c];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + RG * i;
    const float a = s_a[row], kr = s_k[row];
    f32x4 nv;
#pragma unroll
    for (int c = 0; c < 4; ++c) nv[c] = fmaf(a, st[i][c], kr * d[c]);
    __builtin_nontemporal_store(nv, reinterpret_cast<f32x4*>(S + row * DV) + c4);
  }
}

template <int DK, int DV, typename InT, bool VEC>
static hipError_t launch_decode_t(const Params& p, int64_t nheads, hipStream_t s) {
  constexpr int NT = DecodeShape<DK, DV>::NT;
  hipLaunchKernelGGL((decode_kernel<DK, DV, InT, VEC>), dim3((unsigned)(nheads * DecodeShape<DK, DV>::NSPLIT)),
                     dim3(NT), 0, s, p);
  return hipGetLastError();
}

template <int DK, int DV>
static hipError_t dispatch_gate(const Params& p, int64_t nheads, bool bf16, bool vec, hipStream_t s) {
  if (bf16) return vec ? launch_decode_t<DK, DV, __bf16, true>(p, nheads, s)
                       : launch_decode_t<DK, DV, __bf16, false>(p, nheads, s);
  return vec ? launch_decode_t<DK, DV, float, true>(p, nheads, s)
             : launch_decode_t<DK, DV, float, false>(p, nheads, s);
}

template <int DK>
static hipError_t dispatch_dv(const Params& p, int64_t nheads, int dv, bool bf16, bool vec, hipStream_t s) {
  switch (dv) {
    case 16: return dispatch_gate<DK, 16>(p, nheads, bf16, vec, s);
    case 32: return dispatch_gate<DK, 32>(p, nheads, bf16, vec, s);
    case 64: return dispatch_gate<DK, 64>(p, nheads, bf16, vec, s);
    case 128: return dispatch_gate<DK, 128>(p, nheads, bf16, vec, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const Params& p, int64_t nheads, int dk, int dv, bool bf16, bool vec,
                         hipStream_t s) {
  if (nheads == 0) return hipSuccess;
  switch (dk) {
    case 16: return dispatch_dv<16>(p, nheads, dv, bf16, vec, s);
    case 32: return dispatch_dv<32>(p, nheads, dv, bf16, vec, s);
    case 64: return dispatch_dv<64>(p, nheads, dv, bf16, vec, s);
    case 128: return dispatch_dv<128>(p, nheads, dv, bf16, vec, s);
  }
  return hipErrorInvalidValue;
}

// Two KDA transitions per token (PRODUCT2), in the same single pass over the state.
// With X = Diag(alpha) S, u_j = beta_j k_j, m_j = beta_j v_j:
//   delta_1 = m_1 - X^T u_1,            S' = X + k_1 delta_1^T
//   delta_2 = m_2 - S'^T u_2 = m_2 - X^T u_2 - (k_1 . u_2) delta_1
//   S_t = X + k_1 delta_1^T + k_2 delta_2^T
//   o = S_t^T q = X^T q + (k_1 . q) delta_1 + (k_2 . q) delta_2
// so three column reductions of S (against alpha.u_1, alpha.u_2, alpha.q) and three dot
// products of the token's vectors give everything.
template <int DK, int DV, typename InT>
__global__ __launch_bounds__((DecodeShape<DK, DV>::NT)) void decode2_kernel(const Params p) {
  using Sh = DecodeShape<DK, DV>;
  constexpr int DVS = Sh::DVS, COLS4 = Sh::COLS4, RG = Sh::RG, RPT = Sh::RPT, NT = Sh::NT;
  __shared__ float s_q[DK], s_k1[DK], s_k2[DK], s_a[DK], s_au1[DK], s_au2[DK], s_aq[DK];
  __shared__ float s_m1[DVS], s_m2[DVS];
  __shared__ float s_red[3][RG][DVS + 4];
  __shared__ float s_dot[3][RG];
  __shared__ float s_d1[DVS], s_d2[DVS];
  __shared__ float s_norm[3];

  const int tid = threadIdx.x;
  const int c4 = tid % COLS4;
  const int rg = tid / COLS4;
  const int64_t nh = blockIdx.x / Sh::NSPLIT;          // sequence * H + head
  const int col0 = (blockIdx.x % Sh::NSPLIT) * DVS;
  int64_t srow = nh;
  if (p.sidx) {
    const int64_t n = nh / p.H;
    const int32_t sl = p.sidx[n];
    if (sl < 0 || sl >= p.nslots) {
      for (int j = tid; j < DVS; j += NT) p.o[nh * DV + col0 + j] = 0.f;
      return;
    }
    srow = (int64_t)sl * p.H + (nh - n * p.H);
  }
  float* S = p.S + srow * (int64_t)DK * DV + col0;

  // token vectors first, then the state (see decode_kernel)
  const int64_t sn = nh / p.H, sh = nh - sn * p.H;  // sequence and head (inputs through their strides)
  const InT* q = static_cast<const InT*>(p.q) + sn * p.q_bs + sh * DK;
  const InT* k1 = static_cast<const InT*>(p.k) + sn * p.k_bs + (2 * sh) * DK;
  const InT* k2 = k1 + DK;
  const InT* v1 = static_cast<const InT*>(p.v) + sn * p.v_bs + (2 * sh) * DV + col0;
  const InT* v2 = v1 + DV;
  static_assert(DK <= NT && DVS <= NT, "one token element per thread");
  const bool prep = p.a_act || p.g_act || p.a_bf16;  // fused activations (uniform)
  float qi = 0.f, ai = 0.f, bi = 0.f, az = 0.f, w1 = 0.f, w2 = 0.f;
  float b1 = p.erase[2 * nh], b2 = p.erase[2 * nh + 1];
  if (tid < DK) {
    qi = ld_f32(q + tid);
    ai = ld_f32(k1 + tid);
    bi = ld_f32(k2 + tid);
    az = p.a_bf16 ? (float)static_cast<const __bf16*>(p.alpha)[nh * DK + tid]
                  : static_cast<const float*>(p.alpha)[nh * DK + tid];
  }
  if (tid < DVS) {
    w1 = ld_f32(v1 + tid);
    w2 = ld_f32(v2 + tid);
  }
  f32x4 st[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + RG * i;
    st[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + row * DV) + c4);
  }

  float nq = 1.f, nk1 = 1.f, nk2 = 1.f;
  if (p.prep_l2) {
    float sq = qi * qi, s1 = ai * ai, s2 = bi * bi;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      sq += __shfl_xor(sq, o);
      s1 += __shfl_xor(s1, o);
      s2 += __shfl_xor(s2, o);
    }
    if ((tid & 63) == 0 && tid < DK) {
      s_red[0][0][tid >> 6] = sq;
      s_red[1][0][tid >> 6] = s1;
      s_red[2][0][tid >> 6] = s2;
    }
    __syncthreads();
    if (tid == 0) {
      float tq = 0.f, t1 = 0.f, t2 = 0.f;
      for (int wv = 0; wv < (DK + 63) / 64; ++wv) {
        tq += s_red[0][0][wv];
        t1 += s_red[1][0][wv];
        t2 += s_red[2][0][wv];
      }
      s_norm[0] = tq > 0.f ? __builtin_amdgcn_rsqf(tq) : 0.f;
      s_norm[1] = t1 > 0.f ? __builtin_amdgcn_rsqf(t1) : 0.f;
      s_norm[2] = t2 > 0.f ? __builtin_amdgcn_rsqf(t2) : 0.f;
    }
    __syncthreads();
    nq = s_norm[0];
    nk1 = s_norm[1];
    nk2 = s_norm[2];
  }
  if (prep) {
    b1 = prep_gate(b1, p);
    b2 = prep_gate(b2, p);
  }
  if (tid < DK) {
    const float a = prep ? prep_alpha(az, p) : az;
    qi *= nq;
    ai *= nk1;
    bi *= nk2;
    s_q[tid] = qi;
    s_k1[tid] = ai;
    s_k2[tid] = bi;
    s_a[tid] = a;
    s_au1[tid] = a * (b1 * ai);
    s_au2[tid] = a * (b2 * bi);
    s_aq[tid] = a * qi;
  }
  if (tid < DVS) {
    s_m1[tid] = b1 * w1;
    s_m2[tid] = b2 * w2;
  }
  __syncthreads();

  float r1[4] = {0.f, 0.f, 0.f, 0.f}, r2[4] = {0.f, 0.f, 0.f, 0.f}, rq[4] = {0.f, 0.f, 0.f, 0.f};
  float d12 = 0.f, d1q = 0.f, d2q = 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + RG * i;
    const float au1 = s_au1[row], au2 = s_au2[row], aq = s_aq[row];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      r1[c] = fmaf(st[i][c], au1, r1[c]);
      r2[c] = fmaf(st[i][c], au2, r2[c]);
      rq[c] = fmaf(st[i][c], aq, rq[c]);
    }
    const float ka = s_k1[row], kb = s_k2[row], qr = s_q[row];
    d12 = fmaf(ka, b2 * kb, d12);
    d1q = fmaf(ka, qr, d1q);
    d2q = fmaf(kb, qr, d2q);
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    s_red[0][rg][4 * c4 + c] = r1[c];
    s_red[1][rg][4 * c4 + c] = r2[c];
    s_red[2][rg][4 * c4 + c] = rq[c];
  }
  if (c4 == 0) {
    s_dot[0][rg] = d12;
    s_dot[1][rg] = d1q;
    s_dot[2][rg] = d2q;
  }
  __syncthreads();

  if (tid < DVS) {
    float u1 = 0.f, u2 = 0.f, uq = 0.f, e12 = 0.f, e1q = 0.f, e2q = 0.f;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      u1 += s_red[0][g][tid];
      u2 += s_red[1][g][tid];
      uq += s_red[2][g][tid];
      e12 += s_dot[0][g];
      e1q += s_dot[1][g];
      e2q += s_dot[2][g];
    }
    const float delta1 = s_m1[tid] - u1;
    const float delta2 = s_m2[tid] - u2 - e12 * delta1;
    s_d1[tid] = delta1;
    s_d2[tid] = delta2;
    p.o[nh * DV + col0 + tid] = fmaf(e2q, delta2, fmaf(e1q, delta1, uq));
  }
  __syncthreads();

  float d1[4], d2[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    d1[c] = s_d1[4 * c4 + c];
    d2[c] = s_d2[4 * c4 + c];
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + RG * i;
    const float a = s_a[row], ka = s_k1[row], kb = s_k2[row];
    f32x4 nv;
#pragma unroll
    for (int c = 0; c < 4; ++c) nv[c] = fmaf(a, st[i][c], fmaf(ka, d1[c], kb * d2[c]));
    __builtin_nontemporal_store(nv, reinterpret_cast<f32x4*>(S + row * DV) + c4);
  }
}

template <int DK, int DV>
static hipError_t launch_decode2_t(const Params& p, int64_t nheads, bool bf16, hipStream_t s) {
  constexpr int NT = DecodeShape<DK, DV>::NT;
  const dim3 grid((unsigned)(nheads * DecodeShape<DK, DV>::NSPLIT));
  if (bf16) hipLaunchKernelGGL((decode2_kernel<DK, DV, __bf16>), grid, dim3(NT), 0, s, p);
  else hipLaunchKernelGGL((decode2_kernel<DK, DV, float>), grid, dim3(NT), 0, s, p);
  return hipGetLastError();
}

template <int DK>
static hipError_t dispatch2_dv(const Params& p, int64_t nheads, int dv, bool bf16, hipStream_t s) {
  switch (dv) {
    case 16: return launch_decode2_t<DK, 16>(p, nheads, bf16, s);
    case 32: return launch_decode2_t<DK, 32>(p, nheads, bf16, s);
    case 64: return launch_decode2_t<DK, 64>(p, nheads, bf16, s);
    case 128: return launch_decode2_t<DK, 128>(p, nheads, bf16, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode2(const Params& p, int64_t nheads, int dk, int dv, bool bf16, hipStream_t s) {
  if (nheads == 0) return hipSuccess;
  switch (dk) {
    case 16: return dispatch2_dv<16>(p, nheads, dv, bf16, s);
    case 32: return dispatch2_dv<32>(p, nheads, dv, bf16, s);
    case 64: return dispatch2_dv<64>(p, nheads, dv, bf16, s);
    case 128: return dispatch2_dv<128>(p, nheads, dv, bf16, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dr
