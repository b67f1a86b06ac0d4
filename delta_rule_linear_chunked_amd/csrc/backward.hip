// Backward pass of the gated delta rule (gradients of a prefill) on gfx950.
//
// Per token the forward step is (X = Diag(alpha_t) S_{t-1}, u and m the erase / write vectors
// of the KDA, RDA and GDN-2 rules of the Hugging Face discussion "KRAFTON/Raon-1-mini-preview"
// #1, Complex KDA with KDA's rule)
//
//   delta_t = m_t - X^T u_t,   S_t = X + k_t delta_t^T,   o_t = S_t^T q_t
//
// and, with G the gradient reaching S_t (later tokens plus q_t do_t^T),
//
//   dq_t = S_t do_t           d(delta) = G^T k_t       dk_t += G delta_t     dm_t = d(delta)
//   dX   = G - u_t d(delta)^T  du_t = -X d(delta)     dalpha_t = rowsum(dX . S_{t-1})
//   gradient reaching S_{t-1} = Diag(alpha_t) dX
//
// (the reverse of the step rule; the course page "GDN, KDA và Mamba-2", section 3, names the
// checkpoints and scan intermediates that training needs). No step divides by a gate, so
// negative and zero gates need nothing special.
//
// States for the reverse walk: the prefill stores the state after every 64 tokens
// (checkpoints); bwd_kernel walks the chunks in reverse, recomputes each chunk's states
// forward from its checkpoint keeping every 8th in LDS, and for each 8-token block
// recomputes the block's states into registers and steps backwards through them.
//
// Work split: one workgroup of 256 threads per (sequence, head, block of DVB value columns).
// Each lane owns a tile of RPL key rows x CPL value columns (4 x 4 at d = 128); the RG lanes
// of a column group are neighbours, so the sums over key rows on the recurrence's critical path
// (delta, d(delta)) are DPP steps plus one cross-row swap. The sums over value columns (dq, the
// G delta part of dk, du, dalpha) leave the recurrence: summed over the lane's columns, over
// the wave's column groups with permlane swaps, across the four waves in LDS, and written per
// column block; bwd_reduce_kernel adds the blocks and applies the erase / write chain rule.
#include "common.hpp"
#include "launch.hpp"

namespace dr {

constexpr int BW_CH = 64;   // checkpoint spacing (the prefill's chunk)
constexpr int BW_SB = 8;    // tokens per block whose states are held in registers
constexpr int BW_NSB = BW_CH / BW_SB;

// Lane tiling: lane (g, rg) owns rows rg*RPL .. +RPL-1 of columns g*CPL .. +CPL-1 of the
// block; the RG lanes of a column group are neighbours (an aligned 16 or 32 lanes).
template <int DK, int DVB>
struct BwdShape {
  static constexpr int RG = DK < 32 ? DK : 32;  // lanes per column group
  static constexpr int NCG = 256 / RG;          // column groups
  static constexpr int CPL = DVB / NCG;         // columns per lane
  static constexpr int RPL = DK / RG;           // rows per lane
  static constexpr int GPW = 64 / RG;           // column groups per wave
  static constexpr int NV = 4 * RPL;            // row-sum values per lane (4 quantities)
  static constexpr int NVR = NV / GPW;          // values per lane after the in-wave reduction
  static_assert(RG == 16 || RG == 32, "column group");
  static_assert(CPL >= 1 && NCG * CPL == DVB && RG * RPL == DK, "tiling");
  static_assert(NV % GPW == 0, "reduction split");
};

template <int DK, int DVB>
struct BwdSmem {
  float sub[BW_NSB - 1][DVB][DK];   // states at tokens 8, 16, .., 56 of the chunk: [column][row]
  float k[BW_SB][DK], u[BW_SB][DK], q[BW_SB][DK], a[BW_SB][DK];
  float m[BW_SB][DVB], dO[BW_SB][DVB], v[BW_SB][DVB], g[BW_SB][DVB];
  float red[2][4][BwdShape<DK, DVB>::RG][BwdShape<DK, DVB>::NV];  // per-wave row sums, two buffers
  float reds[2][4];                                              // v . dm per wave
};

template <int N>
__device__ __forceinline__ void lds_load(const float* src, float (&x)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(src + 4 * i);
      x[4 * i] = t[0]; x[4 * i + 1] = t[1]; x[4 * i + 2] = t[2]; x[4 * i + 3] = t[3];
    }
  } else if constexpr (N == 2) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 t = *reinterpret_cast<const f32x2*>(src);
    x[0] = t[0]; x[1] = t[1];
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = src[i];
  }
}
template <int N>
__device__ __forceinline__ void lds_store(float* dst, const float (&x)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) *reinterpret_cast<f32x4*>(dst + 4 * i) = f32x4{x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]};
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) dst[i] = x[i];
  }
}

// Cross-lane steps without the LDS crossbar: DPP within rows of 16 lanes, and gfx950's
// permlane swaps across rows.
constexpr int DPP_QUAD_XOR1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

// One butterfly step across lane bit 32 (16): a and b are two values of this lane; afterwards
// lanes without the bit hold a + a(partner) and lanes with it hold b + b(partner).
__device__ __forceinline__ float swap_add32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b),
                                                  false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float swap_add16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b),
                                                  false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Sum over the RG lanes of a column group (an aligned 16 or 32 lanes), left in every lane.
template <int RG>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_or<DPP_QUAD_XOR1>(0.f, x);
  x += dpp_or<DPP_QUAD_XOR2>(0.f, x);
  x += dpp_or<DPP_ROW_HALF_MIRROR>(0.f, x);  // the other quad of the 8
  x += dpp_or<DPP_ROW_MIRROR>(0.f, x);       // the other half of the row of 16
  if constexpr (RG == 32) x = swap_add16(x, x);  // the neighbouring row
  return x;
}

// STR: q, k, v read through the strides of p (an instance of its own: the dense one has no
// scalar registers to spare for them)
template <int DK, int DVB, typename InT, bool VEC, bool STR>
__global__ __launch_bounds__(256, 1) void bwd_kernel(const BwdParams p) {
  if (p.run_flag && *p.run_flag == 0) return;
  using Sh = BwdShape<DK, DVB>;
  constexpr int RG = Sh::RG, CPL = Sh::CPL, RPL = Sh::RPL, NV = Sh::NV, NVR = Sh::NVR;
  __shared__ __align__(16) BwdSmem<DK, DVB> sm;

  // packed sequences: the longest first, so that the last workgroups to start are short ones
  const int pair = p.seq_order ? p.seq_order[blockIdx.x / p.ndvb / p.H] * p.H + (int)(blockIdx.x / p.ndvb % p.H)
                               : (int)(blockIdx.x / p.ndvb);
  const int blk = blockIdx.x % p.ndvb;
  const int dv0 = blk * DVB;
  const int H = p.H, DV = p.DV;
  const int n = pair / H, h = pair % H;
  int64_t bos, len, snap_base;
  if (p.cu) {  // (offsets in steps)
    bos = (int64_t)p.cu[n] << p.lgnh;
    len = ((int64_t)p.cu[n + 1] << p.lgnh) - bos;
    snap_base = p.snap_first[n];
  } else {
    bos = (int64_t)n * p.T;
    len = p.T;
    snap_base = (int64_t)n * (p.T / BW_CH);
  }
  const int nch = (int)((len + BW_CH - 1) / BW_CH);
  const int tid = threadIdx.x;
  const int grp = tid / RG, rg = tid % RG;      // column group, row group
  const int col0 = grp * CPL, row0 = rg * RPL;  // first column / row of the lane's tile
  const int w = tid >> 6, lw = tid & 63;
  const InT* qp = static_cast<const InT*>(p.q);
  const InT* kp = static_cast<const InT*>(p.k);
  const InT* vp = static_cast<const InT*>(p.v);
  // element (row 0, column col0) of this (sequence, head)'s state
  const int64_t state_off = ((int64_t)n * H + h) * DK * (int64_t)DV + dv0 + col0;

  // the lane's state tile S[column][row], and the gradient reaching it
  float dS[CPL][RPL];
#pragma unroll
  for (int cc = 0; cc < CPL; ++cc) {
#pragma unroll
    for (int i = 0; i < RPL; ++i) dS[cc][i] = p.dST ? p.dST[state_off + (int64_t)(row0 + i) * DV + cc] : 0.f;
  }

  // inputs of steps t0 .. t0+7 of the sequence (past the end: zeros), as the rules use them;
  // loaded into registers one staged block ahead of use, then committed to LDS. With two
  // steps per token, q, alpha and dO come from the token's row: the decay only on its first
  // step (1 on the second), the output gradient only after its last.
  const int lastm = (1 << p.lgnh) - 1;
  auto rows = [&](int64_t m, int64_t& tq, int64_t& tk) {  // absolute step -> token / step rows
    tq = (m >> p.lgnh) * H + h;
    tk = (tq << p.lgnh) + (m & lastm);
  };
  // q, k and v through their strides: this (sequence, head)'s rows start at qh, kh, vh; step s of
  // the batch row is (s >> lgnh) token strides further (k, v: plus (s & lastm) d for the step)
  const int64_t brow = p.cu ? 0 : n, srow0 = p.cu ? bos : 0;
  const InT* qh = STR ? qp + brow * p.q_bs + (int64_t)h * DK : qp;
  const InT* kh = STR ? kp + brow * p.k_bs + ((int64_t)h << p.lgnh) * DK : kp;
  const InT* vh = STR ? vp + brow * p.v_bs + ((int64_t)h << p.lgnh) * DV + dv0 : vp;
  constexpr int SK = (BW_SB * DK + 255) / 256, SV = (BW_SB * DVB + 255) / 256;
  static_assert(SK <= 16 && SV <= 16, "flag bits");
  // Raw values as loaded, and per element bit flags (bit x: element x is inside the sequence;
  // bit 16 + x: alpha applies / the output gradient applies). Nothing reads the loaded values
  // before the block is committed, so the loads stay in flight across the steps in between.
  struct Stg {
    InT k[SK], q[SK], v[SV];
    float a[SK], ug[SK], g[SV], dO[SV];
    unsigned fk, fv;
  };
  // (the loads are unconditional, at clamped in-range indices; the flags select at commit)
  auto load_stg = [&](Stg& r, int64_t t0) {
    r.fk = 0u;
    r.fv = 0u;
#pragma unroll
    for (int x = 0; x < SK; ++x) {
      const int e0 = tid + 256 * x;
      const bool in = e0 < BW_SB * DK && t0 + e0 / DK < len;
      const int e = e0 < BW_SB * DK ? e0 : 0;
      const int j = e / DK, i = e % DK;
      const int64_t t = t0 + j < len ? t0 + j : len - 1;
      int64_t tq, tk;
      rows(bos + t, tq, tk);
      if constexpr (STR) {
        const int64_t sr = srow0 + t;
        r.k[x] = kh[(sr >> p.lgnh) * p.k_ts + (sr & lastm) * DK + i];
        r.q[x] = qh[(sr >> p.lgnh) * p.q_ts + i];
      } else {
        r.k[x] = kp[tk * DK + i];
        r.q[x] = qp[tq * DK + i];
      }
      r.a[x] = p.alpha[tq * DK + i];
      r.ug[x] = VEC ? p.erase[tk * DK + i] : p.erase[tk];
      const bool first = ((bos + t) & lastm) == 0;
      r.fk |= (in ? 1u << x : 0u) | (first ? 1u << (16 + x) : 0u);
    }
#pragma unroll
    for (int x = 0; x < SV; ++x) {
      const int e0 = tid + 256 * x;
      const bool in = e0 < BW_SB * DVB && t0 + e0 / DVB < len;
      const int e = e0 < BW_SB * DVB ? e0 : 0;
      const int j = e / DVB, cc = e % DVB;
      const int64_t t = t0 + j < len ? t0 + j : len - 1;
      int64_t tq, tk;
      rows(bos + t, tq, tk);
      if constexpr (STR) {
        const int64_t sr = srow0 + t;
        r.v[x] = vh[(sr >> p.lgnh) * p.v_ts + (sr & lastm) * DV + cc];
      } else {
        r.v[x] = vp[tk * DV + dv0 + cc];
      }
      r.g[x] = VEC ? p.write[tk * DV + dv0 + cc] : p.write[tk];
      r.dO[x] = p.dO[tq * DV + dv0 + cc];
      const bool last = ((bos + t) & lastm) == lastm;
      r.fv |= (in ? 1u << x : 0u) | (last ? 1u << (16 + x) : 0u);
    }
  };
  auto commit_stg = [&](const Stg& r) {
#pragma unroll
    for (int x = 0; x < SK; ++x) {
      const int e = tid + 256 * x;
      if (e < BW_SB * DK) {
        const int j = e / DK, i = e % DK;
        const bool in = (r.fk >> x) & 1u, first = (r.fk >> (16 + x)) & 1u;
        const float kk = (float)r.k[x];
        sm.k[j][i] = in ? kk : 0.f;
        sm.u[j][i] = in ? r.ug[x] * kk : 0.f;
        sm.q[j][i] = in ? (float)r.q[x] : 0.f;
        sm.a[j][i] = in ? (first ? r.a[x] : 1.f) : 0.f;
      }
    }
#pragma unroll
    for (int x = 0; x < SV; ++x) {
      const int e = tid + 256 * x;
      if (e < BW_SB * DVB) {
        const int j = e / DVB, cc = e % DVB;
        const bool in = (r.fv >> x) & 1u, last = (r.fv >> (16 + x)) & 1u;
        const float vv = (float)r.v[x];
        sm.m[j][cc] = in ? r.g[x] * vv : 0.f;
        sm.dO[j][cc] = in && last ? r.dO[x] : 0.f;
        sm.v[j][cc] = in ? vv : 0.f;
        sm.g[j][cc] = in ? r.g[x] : 0.f;
      }
    }
  };
  // Staged blocks, in order: for each chunk (last first) the forward blocks 0 .. nsb-2, then the
  // backward blocks nsb-1 .. 0. The cursor (pch, pi) names the block held in `pre`.
  auto nsb_of = [&](int ch) {
    const int64_t cl = len - (int64_t)ch * BW_CH < BW_CH ? len - (int64_t)ch * BW_CH : BW_CH;
    return (int)((cl + BW_SB - 1) / BW_SB);
  };
  auto block_t0 = [&](int ch, int i) -> int64_t {
    const int nb = nsb_of(ch);
    const int sb = i < nb - 1 ? i : 2 * nb - 2 - i;
    return (int64_t)ch * BW_CH + BW_SB * sb;
  };
  Stg pre;
  int pch = nch - 1, pi = 0;
  if (nch > 0) load_stg(pre, block_t0(pch, pi));
  auto stage_next = [&]() {  // commit the held block, prefetch the following one
    commit_stg(pre);
    if (pi + 1 < 2 * nsb_of(pch) - 1) {
      ++pi;
    } else {
      --pch;
      pi = 0;
    }
    // (past the last block: a harmless reload of the first, never committed)
    load_stg(pre, block_t0(pch >= 0 ? pch : 0, pch >= 0 ? pi : 0));
  };

  // one forward step of token j of the staged block: S <- X + k delta^T; delta of the lane's columns
  auto fwd = [&](float (&S)[CPL][RPL], float (&delta)[CPL], int j) {
    float a[RPL], u[RPL], k[RPL], m[CPL];
    lds_load(&sm.a[j][row0], a);
    lds_load(&sm.u[j][row0], u);
    lds_load(&sm.k[j][row0], k);
    lds_load(&sm.m[j][col0], m);
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
      float r = 0.f;
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        S[cc][i] *= a[i];
        r = fmaf(S[cc][i], u[i], r);
      }
      delta[cc] = m[cc] - group_sum<RG>(r);
    }
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
#pragma unroll
      for (int i = 0; i < RPL; ++i) S[cc][i] = fmaf(k[i], delta[cc], S[cc][i]);
    }
  };

  int buf = 0;
  for (int ch = nch - 1; ch >= 0; --ch) {
    const int64_t c0 = (int64_t)ch * BW_CH;
    const int clen = (int)(len - c0 < BW_CH ? len - c0 : BW_CH);
    const int nsb = (clen + BW_SB - 1) / BW_SB;
    // the chunk's first state: the initial state or the forward checkpoint
    float Sc[CPL][RPL];
    {
      const float* src = ch == 0 ? p.S0 : p.snap;
      const int64_t off = ch == 0 ? state_off : ((snap_base + ch - 1) * H + h) * (int64_t)DK * DV + dv0 + col0;
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) {
#pragma unroll
        for (int i = 0; i < RPL; ++i) Sc[cc][i] = src ? src[off + (int64_t)(row0 + i) * DV + cc] : 0.f;
      }
    }
    // forward through the chunk, keeping the state at every 8th token
    {
      float S[CPL][RPL], dl[CPL];
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) {
#pragma unroll
        for (int i = 0; i < RPL; ++i) S[cc][i] = Sc[cc][i];
      }
      for (int sb = 0; sb + 1 < nsb; ++sb) {
        __syncthreads();  // the staged block is free
        stage_next();     // block sb of the chunk
        __syncthreads();
#pragma unroll
        for (int j = 0; j < BW_SB; ++j) fwd(S, dl, j);
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) lds_store(&sm.sub[sb][col0 + cc][row0], S[cc]);
      }
    }
    // backward through the chunk's blocks in reverse
    for (int sb = nsb - 1; sb >= 0; --sb) {
      const int nt = clen - BW_SB * sb < BW_SB ? clen - BW_SB * sb : BW_SB;
      __syncthreads();  // the staged block and the checkpoints are written
      stage_next();     // block sb of the chunk
      __syncthreads();
      float Sb[BW_SB + 1][CPL][RPL];  // Sb[j] = state before token j of the block
      float dl[BW_SB][CPL];
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) {
        if (sb == 0) {
#pragma unroll
          for (int i = 0; i < RPL; ++i) Sb[0][cc][i] = Sc[cc][i];
        } else {
          lds_load(&sm.sub[sb - 1][col0 + cc][row0], Sb[0][cc]);
        }
      }
#pragma unroll
      for (int j = 0; j < BW_SB; ++j) {
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
#pragma unroll
          for (int i = 0; i < RPL; ++i) Sb[j + 1][cc][i] = Sb[j][cc][i];
        }
        if (j < nt) fwd(Sb[j + 1], dl[j], j);
      }
#pragma unroll
      for (int j = BW_SB - 1; j >= 0; --j) {
        if (j < nt) {
          float a[RPL], u[RPL], k[RPL], q[RPL], dO[CPL], vv[CPL], gg[CPL];
          lds_load(&sm.a[j][row0], a);
          lds_load(&sm.u[j][row0], u);
          lds_load(&sm.k[j][row0], k);
          lds_load(&sm.q[j][row0], q);
          lds_load(&sm.dO[j][col0], dO);
          lds_load(&sm.v[j][col0], vv);
          lds_load(&sm.g[j][col0], gg);
          // row sums over the lane's columns, value index = quantity * RPL + row offset
          float val[NV];
#pragma unroll
          for (int x = 0; x < NV; ++x) val[x] = 0.f;
          float ddelta[CPL];
          float vdm = 0.f;
#pragma unroll
          for (int cc = 0; cc < CPL; ++cc) {
            float G[RPL];
            float dd = 0.f;
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
              G[i] = fmaf(q[i], dO[cc], dS[cc][i]);           // + q_t do_t^T
              dd = fmaf(G[i], k[i], dd);
              val[i] = fmaf(Sb[j + 1][cc][i], dO[cc], val[i]);  // dq  = S_t do_t
              val[RPL + i] = fmaf(G[i], dl[j][cc], val[RPL + i]);  // dk += G delta_t
            }
            ddelta[cc] = group_sum<RG>(dd);
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
              const float X = a[i] * Sb[j][cc][i];
              const float dX = fmaf(-u[i], ddelta[cc], G[i]);
              val[2 * RPL + i] = fmaf(-X, ddelta[cc], val[2 * RPL + i]);     // du = -X d(delta)
              val[3 * RPL + i] = fmaf(dX, Sb[j][cc][i], val[3 * RPL + i]);   // dalpha
              dS[cc][i] = a[i] * dX;                                         // Diag(alpha) dX
            }
            vdm = fmaf(vv[cc], ddelta[cc], vdm);
          }
          const int64_t th = (bos + c0 + BW_SB * sb + j) * H + h;  // step-major row of the partial sums
          if (rg == 0) {
            int64_t tq, tk;
            rows(bos + c0 + BW_SB * sb + j, tq, tk);
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
              p.dv[tk * DV + dv0 + col0 + cc] = gg[cc] * ddelta[cc];  // m = g . v
              if constexpr (VEC) p.dwrite[tk * DV + dv0 + col0 + cc] = vv[cc] * ddelta[cc];
            }
          }
          // sums over the wave's column groups (lane bit 32, and 16 when a group is 16 lanes)
          float r1[NV / 2];
#pragma unroll
          for (int x = 0; x < NV / 2; ++x) r1[x] = swap_add32(val[x], val[x + NV / 2]);
          vdm = swap_add32(vdm, vdm);
          int base = (lw & 32) ? NV / 2 : 0;
          if constexpr (RG == 16) {
            float r2[NV / 4];
#pragma unroll
            for (int x = 0; x < NV / 4; ++x) r2[x] = swap_add16(r1[x], r1[x + NV / 4]);
            vdm = swap_add16(vdm, vdm);
            base += (lw & 16) ? NV / 4 : 0;
#pragma unroll
            for (int x = 0; x < NVR; ++x) sm.red[buf][w][rg][base + x] = r2[x];
          } else {
#pragma unroll
            for (int x = 0; x < NVR; ++x) sm.red[buf][w][rg][base + x] = r1[x];
          }
          if (lw == 0) sm.reds[buf][w] = vdm;
          __syncthreads();
          // across the four waves
#pragma unroll
          for (int x = 0; x < (RG * NV + 255) / 256; ++x) {
            const int o = tid + 256 * x;
            if (o >= RG * NV) break;
            const int org = o / NV, idx = o % NV;
            const float sum = sm.red[buf][0][org][idx] + sm.red[buf][1][org][idx] + sm.red[buf][2][org][idx] +
                              sm.red[buf][3][org][idx];
            const int qn = idx / RPL, row = org * RPL + idx % RPL;
            p.part[(((int64_t)blk * p.TH + th) * 4 + qn) * DK + row] = sum;
          }
          if (tid == 0) p.parts[(int64_t)blk * p.TH + th] = sm.reds[buf][0] + sm.reds[buf][1] + sm.reds[buf][2] + sm.reds[buf][3];
          buf ^= 1;
        }
      }
    }
  }
  if (p.dS0) {
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
#pragma unroll
      for (int i = 0; i < RPL; ++i) p.dS0[state_off + (int64_t)(row0 + i) * DV + cc] = dS[cc][i];
    }
  }
}

// Adds the column blocks' row sums and applies the erase / write chain rule:
// u = beta k (KDA, CKDA) or e k (RDA): dk += u-gate * du, d(gate) = k . du (+ v . dm for beta);
// u = b . k (GDN-2): dk += b . du, db = k . du. One wave per token-head.
// With two steps per token (the partial sums are per step), dq comes from a token's last step
// and dalpha from its first.
template <int DK, typename InT, bool VEC>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const BwdParams p) {
  if (p.run_flag && *p.run_flag == 0) return;
  const int64_t th = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // step-major row
  const int lw = threadIdx.x & 63;
  if (th >= p.TH) return;
  const int lastm = (1 << p.lgnh) - 1;
  const int64_t m = th / p.H, hh = th - m * p.H;
  const int64_t tq = (m >> p.lgnh) * p.H + hh, tk = (tq << p.lgnh) + (m & lastm);
  const bool first = (m & lastm) == 0, last = (m & lastm) == lastm;
  const InT* kp = static_cast<const InT*>(p.k);
  // k of this step through its strides (fixed length: batch row m / T, step m % T)
  const int64_t brow = p.cu ? 0 : m / p.T;
  const int64_t ko = kv_elem(p.k_ts, p.k_bs, p, brow, m - brow * p.T, (int)hh, DK);
  float kdu = 0.f;
  for (int i = lw; i < DK; i += 64) {
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    for (int b = 0; b < p.ndvb; ++b) {
#pragma unroll
      for (int qn = 0; qn < 4; ++qn) s[qn] += p.part[(((int64_t)b * p.TH + th) * 4 + qn) * DK + i];
    }
    const float kk = ld_f32(kp + ko + i);
    const float ug = VEC ? p.erase[tk * DK + i] : p.erase[tk];
    if (last) p.dq[tq * DK + i] = s[0];
    p.dk[tk * DK + i] = fmaf(ug, s[2], s[1]);
    if (first) p.dalpha[tq * DK + i] = s[3];
    if constexpr (VEC) p.derase[tk * DK + i] = kk * s[2];
    kdu = fmaf(kk, s[2], kdu);
  }
  if constexpr (!VEC) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) kdu += __shfl_xor(kdu, o);
    if (lw == 0) {
      float vdm = 0.f;
      for (int b = 0; b < p.ndvb; ++b) vdm += p.parts[(int64_t)b * p.TH + th];
      if (p.variant == 1) {  // RDA: e k and w v are separate gates
        p.derase[tk] = kdu;
        p.dwrite[tk] = vdm;
      } else {               // KDA / CKDA / two transitions: beta is both
        p.derase[tk] = kdu + vdm;
      }
    }
  }
}

template <int DK, int DVB, typename InT, bool VEC>
static hipError_t launch_bwd_t(const BwdParams& p, int64_t pairs, hipStream_t s) {
  if (pairs > 0) {
    if (p.strided)
      hipLaunchKernelGGL((bwd_kernel<DK, DVB, InT, VEC, true>), dim3((unsigned)(pairs * p.ndvb)), dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((bwd_kernel<DK, DVB, InT, VEC, false>), dim3((unsigned)(pairs * p.ndvb)), dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.TH > 0)
    hipLaunchKernelGGL((bwd_reduce_kernel<DK, InT, VEC>), dim3((unsigned)((p.TH + 3) / 4)), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int DK, int DVB>
static hipError_t launch_bwd_g(const BwdParams& p, int64_t pairs, bool bf16, bool vec, hipStream_t s) {
  if (bf16) return vec ? launch_bwd_t<DK, DVB, __bf16, true>(p, pairs, s) : launch_bwd_t<DK, DVB, __bf16, false>(p, pairs, s);
  return vec ? launch_bwd_t<DK, DVB, float, true>(p, pairs, s) : launch_bwd_t<DK, DVB, float, false>(p, pairs, s);
}

template <int DK>
static hipError_t launch_bwd_dk(const BwdParams& p, int64_t pairs, int dvb, bool bf16, bool vec, hipStream_t s) {
  return dvb == 32 ? launch_bwd_g<DK, 32>(p, pairs, bf16, vec, s) : launch_bwd_g<DK, 16>(p, pairs, bf16, vec, s);
}

hipError_t launch_backward(BwdParams p, int64_t pairs, int dk, int dv, bool bf16, bool vec, hipStream_t s) {
  const int dvb = bwd_dv_block(dv);
  p.ndvb = dv / dvb;
  switch (dk) {
    case 16: return launch_bwd_dk<16>(p, pairs, dvb, bf16, vec, s);
    case 32: return launch_bwd_dk<32>(p, pairs, dvb, bf16, vec, s);
    case 64: return launch_bwd_dk<64>(p, pairs, dvb, bf16, vec, s);
    case 128: return launch_bwd_dk<128>(p, pairs, dvb, bf16, vec, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dr
