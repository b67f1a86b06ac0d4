// Sequential state pass of the chunkwise prefill on gfx950 (the second of the two passes
// described at the top of prefill.hip): one workgroup per (sequence, head, block of value
// columns) walks the sequence's chunks in order with the fp32 state in registers, reading the
// operand records that chunk_prep_kernel wrote, and produces the outputs, the final state and
// any snapshots. It is a compilation unit of its own so that it can be built with its own
// scheduling options.
#include <type_traits>

#include "prefill.hpp"

namespace dr {

// ============================================================================ pass 2
// Split-operand tile in LDS: a row-major matrix whose fragments are 8 consecutive
// columns of a row (the reduction index), written 4 columns at a time from an
// accumulator.
template <class Pol, int ROWS, int COLS> struct OpTile;
template <int ROWS, int COLS> struct OpTile<PolBF3, ROWS, COLS> {
  __bf16 hi[ROWS][COLS + 8], lo[ROWS][COLS + 8];
  __device__ __forceinline__ void put4(int row, int col, const f32x4& x) {
    uint32_t h[2], o[2];
    split2(x[0], x[1], h[0], o[0]);
    split2(x[2], x[3], h[1], o[1]);
    *reinterpret_cast<bf16x4*>(&hi[row][col]) = __builtin_bit_cast(bf16x4, h);
    *reinterpret_cast<bf16x4*>(&lo[row][col]) = __builtin_bit_cast(bf16x4, o);
  }
  __device__ __forceinline__ PolBF3::Frag get8(int row, int col) const {
    PolBF3::Frag f;
    f.hi = *reinterpret_cast<const bf16x8*>(&hi[row][col]);
    f.lo = *reinterpret_cast<const bf16x8*>(&lo[row][col]);
    return f;
  }
};
template <int ROWS, int COLS> struct OpTile<PolF32, ROWS, COLS> {
  float v[ROWS][COLS + 4];
  __device__ __forceinline__ void put4(int row, int col, const f32x4& x) { store4(&v[row][col], x); }
  __device__ __forceinline__ PolF32::Frag get8(int row, int col) const {
    PolF32::Frag f;
    load8(&v[row][col], f.v);
    return f;
  }
};

template <class Pol, int DK, int DVB>
struct StateSmem {
  OpTile<Pol, DVB, DK> S;   // state, transposed: [value column][key channel]
  OpTile<Pol, DVB, CH> R;   // (M - Utilde S0)^T: [value column][token]
  OpTile<Pol, DVB, CH> D;   // delta^T
  float X[NBLK][16][DVB + 4];  // per wave: m = w . v in, then O out, between row and accumulator layouts
};

// OUT = false (no output requested): the Qtilde S0 and P delta products and the Qtilde / P loads
// are left out, and only the states are produced.
// OCC: workgroups per CU the registers are sized for (2 only for launches with more workgroups
// than CUs, where a second resident workgroup's chain fills the first one's waits).
template <int DKR, int DVB, typename InT, bool VEC, bool OUT, int OCC = 1>
__global__ __launch_bounds__(256, OCC) void chunk_state_kernel(const Params p) {
  using Pol = typename PolicyFor<InT>::type;
  using Frag = typename Pol::Frag;
  constexpr int DK = DKR < 32 ? 32 : DKR;
  constexpr int KS = DK / 32;
  constexpr int NCT = DVB / 16;
  constexpr int NRT = (DK / 16 + 3) / 4;  // key-channel tiles per wave (rounded up)
  using R = Rec<DK>;
  static_assert(DVB % 16 == 0 && DVB <= 64, "value block");

  __shared__ __align__(16) StateSmem<Pol, DK, DVB> sm;

  const int H = p.H;
  int pair, dv0;
  if (p.cu) {
    // packed sequences: the (sequence, head) pairs in order of decreasing length, dealt
    // round-robin over the XCDs (workgroup b runs on XCD b % 8), each XCD taking its pairs
    // longest first; the value-column blocks of a pair stay on one XCD and share its L2.
    // (In sequence order each XCD took a contiguous range of pairs, and with uneven lengths
    // one XCD held the longest chains back to back.)
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int k = (j / p.ndvb) * 8 + x;
    if (k >= p.num_pairs) return;
    pair = p.seq_order[k / H] * H + k % H;
    dv0 = (j % p.ndvb) * DVB;
  } else {
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    if (lid >= p.grid_logical) return;
    pair = lid / p.ndvb;
    dv0 = (lid % p.ndvb) * DVB;
  }
  const int n = pair / H, h = pair % H;
  int64_t bos, len;
  int first;
  if (p.cu) {
    bos = cu_steps(p, n);
    len = cu_steps(p, n + 1) - bos;
    first = p.seq_first[n];
  } else {  // this window's chunks win_c0 .. sit at record slots n * win_k + (c - win_c0)
    bos = (int64_t)n * p.T;
    len = p.T;
    first = n * p.win_k - p.win_c0;
  }
  const int nch = (int)((len + CH - 1) / CH);
  // the chunks this launch covers: all of them (packed sequences), or the window's
  const int cbeg = p.cu ? 0 : p.win_c0;
  const int cend = p.cu ? nch : (p.win_c0 + p.win_nc < nch ? p.win_c0 + p.win_nc : nch);
  // state slot: row n of S0 / S_T, or state_idx[n] of a pool (outside the pool: start from
  // zero and store no final state)
  int64_t srow = n;
  bool has_row = true;
  if (p.sidx) {
    const int32_t sl = p.sidx[n];
    has_row = sl >= 0 && sl < p.nslots;
    srow = sl;
  }
  const int64_t snap_base = !p.snap ? 0 : p.cu ? (int64_t)p.snap_first[n] : (int64_t)n * (p.T / (p.snap_chunks * CH));
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, r = l & 15, g = l >> 4;
  const int DV = p.DV;
  const InT* vp = static_cast<const InT*>(p.v);

  // ---- state: fp32 master in registers (this wave's key-channel tiles), split copy in LDS
  f32x4 Sm[NRT][NCT];
#pragma unroll
  for (int m = 0; m < NRT; ++m) {
    const int rt = w + 4 * m;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
      if (rt < DK / 16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ch = 16 * rt + 4 * g + i;
          if (ch < DKR) {
            if (p.carry_in) x[i] = p.carry[(((int64_t)n * H + h) * DKR + ch) * DV + dv0 + 16 * ct + r];
            else if (p.S0 && has_row) x[i] = p.S0[((srow * H + h) * DKR + ch) * DV + dv0 + 16 * ct + r];
          }
        }
        sm.S.put4(16 * ct + r, 16 * rt + 4 * g, x);
      }
      Sm[m][ct] = x;
    }
  }

  // ---- operands of a chunk, in registers: one set, each group of fragments loaded again for
  // chunk c + 1 right after its last use in chunk c, so every load has most of a chunk to
  // arrive and the load path works in parallel with the MFMAs (past the last chunk the last
  // record is reloaded and unused). A second, alternating set measured no faster and took 160
  // more registers.
  // v and the write gate move as row segments: lane l holds token 16w + l/4 of the wave's
  // block, value columns (l % 4) * E .. + E - 1 of the block, with 16-byte accesses.
  constexpr int E = DVB / 4;
  typedef InT RowV __attribute__((ext_vector_type(E)));
  typedef float RowF __attribute__((ext_vector_type(E)));
  using WRow = typename std::conditional<VEC, RowF, float>::type;
  const int lr = l >> 2, lc = (l & 3) * E;
  struct Ops {
    Frag fU[KS], fQ[KS], fT[2], fP[2], fK[NRT][2];
    f32x4 gC[NRT];
    RowV pv;
    WRow pw;
  };
  auto rec_ptr = [&](int c) -> __amdgpu_buffer_rsrc_t {
    const int cc = c < cend ? c : cend - 1;
    return rec_rsrc(p.rec + ((int64_t)h * p.slots + first + cc) * p.rec_size, p.rec_size);
  };
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the wave index, as a uniform value
  auto load_uq = [&](Ops& op, __amdgpu_buffer_rsrc_t rc, int ks) {
    op.fU[ks] = ld_frag<Frag>(rc, R::UT, wu * KS + ks, l);
    if constexpr (OUT) op.fQ[ks] = ld_frag<Frag>(rc, R::QT, wu * KS + ks, l);
  };
  // T and P rows of block w are zero past token 16w + 15: only (w + 2) / 2 steps are loaded
  auto load_tp = [&](Ops& op, __amdgpu_buffer_rsrc_t rc) {
    op.fT[0] = ld_frag<Frag>(rc, R::TT, wu * 2, l);
    if constexpr (OUT) op.fP[0] = ld_frag<Frag>(rc, R::PP, wu * 2, l);
    if (w >= 2) {
      op.fT[1] = ld_frag<Frag>(rc, R::TT, wu * 2 + 1, l);
      if constexpr (OUT) op.fP[1] = ld_frag<Frag>(rc, R::PP, wu * 2 + 1, l);
    }
  };
  auto load_k = [&](Ops& op, __amdgpu_buffer_rsrc_t rc, int m) {
    const int rt = wu + 4 * m < DK / 16 ? wu + 4 * m : 0;
#pragma unroll
    for (int st = 0; st < 2; ++st) op.fK[m][st] = ld_frag<Frag>(rc, R::KB, rt * 2 + st, l);
    const u32x4 gc = __builtin_amdgcn_raw_buffer_load_b128(rc, 16 * g, R::GC + 64 * rt, 0);
    op.gC[m] = *reinterpret_cast<const f32x4*>(&gc);
  };
  auto load_vw = [&](Ops& op, int c) {
    const int cc = c < cend ? c : cend - 1;
    const int64_t last = bos + len - 1;
    int64_t tv = bos + (int64_t)cc * CH + 16 * w + lr;
    tv = tv > last ? last : tv;
    const int64_t thv = step_row(p, tv, h);
    const int64_t vo = kv_elem(p.v_ts, p.v_bs, p, p.cu ? 0 : n, p.cu ? tv : tv - bos, h, DV);
    op.pv = *reinterpret_cast<const RowV*>(vp + vo + dv0 + lc);
    if constexpr (VEC) op.pw = *reinterpret_cast<const RowF*>(p.write + thv * DV + dv0 + lc);
    else op.pw = p.write[thv];
  };
  // The first chunk's operands, in the order a chunk reloads them (v and write gate first), so
  // that the waits in the chunk loop, which serve both the first chunk and the later ones,
  // count the same loads in flight on both paths into the loop.
  auto load_ops = [&](Ops& op, int c) {
    const __amdgpu_buffer_rsrc_t rc = rec_ptr(c);
    load_vw(op, c);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) load_uq(op, rc, ks);
    load_tp(op, rc);
#pragma unroll
    for (int m = 0; m < NRT; ++m) load_k(op, rc, m);
  };

  // this workgroup's block of the fp32 state (key rows x DVB value columns) to a
  // [d_k, d_v] state at `dst`
  auto store_state = [&](float* dst) {
#pragma unroll
    for (int m = 0; m < NRT; ++m) {
      const int rt = w + 4 * m;
      if (rt < DK / 16) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int ch = 16 * rt + 4 * g + i;
            if (ch < DKR) dst[(int64_t)ch * DV + dv0 + 16 * ct + r] = Sm[m][ct][i];
          }
        }
      }
    }
  };

  auto chunk = [&](int c, Ops& cur) {
    const int64_t c0 = (int64_t)c * CH;
    // write values m = w . v (zero past the sequence end), row layout -> LDS -> rows 4g+i of
    // the accumulator layout
    {
      const bool vi = c0 + 16 * w + lr < len;
      auto put_m = [&](auto gate) {
#pragma unroll
        for (int j4 = 0; j4 < E / 4; ++j4) {
          f32x4 x;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            float wg;
            if constexpr (VEC) wg = cur.pw[4 * j4 + u];
            else wg = cur.pw;
            x[u] = vi ? gate(wg) * (float)cur.pv[4 * j4 + u] : 0.f;
          }
          store4(&sm.X[w][lr][lc + 4 * j4], x);
        }
      };
      if (p.g_act) put_m([&](float z) { return prep_gate(z, p); });  // fused gate activation
      else put_m([](float z) { return z; });
    }
    wave_lds_sync();
    float mv[NCT][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) mv[ct][i] = sm.X[w][4 * g + i][16 * ct + r];
    }
    // from here on each operand group is reloaded for chunk c + 1 as soon as chunk c is done with it
    const __amdgpu_buffer_rsrc_t rn = rec_ptr(c + 1);
    load_vw(cur, c + 1);

    // ================= X = Utilde S0, Y = Qtilde S0, R = M - X   (block row w)
    f32x4 accY[NCT];
    {
      f32x4 accX[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) { accX[ct] = f32x4{0.f, 0.f, 0.f, 0.f}; accY[ct] = accX[ct]; }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const Frag B = sm.S.get8(16 * ct + r, 32 * ks + 8 * g);
          Pol::mma(accX[ct], cur.fU[ks], B);
          if constexpr (OUT) Pol::mma(accY[ct], cur.fQ[ks], B);
        }
        load_uq(cur, rn, ks);  // this slice's Utilde / Qtilde of the next chunk
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 rv;
#pragma unroll
        for (int i = 0; i < 4; ++i) rv[i] = mv[ct][i] - accX[ct][i];
        sm.R.put4(16 * ct + r, 16 * w + 4 * g, rv);
      }
    }
    __syncthreads();

    // ================= delta = T R   (block row w)
    const int nst = (w + 2) / 2;
    {
      f32x4 accD[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) accD[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if (st < nst) {
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) Pol::mma(accD[ct], cur.fT[st], sm.R.get8(16 * ct + r, 32 * st + 8 * g));
        }
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) sm.D.put4(16 * ct + r, 16 * w + 4 * g, accD[ct]);
      // T of the next chunk (P is reloaded after its last use below)
      cur.fT[0] = ld_frag<Frag>(rn, R::TT, wu * 2, l);
      if (w >= 2) cur.fT[1] = ld_frag<Frag>(rn, R::TT, wu * 2 + 1, l);
    }
    __syncthreads();

    // ================= O = Y + P delta, and S <- Diag(Gamma_C) S0 + Kbar^T delta
    {
      Frag DF[NCT][2];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
        for (int st = 0; st < 2; ++st) DF[ct][st] = sm.D.get8(16 * ct + r, 32 * st + 8 * g);
      }
      if constexpr (OUT) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          if (st < nst) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) Pol::mma(accY[ct], cur.fP[st], DF[ct][st]);
          }
        }
      }
      if constexpr (OUT) {
        cur.fP[0] = ld_frag<Frag>(rn, R::PP, wu * 2, l);
        if (w >= 2) cur.fP[1] = ld_frag<Frag>(rn, R::PP, wu * 2 + 1, l);
      }
      // S <- Diag(Gamma_C) S0 + Kbar^T delta (the sequential chain) issued first ...
      f32x4 accS[NRT][NCT];
#pragma unroll
      for (int m = 0; m < NRT; ++m) {
        const int rt = w + 4 * m;
        if (rt < DK / 16) {
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
            for (int i = 0; i < 4; ++i) accS[m][ct][i] = cur.gC[m][i] * Sm[m][ct][i];
#pragma unroll
            for (int st = 0; st < 2; ++st) Pol::mma(accS[m][ct], cur.fK[m][st], DF[ct][st]);
          }
        }
      }
      // the next chunk's Kbar and Gamma_C, after their last use
#pragma unroll
      for (int m = 0; m < NRT; ++m) load_k(cur, rn, m);
      // ... and O written while those MFMAs run: accumulator layout -> LDS -> row segments
      if constexpr (OUT) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
          for (int i = 0; i < 4; ++i) sm.X[w][4 * g + i][16 * ct + r] = accY[ct][i];
        }
        wave_lds_sync();
        const int64_t rw = c0 + 16 * w + lr;
        const int lastm = (1 << p.lgnh) - 1;
        if (p.o && rw < len && ((bos + rw) & lastm) == lastm) {
          // lane (row, q) stores columns 16 j + 4 q .. + 3: each store of the wave covers 64
          // contiguous bytes of every row it touches
          float* orow = p.o + tok_row(p, bos + rw, h) * DV + dv0 + 4 * (l & 3);
#pragma unroll
          for (int j4 = 0; j4 < E / 4; ++j4)
            __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(&sm.X[w][lr][16 * j4 + 4 * (l & 3)]),
                                        reinterpret_cast<f32x4*>(orow + 16 * j4));
        }
      }
#pragma unroll
      for (int m = 0; m < NRT; ++m) {
        const int rt = w + 4 * m;
        if (rt < DK / 16) {
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            Sm[m][ct] = accS[m][ct];
            sm.S.put4(16 * ct + r, 16 * rt + 4 * g, accS[m][ct]);
          }
        }
      }
    }
    // snapshot: the state after (c + 1) * 64 tokens, when that is a multiple of the stride
    // and still inside the sequence
    if (p.snap && (c + 1) % p.snap_chunks == 0 && (int64_t)(c + 1) * CH <= len)
      store_state(p.snap + ((snap_base + (c + 1) / p.snap_chunks - 1) * H + h) * DKR * DV);
    __syncthreads();
  };

  Ops op;
  if (cend > cbeg) load_ops(op, cbeg);
  __syncthreads();
  for (int c = cbeg; c < cend; ++c) chunk(c, op);

  // ---- the state for the next window, or the final state
  if (p.carry_out) store_state(p.carry + ((int64_t)n * H + h) * DKR * DV);
  else if (p.S && has_row) store_state(p.S + (srow * H + h) * DKR * DV);
}

// ============================================================================ host
template <int DKR, int DVB, typename InT, bool VEC>
static hipError_t launch_state_t(const Params& p, int64_t workgroups, hipStream_t s) {
  // d_k = 128 with 32-column blocks and more workgroups than the 256 CUs of an MI355X (e.g. packed
  // sequences x heads x blocks): two resident workgroups per CU (RDA / GDN-2 varlen 2.5% faster;
  // with one workgroup per CU the one-per-CU instance is faster)
  if constexpr (DKR == 128 && DVB == 32) {
    if (workgroups > 256) {
      if (p.o)
        hipLaunchKernelGGL((chunk_state_kernel<DKR, DVB, InT, VEC, true, 2>), dim3((unsigned)workgroups), dim3(256), 0,
                           s, p);
      else
        hipLaunchKernelGGL((chunk_state_kernel<DKR, DVB, InT, VEC, false, 2>), dim3((unsigned)workgroups), dim3(256), 0,
                           s, p);
      return hipGetLastError();
    }
  }
  if (p.o)
    hipLaunchKernelGGL((chunk_state_kernel<DKR, DVB, InT, VEC, true>), dim3((unsigned)workgroups), dim3(256), 0, s, p);
  else  // states (and snapshots) only
    hipLaunchKernelGGL((chunk_state_kernel<DKR, DVB, InT, VEC, false>), dim3((unsigned)workgroups), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int DKR, int DVB>
static hipError_t launch_state_gate(const Params& p, int64_t wg, bool bf16, bool vec, hipStream_t s) {
  if (bf16) return vec ? launch_state_t<DKR, DVB, __bf16, true>(p, wg, s) : launch_state_t<DKR, DVB, __bf16, false>(p, wg, s);
  return vec ? launch_state_t<DKR, DVB, float, true>(p, wg, s) : launch_state_t<DKR, DVB, float, false>(p, wg, s);
}

template <int DKR>
static hipError_t launch_state_dvb(const Params& p, int64_t wg, int dvb, bool bf16, bool vec, hipStream_t s) {
  if (dvb == 64) return launch_state_gate<DKR, 64>(p, wg, bf16, vec, s);
  if (dvb == 32) return launch_state_gate<DKR, 32>(p, wg, bf16, vec, s);
  return launch_state_gate<DKR, 16>(p, wg, bf16, vec, s);
}

hipError_t launch_state_pass(const Params& p, int64_t workgroups, int dk, int dvb, bool bf16, bool vec,
                             hipStream_t s) {
  switch (dk) {
    case 16: return launch_state_dvb<16>(p, workgroups, dvb, bf16, vec, s);
    case 32: return launch_state_dvb<32>(p, workgroups, dvb, bf16, vec, s);
    case 64: return launch_state_dvb<64>(p, workgroups, dvb, bf16, vec, s);
    case 128: return launch_state_dvb<128>(p, workgroups, dvb, bf16, vec, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dr
