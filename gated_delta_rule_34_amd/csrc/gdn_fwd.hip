// gdn_fwd.hip -- chunked forward of the gated delta rule on gfx950.
//
// Chunk form (derived from the per-token recurrence of the lattice-inference
// gdn_backward.rs page, "Forward recap"; the pages print no chunk algebra). Within a
// chunk of n <= C tokens starting from state S:
//   gamma = cumsum(log g),  b = exp(gamma),  Gamma_rs = exp(gamma_r - gamma_s) [r >= s]
//   L = strictly_lower(diag(beta) (Gamma o K K^T)),  T = (I + L)^-1
//   Delta = T diag(beta) (V - diag(b) K S)       (Delta_r = delta_r of the recurrence)
//   O = scale (diag(b) Q S + M Delta),  M = Gamma o Q K^T (lower incl. diagonal)
//   S_next = b_n S + K^T diag(e) Delta,  e = exp(gamma_n - gamma)
// Rows past the end of a partial chunk carry k = q = v = beta = 0 and log g = 0.
//
// Two kernels after the chunk table:
//  k_prep (chunk x key head, 4 waves): K K^T and Q K^T once for the r value heads of the
//      key head; per value head the gate record (gamma in log2 units, so that every decay
//      factor is one native exp2, and beta), M and the blocked inverse
//      T, each written once in the storage type. Nothing else is materialised: the sweep
//      forms W S as T diag(beta b) (K S) and U as T diag(beta) V itself.
//  k_fwd_sweep (sequence x value head, one wave per 32 state columns): the chunk-serial
//      pass. Columns of S never mix, so each wave owns a column slice of the state in
//      float32 MFMA accumulators and K S, Delta and O never leave its registers: the
//      accumulator of one product is the operand of the next (ACC order). K, Q, V, T, M
//      and the gate record of the next chunk stream into a second LDS buffer by direct
//      loads while the current chunk is computed.
#include "gdn_common.h"

namespace gdn {

constexpr int kPrepWaves = 4;
// The lower 16 x 16 tiles (i, j) of L and M that prep's wave w forms at C = 64, dealt 3, 3,
// 2, 2 (by row tile, 1, 2, 3, 4 per wave: the wave with four held up the barrier behind it)
constexpr int kLmN[4] = {3, 3, 2, 2};
constexpr int kLmI[4][3] = {{0, 1, 1}, {2, 2, 2}, {3, 3, 3}, {3, 3, 3}};
constexpr int kLmJ[4][3] = {{0, 0, 1}, {0, 1, 2}, {0, 1, 1}, {2, 3, 3}};
constexpr int kPrepThreads = kPrepWaves * 64;

// Four accumulator values as consecutive elements of type OT (8 or 16 bytes).
template <typename OT> __device__ __forceinline__ void store4(OT* dst, f32x4 x) {
  if constexpr (sizeof(OT) == 2)
    *reinterpret_cast<bf16x4*>(dst) = bf16x4{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
  else
    *reinterpret_cast<f32x4*>(dst) = x;
}

// Row i and first column j0 of piece q (EPC elements) of a C x C matrix in lower-block
// form: the pieces of a row are consecutive and rows follow one another, so piece q starts
// at element q EPC.
template <int C, int EPC> __device__ __forceinline__ void low_piece(int q, int& i, int& j0) {
  int t = 0;  // row tile
#pragma unroll
  for (int k = 1; k < C / 16; ++k) t += q * EPC >= low_row_off(16 * k) ? 1 : 0;
  const int rl = low_row_len(16 * t) / EPC, qq = q - low_row_off(16 * t) / EPC;
  i = 16 * t + qq / rl;
  j0 = (qq % rl) * EPC;
}

// T := (I + L)^-1 for strictly lower triangular L (float32 LDS, row stride LC), lower
// blocks only: the 16 x 16 blocks above the diagonal are zero and are never written (the
// caller stores zeros for them). Diagonal blocks by forward substitution in one wave (a
// group of 16 lanes per block, one column per lane), then the blocks below the diagonal
// with float32 MFMA, T_ij = -T_ii (sum_{k=j}^{i-1} L_ik T_kj): each sum stays in the
// accumulator and is the B operand of the product with the diagonal block (ACC order).
// With four blocks (C = 64) as a 2 x 2 block inverse of 32 x 32 halves A and B: first the
// halves' own off-diagonal blocks T_10 and T_32, then T_BA = -T_BB (L_BA T_AA), one block
// per wave, the L_B0 T_00 terms formed during the first stage by the waves it leaves
// idle: 24 MFMAs on the longest wave and two barriers, against 36 and three level by level
// (prep 0.0825 -> 0.0802 ms). Otherwise level by level, one barrier per level. Ends with a
// barrier.
template <int C, int LC, int NWV>
__device__ __forceinline__ void invert_unit_lower(const float* L, float* T) {
  constexpr int NB = C / 16;
  static_assert(NWV >= NB && NB <= 4, "one wave per off-diagonal block, one lane group per diagonal block");
  const int w = threadIdx.x / 64, l = threadIdx.x & 63, g = l >> 4, r = l & 15;
  if (w == 0 && g < NB) {  // wave 0: lane group g substitutes in diagonal block g, lane r owns column r
    const int o = g * 16, j = r;
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = i == j ? 1.f : 0.f;
#pragma unroll
      for (int k = 0; k < i; ++k) s -= L[(o + i) * LC + o + k] * t[k];
      t[i] = s;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) T[(o + i) * LC + o + j] = t[i];
  }
  lds_barrier();
  if constexpr (NB == 4) {
    // X += L_{bi,kb} T_{kb,bj} (four f32 MFMAs); lane (g, r) holds X[4 g + e][r]
    auto lt = [&](f32x4& x, int bi, int kb, int bj) {
#pragma unroll
      for (int k0 = 0; k0 < 16; k0 += 4)
        x = __builtin_amdgcn_mfma_f32_16x16x4f32(L[(bi * 16 + r) * LC + kb * 16 + k0 + g],
                                                 T[(kb * 16 + k0 + g) * LC + bj * 16 + r], x, 0, 0, 0);
    };
    // Y += T_{bi,mb} X with X in accumulator order (contraction index 4 g + s at step s)
    auto tx = [&](f32x4& y, int bi, int mb, const f32x4& x) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        y = __builtin_amdgcn_mfma_f32_16x16x4f32(T[(bi * 16 + r) * LC + mb * 16 + 4 * g + s], x[s], y, 0, 0, 0);
    };
    auto put = [&](int bi, int bj, const f32x4& y) {
#pragma unroll
      for (int e = 0; e < 4; ++e) T[(bi * 16 + 4 * g + e) * LC + bj * 16 + r] = -y[e];
    };
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    f32x4 p20 = z, p30 = z;  // L_20 T_00 (waves 2, 3) and L_30 T_00 (wave 3)
    if (w < 2) {  // T_10 = -T_11 L_10 T_00 (wave 0), T_32 = -T_33 L_32 T_22 (wave 1)
      const int b0 = 2 * w;
      f32x4 x = z, y = z;
      lt(x, b0 + 1, b0, b0);
      tx(y, b0 + 1, b0 + 1, x);
      put(b0 + 1, b0, y);
    } else {
      lt(p20, 2, 0, 0);
      if (w == 3) lt(p30, 3, 0, 0);
    }
    lds_barrier();
    f32x4 y = z;
    if (w == 0) {  // T_21 = -T_22 X_21, X_21 = L_21 T_11
      f32x4 x = z;
      lt(x, 2, 1, 1);
      tx(y, 2, 2, x);
      put(2, 1, y);
    } else if (w == 1) {  // T_31 = -(T_32 X_21 + T_33 X_31), X_31 = L_31 T_11
      f32x4 x2 = z, x3 = z;
      lt(x2, 2, 1, 1);
      lt(x3, 3, 1, 1);
      tx(y, 3, 2, x2);
      tx(y, 3, 3, x3);
      put(3, 1, y);
    } else if (w == 2) {  // T_20 = -T_22 X_20, X_20 = L_20 T_00 + L_21 T_10
      lt(p20, 2, 1, 0);
      tx(y, 2, 2, p20);
      put(2, 0, y);
    } else {  // T_30 = -(T_32 X_20 + T_33 X_30), X_30 = L_30 T_00 + L_31 T_10
      lt(p20, 2, 1, 0);
      lt(p30, 3, 1, 0);
      tx(y, 3, 2, p20);
      tx(y, 3, 3, p30);
      put(3, 0, y);
    }
    lds_barrier();
    return;
  }
  for (int d = 1; d < NB; ++d) {
    const int bi = w + d, bj = w;  // wave w < NB - d owns block (w + d, w)
    if (w < NB - d) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};  // X = sum_k L_{bi,k} T_{k,bj}
      for (int kb = bj; kb < bi; ++kb)
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) {
          const float a = L[(bi * 16 + r) * LC + kb * 16 + k0 + g];
          const float b = T[(kb * 16 + k0 + g) * LC + bj * 16 + r];
          x = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, x, 0, 0, 0);
        }
      // T_{bi,bj} = -T_{bi,bi} X, contraction index k = 4 g + s at step s: lane (g, r)
      // holds X[4 g + e][r], i.e. the B operand of step s is its element e = s
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        y = __builtin_amdgcn_mfma_f32_16x16x4f32(T[(bi * 16 + r) * LC + bi * 16 + 4 * g + s], x[s], y, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) T[(bi * 16 + 4 * g + e) * LC + bj * 16 + r] = -y[e];
    }
    lds_barrier();
  }
}

// Grid nc_max * Hk, key head fastest (as the gradient kernel): workgroup c Hk + kh.
// At least four waves per SIMD (registers for four workgroups per CU): the kernel is
// latency-bound (triangular solves, barriers), and four workgroups per CU measured 12%
// faster than three.
template <typename TI, int C, int D>
__global__ __launch_bounds__(kPrepThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void k_prep(Prob p) {
  using OT = TI;
  using LD = Swz<OT, D>;
  constexpr int NW = kPrepWaves, NT = kPrepThreads, LCF = C + 4, RT = C / 16;
  constexpr int KSD = ks_of<OT, D>();
  // K and Q (direct loads) for the Gram products; afterwards the same bytes hold L and T,
  // and before T the staging tile of M (so that four workgroups fit in a CU's LDS).
  constexpr int KQ_BYTES = 2 * C * D * (int)sizeof(OT);
  constexpr int INV_BYTES = 2 * C * LCF * 4;
  static_assert(C * C * (int)sizeof(OT) <= C * LCF * 4, "M staging fits in T");
  constexpr int SM_BYTES = KQ_BYTES > INV_BYTES ? KQ_BYTES : INV_BYTES;
  // (workgroup 0 first uses it as the chunk table's scratch)
  __shared__ __align__(16) char smem[SM_BYTES > kOrderMax * 4 ? SM_BYTES : kOrderMax * 4];
  constexpr int GH = NW;  // gate records formed per pass: one wave per value head
  __shared__ __align__(16) float sg[GH][C], sbeta[GH][C];
  OT* const sK = reinterpret_cast<OT*>(smem);
  OT* const sQ = sK + C * D;
  float* const sL = reinterpret_cast<float*>(smem);
  float* const sT = sL + C * LCF;
  OT* const sM = reinterpret_cast<OT*>(sT);
  // Where M is staged. bf16 at C = 64: in the part of L's rows that L never uses (row tile t
  // of L fills 16 (t + 1) of its LCF floats): M's row tiles 0 and 3 beside L's tile 0, tile 2
  // beside tile 1, tile 1 beside tile 2. M then goes out while T is being formed, and T's
  // store needs no barrier before the next head's L and M. Otherwise in T's tile, behind
  // barriers.
  constexpr bool MINL = sizeof(OT) == 2 && C == 64;
  auto m_row = [&](int i) -> OT* {
    if constexpr (MINL) {
      const int t = i >> 4, r = i & 15;
      const int lr = (t == 0 || t == 3) ? r : (t == 2 ? 16 + r : 32 + r);
      const int lc = t == 0 ? 16 : (t == 3 ? 24 : (t == 2 ? 32 : 48));
      return reinterpret_cast<OT*>(sL + lr * LCF + lc);
    } else {
      return sM + i * C;
    }
  };

  const int kh = blockIdx.x % p.Hk, c = blockIdx.x / p.Hk;
  // The chunk table: every workgroup finds its own chunk; those of key head 0 write the
  // table's entries, and workgroup 0 the per-sequence offsets and the sweep order (in the
  // LDS before its K and Q arrive), so no launch of its own precedes prep.
  if (blockIdx.x == 0) seq_table<C, kPrepThreads>(p, reinterpret_cast<int*>(smem));
  const ChunkInfo ci = find_chunk<C>(p, c);
  if (kh == 0 && threadIdx.x == 0) p.chunks[c] = ci;
  if (ci.seq < 0) return;
  const int n = ci.len, w = wave_id(), l = lane_id(), g4 = (l >> 4) * 4, r16 = l & 15;
  // Gate records of value heads hb .. hb + GH - 1, one per wave (lane = row): gamma (log2
  // units) is the inclusive scan of log2 g, beta is 0 past the end. The raw g and beta of a
  // row are loaded first (gate_load) and turned into the record later (gates), so that the
  // loads' latency hides behind other work.
  auto gate_load = [&](int hb, float& gx, float& bx) {
    const int hh = hb + w, i = l;
    gx = 1.f;
    bx = 0.f;
    if (hh < p.r && i < n && i < C) {
      const int h = kh * p.r + hh;
      gx = p.g[(int64_t)(ci.t0 + i) * p.Hv + h];
      bx = p.beta[(int64_t)(ci.t0 + i) * p.Hv + h];
    }
  };
  float gx0, bx0;
  gate_load(0, gx0, bx0);  // issued before K and Q: they arrive while K and Q do
  {
    TileDma<C, D, NW, OT> dm;
    dm.init(w);
    // Non-temporal: each workgroup reads its K and Q rows once (prep 0.100 -> 0.083 ms with
    // both). K stays temporal when the forward saves its chunk states: the saving sweep that
    // follows reads K again and then finds it in the caches (sweep 0.297 -> 0.285 ms, prep
    // 0.090 ms: the better sum); the sweep without saves measured no such difference.
    const OT* kr = (const OT*)p.k + (int64_t)ci.t0 * p.k_rs + kh * D;
    if (p.sv_S)
      dm.issue(sK, kr, p.k_rs, n, w);
    else
      dm.template issue<true>(sK, kr, p.k_rs, n, w);
    dm.template issue<true>(sQ, (const OT*)p.q + (int64_t)ci.t0 * p.q_rs + kh * D, p.q_rs, n, w);
  }
  auto gates = [&](int hb, float gx, float bx) {
    const int hh = hb + w;
    if (hh < p.r) {
      const int h = kh * p.r + hh;
      const size_t ch = ch_idx(p, c, h);
      const int i = l;
      const bool ok = i < n && i < C;
      float lg = 0.f, be = 0.f, dla = 0.f;  // log2 g, beta, d log g / d alpha of the row
      if (ok) {
        if (p.a_log) {  // the gate chain from alpha and beta_raw
          lg = chain_log2g(gx, p.a_log[h], p.dt_bias[h]);
          be = chain_beta(bx);
          dla = chain_dlogg_dalpha(gx, p.a_log[h], p.dt_bias[h]);
        } else {
          lg = __builtin_amdgcn_logf(gx);
          be = bx;
        }
      }
      const float gam = wave_scan_incl(i < C ? lg : 0.f);
      const float glast = lane_value(gam, C - 1);
      if (i < C) {
        sg[w][i] = gam;
        sbeta[w][i] = be;
        float* rec = p.sv_gb + ch * kGateRows * C;
        rec[i] = gam;
        rec[C + i] = be;
        rec[2 * C + i] = __builtin_amdgcn_exp2f(gam);
        rec[3 * C + i] = __builtin_amdgcn_exp2f(glast - gam);
        rec[4 * C + i] = dla;
      }
    }
  };
  dma_wait();
  lds_barrier();
  if (p.sv_qn) {  // L2-normalise the q and k head rows in LDS and keep them, and the factors,
                  // for the later kernels: PPR lanes per row, one 16-byte piece each, rows of Q
                  // then of K, RPW rows per wave and pass
    using V = Vec16<OT>;
    constexpr int PPR = D / V::N, RPW = 64 / PPR;
    const int sub = l % PPR;
    for (int r0 = w * RPW; r0 < 2 * C; r0 += NW * RPW) {
      const int rr = r0 + l / PPR;
      const bool okr = rr < 2 * C;  // (every lane takes part in the group sum)
      OT* X = rr < C ? sQ : sK;
      const int i = okr ? rr % C : 0;
      typename V::type xv = *reinterpret_cast<const typename V::type*>(X + LD::at(i, sub * V::N));
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < V::N; ++e) ss += (float)xv[e] * (float)xv[e];
#pragma unroll
      for (int o = 1; o < PPR; o <<= 1) ss += __shfl_xor(ss, o);
      const float rf = 1.f / sqrtf(ss + 1e-6f);
#pragma unroll
      for (int e = 0; e < V::N; ++e) xv[e] = (OT)((float)xv[e] * rf);
      if (okr) {
        *reinterpret_cast<typename V::type*>(X + LD::at(i, sub * V::N)) = xv;
        if (i < n) {
          const int64_t hr = (int64_t)(ci.t0 + i) * p.Hk + kh;  // head row
          *reinterpret_cast<typename V::type*>((OT*)(rr < C ? p.sv_qn : p.sv_kn) + hr * D + sub * V::N) = xv;
          if (sub == 0) p.sv_r[hr * 2 + (rr < C ? 0 : 1)] = rf;
        }
      }
    }
    lds_barrier();
  }
  // The tiles (i, j) of K K^T and Q K^T below the diagonal that L and M need, formed
  // transposed (K_j K_i^T and K_j Q_i^T; K K^T is symmetric): lane (g, r) then holds row
  // 16 i + r at the four adjacent columns 16 j + 4 g .. 16 j + 4 g + 3, which go into L and
  // M as one 16-byte and one 8-byte write. At C = 64 wave w takes the tiles of kLmI/kLmJ
  // (one code path per wave, so that every tile index is a constant); otherwise wave
  // w < C / 16 takes row tile i = w.
  const bool rw = w < RT;
  constexpr int NTW = RT == 4 ? 3 : RT;
  f32x4 KK[NTW][1], QK[NTW][1];
  zero(KK);
  zero(QK);
  auto per_wave = [&](auto&& f) {
    if (w == 0) f(std::integral_constant<int, 0>{});
    else if (w == 1) f(std::integral_constant<int, 1>{});
    else if (w == 2) f(std::integral_constant<int, 2>{});
    else f(std::integral_constant<int, 3>{});
  };
  if constexpr (RT == 4) {
    per_wave([&](auto wc) {
      constexpr int W = decltype(wc)::value;
      using M = Mf<OT, KSD>;
#pragma unroll
      for (int s = 0; s < D / KSD; ++s)
        static_for<kLmN[W]>([&](auto tc) {
          constexpr int t = decltype(tc)::value, ti = kLmI[W][t], tj = kLmJ[W][t];
          const typename M::frag a = ld_n<OT, KSD, STD, LD>(sK, 16 * tj, s);
          KK[t][0] = M::run(a, ld_n<OT, KSD, STD, LD>(sK, 16 * ti, s), KK[t][0]);
          QK[t][0] = M::run(a, ld_n<OT, KSD, STD, LD>(sQ, 16 * ti, s), QK[t][0]);
        });
    });
  } else if (rw) {
    auto fa = [&](int j, int s) { return ld_n<OT, KSD, STD, LD>(sK, 16 * j, s); };
    wave_mm<OT, D, RT, 1>(KK, fa, [&](int, int s) { return ld_n<OT, KSD, STD, LD>(sK, 16 * w, s); });
    wave_mm<OT, D, RT, 1>(QK, fa, [&](int, int s) { return ld_n<OT, KSD, STD, LD>(sQ, 16 * w, s); });
  }
  gates(0, gx0, bx0);  // the first GH records (their raw values were loaded at the start)
  // The raw gate loads count as consumed on every path (waves past the last head skip the
  // record). Otherwise the compiler keeps them pending into the head loop, and each reuse of
  // their registers there waits for every outstanding memory operation, the T and M stores
  // included: prep 0.089 -> 0.084 ms.
  asm volatile("" ::"v"(gx0), "v"(bx0));
  lds_barrier();  // K and Q consumed; the records are in LDS
  for (int hh = 0; hh < p.r; ++hh) {
    const int h = kh * p.r + hh;
    const size_t ch = ch_idx(p, c, h);
    if (hh > 0 && hh % GH == 0) {  // the next group of gate records (the last head's barrier freed sg)
      float gx, bx;
      gate_load(hh, gx, bx);
      gates(hh, gx, bx);
      asm volatile("" ::"v"(gx), "v"(bx));  // (as above)
      lds_barrier();
    }
    const float* sgh = sg[hh % GH];
    const float* sbh = sbeta[hh % GH];
    // Tile (ti, tj) of L and M from the wave's Gram tiles. Above the diagonal neither is
    // stored (M and T go out in lower-block form, and L is never read there); below it no
    // element mask is needed.
    auto lm_tile = [&](int ti, int tj, const f32x4& kk, const f32x4& qk) {
      const int i = 16 * ti + r16;  // this lane's row
      const float gi = sgh[i], bi = sbh[i];
      const f32x4 gj = *reinterpret_cast<const f32x4*>(sgh + 16 * tj + g4);
      f32x4 lv4, mv4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {  // column 16 tj + g4 + e
        const float gd = __builtin_amdgcn_exp2f(gi - gj[e]);
        float lv = bi * gd * kk[e], mv = gd * qk[e];
        if (ti == tj) {
          lv = r16 > g4 + e ? lv : 0.f;
          mv = r16 >= g4 + e ? mv : 0.f;
        }
        if (n < C) mv = i < n ? mv : 0.f;
        lv4[e] = lv;
        mv4[e] = mv;
      }
      *reinterpret_cast<f32x4*>(sL + i * LCF + 16 * tj + g4) = lv4;
      store4(m_row(i) + 16 * tj + g4, mv4);
    };
    if constexpr (RT == 4) {
      per_wave([&](auto wc) {
        constexpr int W = decltype(wc)::value;
        static_for<kLmN[W]>([&](auto tc) {
          constexpr int t = decltype(tc)::value;
          lm_tile(kLmI[W][t], kLmJ[W][t], KK[t][0], QK[t][0]);
        });
      });
    } else if (rw) {
#pragma unroll
      for (int j = 0; j < RT; ++j)
        if (j <= w) lm_tile(w, j, KK[j][0], QK[j][0]);
    }
    lds_barrier();
    {  // M in lower-block form, 16-byte non-temporal stores (T's as well: 2% faster prep), beside
       // L: by the waves that do not start T
      using V = Vec16<OT>;
      OT* dst = (OT*)p.sv_M + ch * C * C;
      constexpr int Q0 = MINL ? 64 : 0;
      for (int q = (int)threadIdx.x - Q0; q < low_row_off(C) / V::N; q += NT - Q0) {
        if (q < 0) break;
        int i, j0;
        low_piece<C, V::N>(q, i, j0);
        store_nt(reinterpret_cast<typename V::type*>(dst + q * V::N), *reinterpret_cast<const typename V::type*>(m_row(i) + j0));
      }
    }
    if constexpr (!MINL) lds_barrier();  // M is out: its staging tile becomes T
    invert_unit_lower<C, LCF, NW>(sL, sT);
    {  // T in lower-block form, 16-byte stores. With M beside L, by waves 0 and 1 only: the
       // others start the next head's L and M at once (waves 2 and 3 hold its most tiles).
      OT* dst = (OT*)p.sv_T + ch * C * C;
      constexpr int E8 = 16 / (int)sizeof(OT);  // elements per 16-byte store
      constexpr int TW = MINL ? 2 : NW;           // waves that store T
      // Row tile by row tile, so that the pieces per row are a constant (no run-time
      // division in the piece's row and column; 1% faster prep)
      static_for<RT>([&](auto tt) {
        constexpr int t = decltype(tt)::value, RL = low_row_len(16 * t) / E8;
        for (int u = threadIdx.x; u < 16 * RL; u += TW * 64) {
          if (threadIdx.x >= TW * 64) break;
          const int i = 16 * t + u / RL, j0 = (u % RL) * E8;
          OT* const d = dst + low_row_off(16 * t) + u * E8;
          const f32x4 a = *reinterpret_cast<const f32x4*>(sT + i * LCF + j0);
          if constexpr (E8 == 8) {
            const f32x4 b = *reinterpret_cast<const f32x4*>(sT + i * LCF + j0 + 4);
            store_nt(reinterpret_cast<bf16x8*>(d), bf16x8{(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3],
                                                          (__bf16)b[0], (__bf16)b[1], (__bf16)b[2], (__bf16)b[3]});
          } else {
            store4(d, a);
          }
        }
      });
    }
    if constexpr (!MINL) lds_barrier();  // sL, sT, sM free for the next head (with MINL the next
                                         // head's first barrier orders T's reads before T is rewritten)
  }
}

// ---------------------------------------------------------------------------- sweep
template <typename TI, int C, int D> struct SwCfg {
  static constexpr int WC = 16;       // state columns per wave: two waves per SIMD at D = 128
  static constexpr int NW = D / WC;   // waves: one workgroup holds every column of a head
  static constexpr int CT = WC / 16, DT = D / 16, RT = C / 16;
  static constexpr int CE = 16 / (int)sizeof(TI);  // elements per 16-byte chunk
  static constexpr int LSO = D + CE;               // row stride of the output staging tile
  // LDS layouts of the [C][D] tiles K, Q, V and the [C][C] tiles T, M: plain chunk map,
  // with the 16-row tile gap where rows hold four or more chunks.
  static constexpr bool PTD = D * (int)sizeof(TI) >= 64, PTC = C * (int)sizeof(TI) >= 64;
  using LDL = Swz<TI, D, false, PTD>;
  using LCL = Swz<TI, C, false, PTC>;
  // One LDS buffer: K, Q, V, then T, M, each region followed by a 128-byte gap (so that
  // equal offsets in two regions are not a multiple of 512 bytes apart either).
  static constexpr int G = 128 / (int)sizeof(TI), SD = LDL::size(C) + G, SC = LCL::size(C) + G;
  static constexpr int O_K = 0, O_Q = SD, O_V = 2 * SD, O_T = 3 * SD, O_M = O_T + SC, BUF = O_M + SC;
};

// One saved row segment per lane and column tile: the transposed tile X^T[v][j] of a
// wave's accumulators Xc[ct][t] (rows j = 16 t + g4 + e of column v = v0 + 16 ct + r16),
// into rows of LEN elements in RowOrd<OT, LEN> order. In fragment order every lane stores
// its 16-byte MFMA fragment (frag[ct][s], ACC order over j) with one instruction.
template <typename OT, int LEN, int CT, int NT, int NS>
__device__ __forceinline__ void save_rows(OT* dst, int v0, const f32x4 (&Xc)[CT][NT],
                                          const typename Mf<OT, ks_of<OT, LEN>()>::frag (&frag)[CT][NS]) {
  const int l = lane_id(), g4 = (l >> 4) * 4, r16 = l & 15;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    OT* row = dst + (size_t)(v0 + 16 * ct + r16) * LEN;
    if constexpr (RowOrd<OT, LEN>::frag) {
#pragma unroll
      for (int s = 0; s < NS; ++s) *reinterpret_cast<bf16x8*>(row + 32 * s + 2 * g4) = frag[ct][s];
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) store4(row + 16 * t + g4, Xc[ct][t]);
    }
  }
}

// Wave-local ordering of LDS writes before reads by other lanes of the same wave.
__device__ __forceinline__ void lds_wave_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Grid xcd_grid(N * Hk, r): one workgroup per (sequence, value head); the r value heads
// of a key head run on one XCD (they read the same K and Q). SAVE: keep the chunk-start
// state and Delta of every chunk for the backward (off for a forward-only call, which then
// writes only o and S_T).
template <typename TI, int C, int D, bool SAVE>
__global__ __launch_bounds__((SwCfg<TI, C, D>::NW * 64)) void k_fwd_sweep(Prob p) {
  using OT = TI;
  using CF = SwCfg<TI, C, D>;
  constexpr int NW = CF::NW, WC = CF::WC, CT = CF::CT, DT = CF::DT, RT = CF::RT, CE = CF::CE;
  constexpr int KSD = ks_of<OT, D>(), KSC = ks_of<OT, C>(), NSD = D / KSD, NSC = C / KSC;
  using LD = typename CF::LDL;
  using LC = typename CF::LCL;
  using FragD = typename Mf<OT, KSD>::frag;
  using FragC = typename Mf<OT, KSC>::frag;
  __shared__ __align__(16) OT sbuf[2][CF::BUF];
  __shared__ __align__(16) float sgb[2][kSweepGateRows * C];
  __shared__ __align__(16) OT stg[C * CF::LSO];  // the chunk's output rows, all D columns

  int grp, hh;
  if (!xcd_group(blockIdx.x, p.N * p.Hk, p.r, grp, hh)) return;
  const int n = p.seq_order[grp / p.Hk], kh = grp % p.Hk, h = kh * p.r + hh;  // longest sequences first
  const size_t nh = (size_t)n * p.Hv + h;
  const int c0 = p.seq_chunk[n], c1 = p.seq_chunk[n + 1];
  int64_t sa, sb;  // rows of the sequence; chunk c starts at sa + (c - c0) C (as in the chunk table)
  seq_bounds(p, n, sa, sb);
  const int w = wave_id(), l = lane_id(), g4 = (l >> 4) * 4, r16 = l & 15;
  const int v0 = w * WC;  // first state column of this wave

  TileDma<C, D, NW, OT, false, CF::PTD> dmD;  // K, Q, V
  TileDmaLow<C, NW, OT, false, CF::PTC> dmC;  // T, M (lower-block form)
  TileDma<1, kSweepGateRows * C, NW, float> dmG;  // gate record rows 0-3
  dmD.init(w);
  dmC.init(w);
  dmG.init(w);
  // The next chunk's loads, in parts: part 0 right after the step's first barrier, part 1
  // after K S, part 2 after T X. With the saves every load goes in part 0 (their stores share
  // the memory queue, and loads issued later in the step arrive late); without them K goes
  // first, Q next and V, T, M and the gate record last (a shorter stall at each issue: the
  // forward-only step measured 12% shorter than with every load in part 0).
  auto issue = [&](int c, int buf, int part) {
    const int64_t t0 = sa + (int64_t)(c - c0) * C;
    const int len = (int)(sb - t0 < C ? sb - t0 : C);
    const size_t ch = ch_idx(p, c, h);
    OT* b = sbuf[buf];
    if (part == 0) dmD.issue(b + CF::O_K, (const OT*)p.ku + t0 * p.ku_rs + kh * D, p.ku_rs, len, w);
    if (part == (SAVE ? 0 : 1)) dmD.issue(b + CF::O_Q, (const OT*)p.qu + t0 * p.qu_rs + kh * D, p.qu_rs, len, w);
    if (part == (SAVE ? 0 : 2)) {
      // V, T and M are this workgroup's alone (non-temporal); K and Q are shared by the r
      // value heads of the key head, which run on the same XCD
      dmD.template issue<true>(b + CF::O_V, (const OT*)p.v + t0 * p.v_rs + h * D, p.v_rs, len, w);
      dmC.template issue<true>(b + CF::O_T, (const OT*)p.sv_T + ch * C * C, w);
      dmC.template issue<true>(b + CF::O_M, (const OT*)p.sv_M + ch * C * C, w);
      dmG.issue(sgb[buf], p.sv_gb + ch * kGateRows * C, kSweepGateRows * C, 1, w);
    }
  };
#pragma unroll
  for (int bf = 0; bf < 2; ++bf) {  // the blocks above the diagonal of T and M stay zero
    dmC.zero_upper(sbuf[bf] + CF::O_T, w);
    dmC.zero_upper(sbuf[bf] + CF::O_M, w);
  }

  // The state: S[ct][dt] holds S[16 dt + g4 + e][v0 + 16 ct + r16].
  f32x4 S[CT][DT];
  if (p.S0) {
    const float* s0 = p.S0 + nh * D * D;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[ct][dt][e] = s0[(16 * dt + g4 + e) * D + v0 + 16 * ct + r16];
  } else {
    zero(S);
  }

  if (c0 < c1)
    for (int part = 0; part < 3; ++part) issue(c0, 0, part);
  int buf = 0;
  for (int c = c0; c < c1; ++c, buf ^= 1) {
    dma_wait();
    lds_barrier();  // chunk c is in sbuf[buf]; every wave is done with sbuf[buf ^ 1] and stg
    if (c + 1 < c1) issue(c + 1, buf ^ 1, 0);
    const int64_t t0 = sa + (int64_t)(c - c0) * C;
    const int len = (int)(sb - t0 < C ? sb - t0 : C);
    const size_t ch = ch_idx(p, c, h);
    const OT* sK = sbuf[buf] + CF::O_K;
    const OT* sQ = sbuf[buf] + CF::O_Q;
    const OT* sV = sbuf[buf] + CF::O_V;
    const OT* sT = sbuf[buf] + CF::O_T;
    const OT* sM = sbuf[buf] + CF::O_M;
    const float* bet = sgb[buf] + C;
    const float* brec = sgb[buf] + 2 * C;  // b = 2^gamma
    const float* erec = sgb[buf] + 3 * C;  // e = 2^(gamma_last - gamma)
    // decay factors of this lane's accumulator rows i = 16 t + g4 + e
    const float bn = brec[C - 1];
    f32x4 bx[RT], ex[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      bx[t] = *reinterpret_cast<const f32x4*>(brec + 16 * t + g4);
      ex[t] = *reinterpret_cast<const f32x4*>(erec + 16 * t + g4);
    }
    // the state's MFMA fragments (B operand over d), shared by K S, Q S and the saved copy
    FragD Sb[CT][NSD];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int s = 0; s < NSD; ++s) Sb[ct][s] = from_acc<OT, KSD>(S[ct], s, Ident{});
    // X = beta o (V - b o K S), then Delta = T X
    f32x4 X[CT][RT];
    {
      f32x4 KS[RT][CT];
      zero(KS);
      wave_mm<OT, D, RT, CT>(KS, [&](int m, int s) { return ld_n<OT, KSD, ACC, LD>(sK, 16 * m, s); },
                             [&](int j, int s) { return Sb[j][s]; });
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const f32x4 bb = *reinterpret_cast<const f32x4*>(bet + 16 * t + g4);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const f32x4 vv = ld_col4<OT, LD>(sV, 16 * t + g4, v0 + 16 * ct);
#pragma unroll
          for (int e = 0; e < 4; ++e) X[ct][t][e] = bb[e] * (vv[e] - bx[t][e] * KS[t][ct][e]);
        }
      }
    }
    if (!SAVE && c + 1 < c1) issue(c + 1, buf ^ 1, 1);
    f32x4 Dl[CT][RT];
    zero(Dl);
    wave_mm_cm<OT, C, RT, CT, TRI_LOW>(Dl, [&](int m, int s) { return ld_n<OT, KSC, ACC, LC>(sT, 16 * m, s); },
                              [&](int j, int s) { return from_acc<OT, KSC>(X[j], s, Ident{}); });
    FragC Db[CT][NSC];  // Delta's fragments: B operand of M Delta
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int s = 0; s < NSC; ++s) Db[ct][s] = from_acc<OT, KSC>(Dl[ct], s, Ident{});
    if constexpr (SAVE) {  // Delta's columns of this wave replace the wave's own (consumed)
                           // columns of V in LDS; the full rows are written out with the output rows
      OT* sDw = sbuf[buf] + CF::O_V;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) sDw[LD::at(16 * t + g4 + e, v0 + 16 * ct + r16)] = (OT)Dl[ct][t][e];
    }
    if (!SAVE && c + 1 < c1) issue(c + 1, buf ^ 1, 2);
    {  // O = b o Q S + M Delta, staged as rows for the whole workgroup
      f32x4 O[RT][CT];
      zero(O);
      wave_mm<OT, D, RT, CT>(O, [&](int m, int s) { return ld_n<OT, KSD, ACC, LD>(sQ, 16 * m, s); },
                             [&](int j, int s) { return Sb[j][s]; });
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e) O[t][ct][e] *= bx[t][e];
      wave_mm<OT, C, RT, CT, TRI_LOW>(O, [&](int m, int s) { return ld_n<OT, KSC, ACC, LC>(sM, 16 * m, s); },
                             [&](int j, int s) { return Db[j][s]; });
      const float sc = p.scale;
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e) stg[(16 * t + g4 + e) * CF::LSO + v0 + 16 * ct + r16] = (OT)(sc * O[t][ct][e]);
    }
    // S^T[v][d] at the chunk start, stored late in the step (the stores then queue behind the
    // next chunk's loads, not before them; 1% shorter step)
    if constexpr (SAVE) save_rows<OT, D, CT, DT, NSD>((OT*)p.sv_S + ch * D * D, v0, S, Sb);
    lds_barrier();  // the chunk's output rows and Delta rows are staged
    {  // full output (and Delta) rows, 16-byte stores spread over every wave
      using V = Vec16<OT>;
      constexpr int VPR = D / CE;
      TI* o = (TI*)p.o + t0 * p.o_rs + h * D;
      OT* dl = (OT*)p.sv_D + ch * C * D;
      constexpr int BV = grad_block<OT, D>();  // Delta goes out in blocks of BV columns
      const OT* sD = sbuf[buf] + CF::O_V;
#pragma unroll
      for (int idx = threadIdx.x; idx < C * VPR; idx += NW * 64) {
        const int i = idx / VPR, q = idx % VPR;
        if (i < len) {
          // (non-temporal without the saves: 0.3% shorter forward-only call; with them the
          // temporal store measured faster)
          const typename V::type ov = *reinterpret_cast<const typename V::type*>(stg + i * CF::LSO + q * CE);
          if constexpr (SAVE)
            *reinterpret_cast<typename V::type*>(o + (int64_t)i * p.o_rs + q * CE) = ov;
          else
            store_nt(reinterpret_cast<typename V::type*>(o + (int64_t)i * p.o_rs + q * CE), ov);
          if constexpr (SAVE)
            *reinterpret_cast<typename V::type*>(dl + (q * CE / BV) * C * BV + i * BV + (q * CE) % BV) =
                *reinterpret_cast<const typename V::type*>(sD + LD::at(i, q * CE));
        }
      }
    }
    // S <- b_n S + K^T (e o Delta)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) S[ct][dt] *= bn;
    wave_mm_cm<OT, C, DT, CT>(
        S, [&](int m, int s) { return ld_t<OT, KSC, ACC, LD>(sK, 16 * m, s); },
        [&](int j, int s) {
          return from_acc<OT, KSC>(Dl[j], s, [&](int t, int e, float x) { return ex[t][e] * x; });
        });
  }
  if (p.ST) {
    float* st = p.ST + nh * D * D;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) st[(16 * dt + g4 + e) * D + v0 + 16 * ct + r16] = S[ct][dt][e];
  }
}

template <typename TI, int C, int D>
static hipError_t fwd_seq(const Prob& p, hipStream_t s) {
  using CF = SwCfg<TI, C, D>;
  if (p.nc_max > 0)
    traced("k_prep", s, [&] { k_prep<TI, C, D><<<p.nc_max * p.Hk, kPrepThreads, 0, s>>>(p); });
  else  // no chunk slots: the table still gives the sweeps their (empty) chunk ranges
    traced("k_table", s, [&] { k_table<C><<<1, NTHREADS, 0, s>>>(p); });
  if (p.N > 0) {
    if (p.sv_S)
      traced("k_fwd_sweep", s,
             [&] { k_fwd_sweep<TI, C, D, true><<<xcd_grid(p.N * p.Hk, p.r), CF::NW * 64, 0, s>>>(p); });
    else
      traced("k_fwd_sweep_nosave", s,
             [&] { k_fwd_sweep<TI, C, D, false><<<xcd_grid(p.N * p.Hk, p.r), CF::NW * 64, 0, s>>>(p); });
  }
  return hipGetLastError();
}

template <typename TI, int C>
static hipError_t fwd_d(const Prob& p, hipStream_t s) {
  switch (p.D) {
    case 16: return fwd_seq<TI, C, 16>(p, s);
    case 32: return fwd_seq<TI, C, 32>(p, s);
    case 64:
      if constexpr (sizeof(TI) == 4 && C == 64)
        return hipErrorInvalidValue;  // rejected on the host (LDS)
      else
        return fwd_seq<TI, C, 64>(p, s);
    case 128:
      if constexpr (sizeof(TI) == 4 && C == 64)
        return hipErrorInvalidValue;
      else
        return fwd_seq<TI, C, 128>(p, s);
  }
  return hipErrorInvalidValue;
}

template <typename TI>
static hipError_t fwd_c(const Prob& p, hipStream_t s) {
  return p.C == 16 ? fwd_d<TI, 16>(p, s) : fwd_d<TI, 64>(p, s);
}

hipError_t launch_forward(const Prob& p, int dtype, hipStream_t s) {
  return dtype == 0 ? fwd_c<float>(p, s) : fwd_c<__bf16>(p, s);
}

}  // namespace gdn
