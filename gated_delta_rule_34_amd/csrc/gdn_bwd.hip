// gdn_bwd.hip -- chunked reverse-mode backward of the gated delta rule on gfx950.
//
// Per-token form: lattice-inference gdn_backward.rs, gdn_backward steps 4a-4d (output,
// state update, delta, retrieval), with the state adjoint dS carried in reverse time.
// Chunk form (derived here; the pages give none), with dO~ = scale dO, e = exp(gamma_n -
// gamma), M = Gamma o Q K^T (lower incl.) and dS_C the adjoint flowing into the end of a
// chunk:
//   dDelta = M^T dO~ + diag(e) K dS_C
//   dS_0   = b_n dS_C + Q^T diag(b) dO~ - K^T diag(beta b) T^T dDelta   (W^T = K^T diag(beta b) T^T)
//   XQ = dO~ S0^T,  XK = Delta dS_C^T,  A = T^T dDelta,  Y = A S0^T,  P = tril(dO~ Delta^T)
//   dQ     = diag(b) XQ + (P o Gamma) K
//   dV     = diag(beta) A;  dL = -stril(A Delta^T)   (dT = dDelta ((I + L) Delta)^T, T (I + L) = I)
//   dK     = (P o Gamma)^T Q + diag(e) XK - diag(beta b) Y + G K + G^T K,  G = dL o (beta_i Gamma_ij)
//   dbeta  = rowsum(A o V) + b o rho + rowsum(dL o Gamma o K K^T),  rho = -rowsum(Y o K)
//   dgamma = b o rowsum(Q o XQ) + beta b rho - ebar + rowsum(Gbar o Gamma) - colsum(Gbar o Gamma),
//            ebar = e o rowsum(K o XK), Gbar o Gamma = P o M + dL o beta_i K K^T o Gamma,
//            and the last valid row also gets b_n <S0, dS_C> + sum(ebar)
//   dlog g = reverse cumulative sum of dgamma within the chunk;  dg = dlog g / g.
//
// Kernels after the chunk table:
//  k_bwd_sweep (sequence x value head, one wave per 32 adjoint columns): the reverse
//      chunk-serial pass; dS, K dS, dDelta and A = T^T dDelta stay in float32 accumulators.
//      Writes dV = diag(beta) A (staged as full rows) and saves dS_C and A per chunk.
//  k_bwd_grad (chunk x key head, 8 waves): the remaining gradients for the r value heads
//      of the key head, one head after the other, streaming the value dimension in
//      blocks (the next block in flight while the current one is used). dq and dk of
//      the key head are summed over its value heads in ascending order in registers and
//      stored once: no atomics, every run is bit-identical. Row sums go through partial
//      arrays indexed by column block and are added in a fixed order.
#include "gdn_common.h"

namespace gdn {

template <typename OT> __device__ __forceinline__ void store4b(OT* dst, f32x4 x) {
  if constexpr (sizeof(OT) == 2)
    *reinterpret_cast<bf16x4*>(dst) = bf16x4{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
  else
    *reinterpret_cast<f32x4*>(dst) = x;
}

// ---------------------------------------------------------------------------- sweep
template <typename TI, int C, int D> struct BwCfg {
  static constexpr int WC = 16;  // adjoint columns per wave: two waves per SIMD at D = 128
  static constexpr int NW = D / WC;
  static constexpr int CT = WC / 16, DT = D / 16, RT = C / 16;
  static constexpr int CE = 16 / (int)sizeof(TI);  // elements per 16-byte chunk
  static constexpr int LSO = D + CE;               // row stride of the dV staging tile
  // One LDS buffer: K, Q, dO [C][D] and T, M [C][C], all Swz layouts.
  static constexpr int O_K = 0, O_Q = C * D, O_O = 2 * C * D, O_T = 3 * C * D, O_M = O_T + C * C, BUF = O_M + C * C;
};

// Saved rows X^T[v][j] of a wave's accumulator tiles, in RowOrd<OT, LEN> order (the same
// writer as the forward's: fragment order stores each lane's 16-byte fragment at once).
template <typename OT, int LEN, int CT, int NT, int NS>
__device__ __forceinline__ void save_rows_b(OT* dst, int v0, const f32x4 (&Xc)[CT][NT],
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
      for (int t = 0; t < NT; ++t) store4b(row + 16 * t + g4, Xc[ct][t]);
    }
  }
}

// Grid xcd_grid(N * Hk, r). Reverse chunk-serial pass over one sequence and one value head.
template <typename TI, int C, int D>
__global__ __launch_bounds__((BwCfg<TI, C, D>::NW * 64)) void k_bwd_sweep(Prob p) {
  using OT = TI;
  using CF = BwCfg<TI, C, D>;
  constexpr int NW = CF::NW, WC = CF::WC, CT = CF::CT, DT = CF::DT, RT = CF::RT, CE = CF::CE;
  constexpr int KSD = ks_of<OT, D>(), KSC = ks_of<OT, C>(), NSD = D / KSD, NSC = C / KSC;
  using LD = Swz<OT, D, true>;
  using LC = Swz<OT, C, true>;
  using FragD = typename Mf<OT, KSD>::frag;
  using FragC = typename Mf<OT, KSC>::frag;
  __shared__ __align__(16) OT sbuf[2][CF::BUF];
  __shared__ __align__(16) float sgb[2][kSweepGateRows * C];
  __shared__ __align__(16) OT stg[C * CF::LSO];  // the chunk's dV rows, all D columns

  int grp, hh;
  if (!xcd_group(blockIdx.x, p.N * p.Hk, p.r, grp, hh)) return;
  const int n = p.seq_order[grp / p.Hk], kh = grp % p.Hk, h = kh * p.r + hh;  // longest sequences first
  const size_t nh = (size_t)n * p.Hv + h;
  const int c0 = p.seq_chunk[n], c1 = p.seq_chunk[n + 1];
  int64_t sa, sb;  // rows of the sequence; chunk c starts at sa + (c - c0) C (as in the chunk table)
  seq_bounds(p, n, sa, sb);
  const int w = wave_id(), l = lane_id(), g4 = (l >> 4) * 4, r16 = l & 15;
  const int v0 = w * WC;

  TileDma<C, D, NW, OT, true> dmD;   // K, Q, dO
  TileDmaLow<C, NW, OT, true> dmC;  // T, M (lower-block form)
  TileDma<1, kSweepGateRows * C, NW, float> dmG;  // gate record rows 0-3
  dmD.init(w);
  dmC.init(w);
  dmG.init(w);
  auto issue = [&](int c, int buf) {
    const int64_t t0 = sa + (int64_t)(c - c0) * C;
    const int len = (int)(sb - t0 < C ? sb - t0 : C);
    const size_t ch = ch_idx(p, c, h);
    OT* b = sbuf[buf];
    dmD.issue(b + CF::O_K, (const OT*)p.ku + t0 * p.ku_rs + kh * D, p.ku_rs, len, w);
    dmD.issue(b + CF::O_Q, (const OT*)p.qu + t0 * p.qu_rs + kh * D, p.qu_rs, len, w);
    // dO, T and M are this workgroup's alone (non-temporal); K and Q are shared by the r value
    // heads of the key head, which run on the same XCD
    dmD.template issue<true>(b + CF::O_O, (const OT*)p.dO + t0 * p.dO_rs + h * D, p.dO_rs, len, w);
    dmC.template issue<true>(b + CF::O_T, (const OT*)p.sv_T + ch * C * C, w);
    dmC.template issue<true>(b + CF::O_M, (const OT*)p.sv_M + ch * C * C, w);
    dmG.issue(sgb[buf], p.sv_gb + ch * kGateRows * C, kSweepGateRows * C, 1, w);
  };
#pragma unroll
  for (int bf = 0; bf < 2; ++bf) {  // the blocks above the diagonal of T and M stay zero
    dmC.zero_upper(sbuf[bf] + CF::O_T, w);
    dmC.zero_upper(sbuf[bf] + CF::O_M, w);
  }

  // The adjoint: dS[ct][dt] holds dS[16 dt + g4 + e][v0 + 16 ct + r16].
  f32x4 dS[CT][DT];
  if (p.dST) {
    const float* s = p.dST + nh * D * D;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) dS[ct][dt][e] = s[(16 * dt + g4 + e) * D + v0 + 16 * ct + r16];
  } else {
    zero(dS);
  }

  if (c0 < c1) issue(c1 - 1, 0);
  int buf = 0;
  for (int c = c1 - 1; c >= c0; --c, buf ^= 1) {
    dma_wait();
    lds_barrier();  // chunk c is in sbuf[buf]; every wave is done with sbuf[buf ^ 1] and stg
    if (c - 1 >= c0) issue(c - 1, buf ^ 1);
    const int64_t t0 = sa + (int64_t)(c - c0) * C;
    const int len = (int)(sb - t0 < C ? sb - t0 : C);
    const size_t ch = ch_idx(p, c, h);
    const OT* sK = sbuf[buf] + CF::O_K;
    const OT* sQ = sbuf[buf] + CF::O_Q;
    const OT* sO = sbuf[buf] + CF::O_O;
    const OT* sT = sbuf[buf] + CF::O_T;
    const OT* sM = sbuf[buf] + CF::O_M;
    const float* bet = sgb[buf] + C;
    const float* brec = sgb[buf] + 2 * C;  // b = 2^gamma
    const float* erec = sgb[buf] + 3 * C;  // e = 2^(gamma_last - gamma)
    const float bn = brec[C - 1], sc = p.scale;
    // per-row factors of this lane's accumulator rows i = 16 t + g4 + e, each formed from
    // the gate record where it is used (fewer registers live across the step)
    auto row_factors = [&](float (&f)[RT][4], auto&& fn) {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const f32x4 bv = *reinterpret_cast<const f32x4*>(bet + 16 * t + g4);
        const f32x4 b4 = *reinterpret_cast<const f32x4*>(brec + 16 * t + g4);
        const f32x4 e4 = *reinterpret_cast<const f32x4*>(erec + 16 * t + g4);
#pragma unroll
        for (int e = 0; e < 4; ++e) f[t][e] = fn(bv[e], b4[e], e4[e]);
      }
    };
    float ex[RT][4];  // e_i
    row_factors(ex, [](float, float, float e_) { return e_; });
    // dS_C's fragments (B operand over d) and its saved copy dS^T[v][d]
    FragD dSb[CT][NSD];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int s = 0; s < NSD; ++s) dSb[ct][s] = from_acc<OT, KSD>(dS[ct], s, Ident{});
    // dDelta = e o (K dS) + scale M^T dO
    f32x4 dD[CT][RT];
    {
      f32x4 KdS[RT][CT], MdO[RT][CT];
      zero(KdS);
      zero(MdO);
      wave_mm<OT, D, RT, CT>(KdS, [&](int m, int s) { return ld_n<OT, KSD, ACC, LD>(sK, 16 * m, s); },
                             [&](int j, int s) { return dSb[j][s]; });
      wave_mm<OT, C, RT, CT, TRI_UP>(MdO, [&](int m, int s) { return ld_t<OT, KSC, STD, LC>(sM, 16 * m, s); },
                             [&](int j, int s) { return ld_t<OT, KSC, STD, LD>(sO, v0 + 16 * j, s); });
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e) dD[ct][t][e] = ex[t][e] * KdS[t][ct][e] + sc * MdO[t][ct][e];
    }
    FragC dDb[CT][NSC];  // dDelta's fragments: B operand of T^T dDelta
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int s = 0; s < NSC; ++s) dDb[ct][s] = from_acc<OT, KSC>(dD[ct], s, Ident{});
    // A = T^T dDelta, staged as rows: the flush writes the gradient kernel's A (in blocks
    // of BV value columns) and dV = diag(beta) A from them
    f32x4 Z[CT][RT];
    zero(Z);
    wave_mm_cm<OT, C, RT, CT, TRI_UP>(Z, [&](int m, int s) { return ld_t<OT, KSC, ACC, LC>(sT, 16 * m, s); },
                              [&](int j, int s) { return dDb[j][s]; });
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) stg[(16 * t + g4 + e) * CF::LSO + v0 + 16 * ct + r16] = (OT)Z[ct][t][e];
    // the saved dS^T[v][d] (stored here rather than at the top of the step, where its stores
    // would queue ahead of the next chunk's loads: 3% shorter step)
    save_rows_b<OT, D, CT, DT, NSD>((OT*)p.ws_dS + ch * D * D, v0, dS, dSb);
    // dS <- b_n dS + Q^T (scale b o dO) while the other waves finish staging
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dS[ct][dt] *= bn;
    float sbx[RT][4];  // scale b_i
    row_factors(sbx, [&](float, float b_, float) { return sc * b_; });
    wave_mm_cm<OT, C, DT, CT>(
        dS, [&](int m, int s) { return ld_t<OT, KSC, ACC, LD>(sQ, 16 * m, s); },
        [&](int j, int s) { return scale_acc<OT, KSC, RT>(ld_t<OT, KSC, ACC, LD>(sO, v0 + 16 * j, s), s, sbx); });
    lds_barrier();  // the chunk's A rows are staged
    {  // A blocks and full dV rows, 16-byte stores spread over every wave
      using V = Vec16<OT>;
      constexpr int VPR = D / CE;
      constexpr int BV = grad_block<OT, D>();  // A goes out in blocks of BV columns
      TI* dv = (TI*)p.dv + t0 * p.dv_rs + h * D;
      OT* ab = (OT*)p.ws_A + ch * C * D;
#pragma unroll
      for (int idx = threadIdx.x; idx < C * VPR; idx += NW * 64) {
        const int i = idx / VPR, q = idx % VPR;
        if (i < len) {
          const typename V::type a = *reinterpret_cast<const typename V::type*>(stg + i * CF::LSO + q * CE);
          *reinterpret_cast<typename V::type*>(ab + (q * CE / BV) * C * BV + i * BV + (q * CE) % BV) = a;
          const float be = bet[i];
          typename V::type dvv;
#pragma unroll
          for (int k = 0; k < CE; ++k) dvv[k] = (OT)(be * (float)a[k]);
          // non-temporal: dV is a result no later kernel reads, and left in the caches it
          // displaces the saved blocks the gradient kernel reads next (that kernel 0.400 ->
          // 0.396 ms)
          store_nt(reinterpret_cast<typename V::type*>(dv + (int64_t)i * p.dv_rs + q * CE), dvv);
        }
      }
    }
    // dS <- dS - K^T (beta b o Z)
    float nbb[RT][4];  // -beta_i b_i
    row_factors(nbb, [](float be, float b_, float) { return -be * b_; });
    wave_mm_cm<OT, C, DT, CT>(
        dS, [&](int m, int s) { return ld_t<OT, KSC, ACC, LD>(sK, 16 * m, s); },
        [&](int j, int s) {
          return from_acc<OT, KSC>(Z[j], s, [&](int t, int e, float x) { return nbb[t][e] * x; });
        });
  }
  if (p.dS0) {
    float* s = p.dS0 + nh * D * D;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[(16 * dt + g4 + e) * D + v0 + 16 * ct + r16] = dS[ct][dt][e];
  }
}

// ---------------------------------------------------------------------------- grad
// Wave tiling of the C x D products (RT x DT tiles of 16 x 16) and of the C x C products
// (RT x RT tiles) over NW waves. Wave w owns row block rb = w % WRB (MT row tiles) and
// column block cb = w / WRB: NT of the D tiles and NTC of the C tiles. The C x C tiles of a
// wave lie in its own row tiles, so both kinds of product share the wave's A fragments, and
// with MT = 2 every fragment read from LDS feeds at least two MFMAs.
template <int RT, int DT, int NW> struct Part {
  static constexpr int MT = (RT >= 2 && RT * DT >= 2 * NW) ? 2 : 1;
  static constexpr int WRB = RT / MT;
  static_assert(WRB <= NW && NW % WRB == 0, "row blocks must divide the waves");
  static constexpr int WCB = NW / WRB;
  static constexpr int NT = DT >= WCB ? DT / WCB : 1;
  static constexpr int NTC = RT >= WCB ? RT / WCB : 1;
  __host__ __device__ static constexpr int rb(int w) { return w % WRB; }
  __host__ __device__ static constexpr int cb(int w) { return w / WRB; }
  __device__ __forceinline__ static bool activeD(int w) { return cb(w) * NT < DT; }
  __device__ __forceinline__ static bool activeC(int w) { return cb(w) * NTC < RT; }
};

// Row-vector slots of the partial sums in k_bwd_grad (column sums have their own array).
enum { R_EBAR = 0, R_DB1, R_RQ, R_RHO, R_DB3, R_GROW, R_NSLOT };

constexpr int kWavesG = 8;
constexpr int kThreadsG = kWavesG * 64;

template <typename TI, int C, int D> struct GradCfg {
  static constexpr int BV = grad_block<TI, D>();  // value columns per block
  static constexpr int NBH = D / BV;              // blocks per head
  static constexpr int PB = NBH >= 2 ? 2 : 1;     // blocks per pair (dO and V are loaded by pairs)
  static constexpr int RT = C / 16, DT = D / 16;
  using PT = Part<RT, DT, kWavesG>;
  static constexpr int NCB = PT::WCB;  // column blocks of the partial row sums
  // One block buffer (elements): S0^T and dS^T row blocks [BV][D], the A block [C][BV]
  // and the Delta block [C][BV] (all contiguous in memory).
  static constexpr int O_S0 = 0, O_DS = BV * D, O_A = 2 * BV * D, O_DL = O_A + C * BV, BUF = O_DL + C * BV;
  static constexpr int NBUF = 3;  // block buffers: two blocks in flight
  // One pair buffer: the dO and V column blocks [C][PB BV] of a pair of blocks. dO and V
  // are row views with long strides; a pair makes each row segment a whole 128-byte line.
  // With one block per pair, a pair is issued in the step two blocks before its own, so
  // three pair buffers are needed; with two, in the step of the previous pair's first block.
  static constexpr int PW = PB * BV, O_DO = 0, O_V = C * PW, PBUF = 2 * C * PW, NPBUF = PB == 1 ? 3 : 2;
  // Block and pair buffers are one LDS array; after the last block it holds the head-summed
  // C x C matrices and then the dq, dk rows.
  static constexpr int O_P = NBUF * BUF, SMEM = O_P + NPBUF * PBUF;
  static_assert(SMEM >= 2 * C * C && SMEM >= 2 * C * D, "end-phase scratch must fit the buffers");
  static_assert(NBH % PB == 0, "pairs do not straddle heads");
};

// Row sums of f(y, e, x) over a wave's accumulator tiles (one row tile, NT column tiles),
// stored to red[16 m + 4 g + e] (each wave owns its slots: no read-modify-write).
template <int NT, class F>
__device__ __forceinline__ void acc_rowsum(const f32x4 (&t)[NT], int m, F&& f, float* red) {
  const int l = lane_id(), g4 = (l >> 4) * 4, r16 = l & 15;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int y = 0; y < NT; ++y)
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] += f(y, e, t[y][e]);
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = row16_sum(v[e]);
  if (r16 == 0)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[16 * m + g4 + e] = v[e];
}

__device__ __forceinline__ float pick4(f32x4 v, int e) { return e == 0 ? v[0] : e == 1 ? v[1] : e == 2 ? v[2] : v[3]; }

// Elements c .. c + 3 of row r of an LDS tile (c % 4 == 0: one 8- or 16-byte read).
template <typename OT, class L> __device__ __forceinline__ f32x4 ld_row4(const OT* X, int r, int c) {
  if constexpr (sizeof(OT) == 2) {
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(X + L::at(r, c));
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  } else {
    return *reinterpret_cast<const f32x4*>(X + L::at(r, c));
  }
}

// Sum over the four lanes l % 16 + {0, 16, 32, 48} (the four row groups of an accumulator).
__device__ __forceinline__ float group4_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// Grid nc_max * Hk, key head fastest: workgroup c Hk + kh takes the gradients of the r value
// heads of key head kh in chunk c. Workgroups that start together then read the same rows
// of q, k, v and dO (all key heads of a few chunks) and neighbouring saved blocks, which
// the memory keeps in open rows: measurably faster than the chunk-fastest order.
//
// Phase 1 streams the value dimension in blocks of BV columns (direct loads, the next two
// blocks in flight while the current one is used; one workgroup barrier per block).
// A = T^T dDelta comes from the reverse sweep (in blocks of BV value columns), which formed
// it anyway and already wrote dV = diag(beta) A. Per block, with dO unscaled (the scale is applied afterwards):
//   XQ^T += S0 dO^T,  Y^T += S0 A^T,  XK^T += dS_C Delta^T  (kept transposed, D x C, so that
//   their row sums over d are sums within a lane),  P += dO Delta^T,  AD += A Delta^T,
//   A V^T on the diagonal tiles (its diagonal is rowsum(A o V)), and S0 dS_C^T on the
//   diagonal D tiles (its trace is <S0, dS_C>).
// Since (I + L) Delta is exactly the right factor of dT, dL = -stril(T^T dT T^T) reduces to
// -stril(A Delta^T) = -stril(AD), and the W-path gradient of K is -diag(beta b) Y with
// rho = -rowsum(Y o K).
// Per head, the rest is elementwise on the wave's tiles: PG = P o Gamma (scaled),
// G' = -stril(AD) o Gamma, Gb = diag(beta) G', and the gate sums
//   rowsum(P o M) = rowsum(PG o Q K^T),  colsum(P o M) = colsum(PG o Q K^T),
//   rowsum(dL o Gamma o K K^T) = rowsum(G' o K K^T),  colsum(beta_i dL o Gamma o K K^T) = colsum(Gb o K K^T),
// with Q K^T and K K^T formed once per key head. The products with K and Q are linear in
// PG and Gb and dq, dk sum over the value heads, so they run once per key head on the
// head sums: dq^T += K^T (sum PG)^T,  dk^T += Q^T (sum PG) + K^T ((sum Gb) + (sum Gb)^T).
template <typename TI, int C, int D, bool CHAIN>
__global__ __launch_bounds__(kThreadsG) void k_bwd_grad(Prob p) {
  using OT = TI;
  using CF = GradCfg<TI, C, D>;
  using PT = typename CF::PT;
  constexpr int NW = kWavesG, BV = CF::BV, NBH = CF::NBH, RT = CF::RT, NCB = CF::NCB;
  constexpr int MT = PT::MT, NT = PT::NT, NTC = PT::NTC;
  constexpr int KSC = ks_of<OT, C>(), KSB = ks_of<OT, BV>(), KSD = ks_of<OT, D>();
  using M = Mf<OT, KSB>;
  using FragB = typename M::frag;
  using LD = Swz<OT, D, true>;
  using LC = Swz<OT, C, true>;
  using LB = Swz<OT, BV, true>;
  using LP = Swz<OT, CF::PW, true>;
  using OrdD = RowOrd<OT, D>;  // storage order of the saved S^T and dS^T rows
  constexpr int RS = NCB * C;  // one partial-sum slot

  __shared__ __align__(16) OT sK[C * D];
  __shared__ __align__(16) OT sQ[C * D];
  // block buffers (job j uses block buffer j % NBUF), then pair buffers (pair q uses q % NPBUF)
  __shared__ __align__(16) OT smem[CF::SMEM];
  auto sB = [&](int i) { return smem + i * CF::BUF; };
  auto sP = [&](int i) { return smem + CF::O_P + i * CF::PBUF; };
  __shared__ __align__(16) float sgb[3][2 * C];        // gate records (head hh uses sgb[hh % 3])
  __shared__ float red[2][R_NSLOT * RS];
  __shared__ float redc[2][RT * C];  // column sums of PG o QK^T + Gb o KK^T per row tile
  __shared__ float swv[2][NW];
  // dbeta and dg of up to GRM value heads, written at the end as the key head's r columns
  // of each row (the rows of dg and dbeta are tokens: one head's column alone is a strided
  // run of single floats)
  constexpr int GRM = 4;
  __shared__ float sgo[2][GRM][C];
  // q/k L2 normalisation: per dq, dk row the dot of the normalised row with its gradient,
  // and the row's factor (the norm's backward is applied at the store)
  __shared__ float sdot[2 * C], srf[2 * C];
  __shared__ __align__(16) float sdl[3][C];  // d log g / d alpha per row (gate chain), with sgb

  const int kh = blockIdx.x % p.Hk, c = blockIdx.x / p.Hk;
  const ChunkInfo ci = p.chunks[c];
  if (ci.seq < 0) return;
  const int n = ci.len;
  const int w = wave_id(), lane = lane_id(), g4 = (lane >> 4) * 4, r16 = lane & 15;

  const int h0 = kh * p.r;
  constexpr int NH = NW / 2;  // the two halves of the waves load different tensors
  constexpr int PB = CF::PB, PW = CF::PW;
  const int wh = w % NH;
  const bool lo = w < NH;  // first half: A and dO; second half: Delta and V
  TileDma<BV, D, NW, OT, true> dmS;   // S0^T, dS^T row blocks (every wave)
  TileDma<C, BV, NH, OT, true> dmAL;  // A block (first half) or Delta block (second half)
  TileDma<C, PW, NH, OT, true> dmP;   // dO (first half) or V (second half) for a pair of blocks
  TileDma<C, D, NW, OT, true> dmD;    // K, Q
  TileDma<1, 2 * C, NW, float> dmG;  // gate record
  TileDma<1, C, NW, float> dmGc;     // its d log g / d alpha row (gate chain only)
  dmS.init(w);
  dmAL.init(wh);
  dmP.init(wh);
  dmD.init(w);
  dmG.init(w);
  dmGc.init(w);
  // The item's sources. The saved blocks of the key head's r value heads are consecutive
  // (chunk, head, block order), so job j = (head h0 + j / NBH, block j % NBH) finds its S^T
  // and dS^T blocks j BV D elements, and its A and Delta blocks j C BV elements, past the
  // first head's first block; pair q finds its dO and V columns q PW columns past the first
  // head's. One resource per tensor serves every job (byte offsets go in the instructions'
  // scalar offset); only the A and Delta blocks, whose rows past the chunk's end must read
  // as zero, take a resource of their own per job.
  const size_t ch0 = ch_idx(p, c, h0);
  constexpr uint32_t SBB = BV * D * sizeof(OT), ABB = C * BV * sizeof(OT);
  const uint32_t head_saved = (uint32_t)(p.r * D * D * sizeof(OT));
  const i32x4 rS = buf_rsrc((const OT*)p.sv_S + ch0 * D * D, head_saved);
  const i32x4 rDS = buf_rsrc((const OT*)p.ws_dS + ch0 * D * D, head_saved);
  const uint64_t aAL =
      reinterpret_cast<uint64_t>((lo ? (const OT*)p.ws_A : (const OT*)p.sv_D) + ch0 * C * D);
  const int64_t prs = lo ? p.dO_rs : p.v_rs;
  const uint32_t prsb = (uint32_t)(prs * (int64_t)sizeof(OT));
  const i32x4 rP = buf_rsrc((lo ? (const OT*)p.dO : (const OT*)p.v) + (int64_t)ci.t0 * prs + h0 * D, (uint32_t)n * prsb);
  const i32x4 rG = buf_rsrc(p.sv_gb + ch0 * kGateRows * C, (uint32_t)(p.r * kGateRows * C * 4));
  const int njobs = p.r * NBH, npairs = njobs / PB;
  // Job j goes into sB(j % NBUF); the first block of a head also brings the head's gate
  // record. Job j's loads are issued in the step of job j - 2, in parts spread over the step
  // (a long run of loads would stall the issuing wave). Pair q (the dO and V columns of jobs
  // q PB .. q PB + PB - 1) goes into sP(q % NPBUF) and is issued after that step's job loads
  // in the step of job (q - 1) PB (PB = 2) or q - 2 (PB = 1). Before the first step: job 0,
  // pair 0, job 1 (and pair 1 when PB = 1).
  auto issue_part = [&](int j, int part) {
    const int hh = j / NBH, blk = j % NBH;
    OT* b = sB(j % CF::NBUF);
    if (part == 0) {
      dmS.template issue_rs<true>(b + CF::O_S0, rS, D * sizeof(OT), (uint32_t)j * SBB, w);
      if (blk == 0) {
        const uint32_t go = (uint32_t)(hh * kGateRows * C * 4);
        dmG.template issue_rs<true>(sgb[hh % 3], rG, 0, go, w);  // gamma, beta
        if constexpr (CHAIN) dmGc.template issue_rs<true>(sdl[hh % 3], rG, 0, go + 4 * C * 4, w);
      }
    } else if (part == 1) {
      dmS.template issue_rs<true>(b + CF::O_DS, rDS, D * sizeof(OT), (uint32_t)j * SBB, w);
    } else {
      const uint64_t a = aAL + (uint64_t)j * ABB;
      const i32x4 r = {__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a),
                       __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(a >> 32)),
                       (int32_t)((uint32_t)n * BV * sizeof(OT)), 0x00020000};
      dmAL.template issue_rs<true>(b + (lo ? CF::O_A : CF::O_DL), r, BV * sizeof(OT), 0, wh);
    }
  };
  auto issue_job = [&](int j) {
    for (int part = 0; part < 3; ++part) issue_part(j, part);
  };
  auto issue_pair = [&](int q) {
    OT* b = sP(q % CF::NPBUF);
    dmP.template issue_rs<true>(b + (lo ? CF::O_DO : CF::O_V), rP, prsb, (uint32_t)(q * PW * sizeof(OT)), wh);
  };
  // This wave's load instructions of job j, of a pair, and of the step of job j.
  auto job_loads = [&](int j) {
    return j < njobs ? 2 * dmS.count(w) + dmAL.count(wh) +
                           (j % NBH == 0 ? dmG.count(w) + (CHAIN ? dmGc.count(w) : 0) : 0)
                     : 0;
  };
  const int pair_loads = dmP.count(wh);
  constexpr bool UNI = decltype(dmS)::CNT >= 0 && decltype(dmAL)::CNT >= 0 && decltype(dmP)::CNT >= 0;
  auto step_loads = [&](int j) {  // issued in the step of job j: job j + 2 and, maybe, a pair
    const int q = PB == 1 ? j + 2 : j / PB + 1;
    return job_loads(j + 2) + ((j % PB == 0 && q < npairs) ? pair_loads : 0);
  };
  // every load of the item is non-temporal (each byte is read once per item; 8% faster)
  dmD.template issue<true>(sK, (const OT*)p.ku + (int64_t)ci.t0 * p.ku_rs + kh * D, p.ku_rs, n, w);
  dmD.template issue<true>(sQ, (const OT*)p.qu + (int64_t)ci.t0 * p.qu_rs + kh * D, p.qu_rs, n, w);
  issue_job(0);
  issue_pair(0);
  if (1 < njobs) {
    issue_job(1);
    if (PB == 1) issue_pair(1);
  }

  const bool aD = PT::activeD(w), aC = PT::activeC(w);
  const int rb = PT::rb(w), cb = PT::cb(w);
  const int m0 = rb * MT, nD = cb * NT, nC = cb * NTC;  // first row tile, first D tile, first C tile
  // The wave's diagonal C x C tile (row tile m0 + dmi = column tile nC + dyc), if it has one.
  int dmi = -1;
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int yc = 0; yc < NTC; ++yc)
      if (m0 + mi == nC + yc) dmi = mi;
  const bool dgw = aC && dmi >= 0;
  // The wave that finishes each head's per-row gate gradients: the highest-numbered wave
  // whose C x C tiles all lie above the diagonal (it skips their products and elementwise
  // work), else the last wave.
  constexpr int FIN = [] {
    for (int v = NW - 1; v >= 0; --v) {
      const int r0 = PT::rb(v) * MT, c0 = PT::cb(v) * NTC;
      if (r0 + MT - 1 < c0) return v;
    }
    return NW - 1;
  }();

  // dq^T, dk^T of the key head on the wave's D x C tiles [y][mi], summed over its value
  // heads in order: lane (g, r) element e holds row i = 16 (m0 + mi) + r, column
  // d = 16 (nD + y) + 4 g + e.
  f32x4 dqt[NT][MT], dkt[NT][MT];
  zero(dqt);
  zero(dkt);
  f32x4 QKt[MT][NTC], KKt[MT][NTC], PGs[MT][NTC], Gbs[MT][NTC];  // Q K^T, K K^T, sum PG, sum Gb
  zero(QKt);
  zero(KKt);
  zero(PGs);
  zero(Gbs);

  // Per-row gate gradients of head fh (dg, dbeta from the head's partial row sums, with the
  // reverse scan of d log g), done by one wave. Head fh's partials stay in their slots (parity
  // fh & 1) until head fh + 2 zeroes them, so with two or more value blocks per head the wave
  // does this inside the first block step of head fh + 1, after its own products, while the
  // other waves work on that step (the next block step's barrier then orders its reads before
  // that zeroing), and the last head's in the end phase. With one block per head it follows
  // the head's elementwise phase behind a barrier.
  auto finish = [&](int fh) {
    const int hh = fh, h = h0 + hh, par = hh & 1;
    const float* gam = sgb[hh % 3];
    const float* bet = gam + C;
    const float gn = gam[C - 1];
    const float* redh = red[par];
    const float* redch = redc[par];
    const bool ok = lane < C;
    const int i = ok ? lane : C - 1;  // lanes past C read a valid row and contribute nothing
    // every partial sum first (independent reads), then the sums in a fixed order
    float part[R_NSLOT][NCB], pc[RT];
#pragma unroll
    for (int sl = 0; sl < R_NSLOT; ++sl)
#pragma unroll
      for (int q = 0; q < NCB; ++q) part[sl][q] = redh[sl * RS + q * C + i];
#pragma unroll
    for (int m = 0; m < RT; ++m) pc[m] = redch[m * C + i];
    const float gi = gam[i], gprev = i > 0 ? gam[i - 1] : 0.f, bei = bet[i];
    float rv[R_NSLOT], gcol = 0.f;
#pragma unroll
    for (int sl = 0; sl < R_NSLOT; ++sl) {
      float a = 0.f;
#pragma unroll
      for (int q = 0; q < NCB; ++q) a += part[sl][q];
      rv[sl] = ok ? a : 0.f;
    }
#pragma unroll
    for (int m = 0; m < RT; ++m) gcol += pc[m];
    if (!ok) gcol = 0.f;
    const float bi = ok ? __builtin_amdgcn_exp2f(gi) : 0.f, be = ok ? bei : 0.f;
    float dgam = 0.f;
    if (ok) dgam = bi * rv[R_RQ] + be * bi * rv[R_RHO] - rv[R_EBAR] + rv[R_GROW] + be * rv[R_DB3] - gcol;
    const float ebsum = wave_sum(rv[R_EBAR]);
    if (lane == n - 1) {
      float st = 0.f;
#pragma unroll
      for (int k = 0; k < NW; ++k) st += swv[par][k];
      dgam += __builtin_amdgcn_exp2f(gn) * st + ebsum;
    }
    const float dlg = wave_rscan_incl(dgam);
    if (lane < n) {  // (lane < n implies lane < C: i is the lane)
      float db = rv[R_DB1] + bi * rv[R_RHO] + rv[R_DB3];
      // dg = dlog g / g, with 1 / g_i = 2^(gamma_{i-1} - gamma_i) from the record
      float dgv = dlg * __builtin_amdgcn_exp2f(gprev - gi);
      if constexpr (CHAIN) {  // gate chain: d alpha = dlog g * dlog g / d alpha (from the record), d beta_raw = dbeta beta (1 - beta)
        dgv = dlg * sdl[hh % 3][i];
        db *= be * (1.f - be);
      }
      if (p.r <= GRM) {
        // the row offset is formed here rather than kept live across the item's loops
        int li = i;
        asm volatile("" : "+v"(li));
        sgo[0][hh][li] = db;
        sgo[1][hh][li] = dgv;
      } else {
        int li = i;  // the row offset is formed here, not kept live across the item
        asm volatile("" : "+v"(li));
        const int64_t row = (int64_t)(ci.t0 + li) * p.Hv + h;
        p.dbeta[row] = db;
        p.dg[row] = dgv;
      }
    }
  };

  for (int hh = 0; hh < p.r; ++hh) {
    const int h = h0 + hh, par = hh & 1;
    const float* gam = sgb[hh % 3];  // log2 units
    const float* bet = gam + C;
    float* redh = red[par];
    float* redch = redc[par];
    for (int i = threadIdx.x; i < R_NSLOT * RS; i += kThreadsG) redh[i] = 0.f;
    for (int i = threadIdx.x; i < RT * C; i += kThreadsG) redch[i] = 0.f;

    // ---- phase 1: stream the value dimension
    f32x4 XQt[NT][MT], XKt[NT][MT], Yt[NT][MT], P[MT][NTC], AD[MT][NTC];
    f32x4 AV = {0.f, 0.f, 0.f, 0.f}, SD = {0.f, 0.f, 0.f, 0.f};
    zero(XQt);
    zero(XKt);
    zero(Yt);
    zero(P);
    zero(AD);
    auto block_step = [&](auto bc) {
      constexpr int b = decltype(bc)::value;
      const int j = hh * NBH + b;
      const OT* cur = sB(j % CF::NBUF);
      const OT* curp = sP((j / PB) % CF::NPBUF);
      constexpr int sp = (b % PB) * (BV / KSB);  // this block's first contraction step within the pair
      // Job j and its pair are done once at most the loads issued after them are outstanding:
      // job 1 before the first step, else the previous step's loads (job j + 1, and the pair
      // issued with it). Where every wave issues the same loads per tile, that count is a
      // constant of the block (the gate record's load, issued by wave 0 alone, is not
      // counted: wave 0 then waits for one load more than it needs to).
      if constexpr (UNI) {
        constexpr int K = 2 * decltype(dmS)::CNT + decltype(dmAL)::CNT +
                          ((((b == 0 ? NBH : b) - 1) % PB == 0) ? decltype(dmP)::CNT : 0);
        if (b + 1 < NBH || hh + 1 < p.r)
          dma_wait_keep(K);
        else
          dma_wait_keep(0);
      } else {
        dma_wait_keep(j == 0 ? job_loads(1) + (PB == 1 && 1 < npairs ? pair_loads : 0) : step_loads(j - 1));
      }
      lds_barrier();  // job j (and K, Q, gates with it) is in LDS; every wave is done with job j - 1
      const bool nxt2 = j + 2 < njobs;  // every wave issues every part (the wait counts rely on it)
      if (nxt2) {
        issue_part(j + 2, 0);
        issue_part(j + 2, 1);
      }
      if (b == 0 && hh == 0 && aC) {  // Q K^T and K K^T of the key head on this wave's C x C tiles
        f32x4 G2[2 * MT][NTC];
        zero(G2);
        wave_mm<OT, D, 2 * MT, NTC>(
            G2, [&](int m, int s) { return ld_n<OT, KSD, STD, LD>(m < MT ? sQ : sK, 16 * (m0 + m % MT), s); },
            [&](int yc, int s) { return ld_n<OT, KSD, STD, LD>(sK, 16 * (nC + yc), s); });
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
#pragma unroll
          for (int yc = 0; yc < NTC; ++yc) {
            QKt[mi][yc] = G2[mi][yc];
            KKt[mi][yc] = G2[MT + mi][yc];
          }
      }
      const OT* sS0 = cur + CF::O_S0;
      const OT* sDS = cur + CF::O_DS;
      const OT* sA = cur + CF::O_A;
      const OT* sDL = cur + CF::O_DL;
      const OT* sDO = curp + CF::O_DO;
      const OT* sV = curp + CF::O_V;
#pragma unroll
      for (int s = 0; s < BV / KSB; ++s) {
        FragB fo[MT], fa[MT];  // dO and A rows of the wave's row tiles (A operands)
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
          fo[mi] = ld_n<OT, KSB, STD, LP>(sDO, 16 * (m0 + mi), sp + s);
          fa[mi] = ld_n<OT, KSB, STD, LB>(sA, 16 * (m0 + mi), s);
        }
        if (aD) {
          FragB fs[NT], fds[NT], fd[MT];
#pragma unroll
          for (int y = 0; y < NT; ++y) {
            fs[y] = ld_t<OT, KSB, STD, LD, OrdD>(sS0, 16 * (nD + y), s);
            fds[y] = ld_t<OT, KSB, STD, LD, OrdD>(sDS, 16 * (nD + y), s);
          }
#pragma unroll
          for (int mi = 0; mi < MT; ++mi) fd[mi] = ld_n<OT, KSB, STD, LB>(sDL, 16 * (m0 + mi), s);
#pragma unroll
          for (int y = 0; y < NT; ++y)
#pragma unroll
            for (int mi = 0; mi < MT; ++mi) {
              XQt[y][mi] = M::run(fs[y], fo[mi], XQt[y][mi]);
              Yt[y][mi] = M::run(fs[y], fa[mi], Yt[y][mi]);
              XKt[y][mi] = M::run(fds[y], fd[mi], XKt[y][mi]);
            }
          if (rb == 0)  // S0 dS_C^T on the diagonal D tiles (the waves of row block 0 cover every d)
#pragma unroll
            for (int y = 0; y < NT; ++y) SD = M::run(fs[y], fds[y], SD);
        }
        if (s == 0) {
          if (nxt2) issue_part(j + 2, 2);
          const int q = PB == 1 ? j + 2 : j / PB + 1;
          if constexpr (b % PB == 0)
            if (q < npairs) issue_pair(q);
        }
        if (aC) {
          FragB fb[NTC];  // Delta rows of the wave's C tiles (B operands over v)
#pragma unroll
          for (int yc = 0; yc < NTC; ++yc) fb[yc] = ld_n<OT, KSB, STD, LB>(sDL, 16 * (nC + yc), s);
#pragma unroll
          for (int mi = 0; mi < MT; ++mi)
#pragma unroll
            for (int yc = 0; yc < NTC; ++yc)
              if (m0 + mi >= nC + yc) {  // tiles above the diagonal are masked to zero later
                P[mi][yc] = M::run(fo[mi], fb[yc], P[mi][yc]);
                AD[mi][yc] = M::run(fa[mi], fb[yc], AD[mi][yc]);
              }
          if (dgw) {  // A V^T on the diagonal tile
            FragB fad = fa[0];
#pragma unroll
            for (int mi = 1; mi < MT; ++mi)
              if (dmi == mi) fad = fa[mi];
            AV = M::run(fad, ld_n<OT, KSB, STD, LP>(sV, 16 * (m0 + dmi), sp + s), AV);
          }
        }
      }
      if constexpr (NBH >= 2 && b == 0)  // the previous head's rows, off the barrier path (see finish)
        if (hh > 0 && w == FIN) finish(hh - 1);
    };
    static_for<NBH>(block_step);

    // ---- phase 2 of the head: elementwise on the wave's tiles
    const float sc = p.scale, gn = gam[C - 1];
    float bb[MT][4];  // beta of the rows 16 (m0 + mi) + 4 g + e of the C x C tiles
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int e = 0; e < 4; ++e) bb[mi][e] = bet[16 * (m0 + mi) + g4 + e];
    if (dgw) {  // lane (g, r) holds (A V^T)[4 g + e][r]: the diagonal is e = r - 4 g
      const int e = r16 - g4;
      if (e >= 0 && e < 4) redh[R_DB1 * RS + 16 * (m0 + dmi) + r16] = pick4(AV, e);
    }
    if (aC) {
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        float grow[4] = {0.f, 0.f, 0.f, 0.f}, db3[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int yc = 0; yc < NTC; ++yc) {
          // P o Gamma and dL vanish above the diagonal (tile row < tile column, wave-uniform):
          // such tiles add nothing; only the diagonal tile needs an element mask
          const int tm = m0 + mi, tn = nC + yc;
          if (tm < tn) continue;
          float col = 0.f;
          const int jj = 16 * tn + r16;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 16 * tm + g4 + e;
            const float gd = __builtin_amdgcn_exp2f(gam[i] - gam[jj]);
            float pg = sc * P[mi][yc][e] * gd, gp = -AD[mi][yc][e] * gd;
            if (tm == tn) {
              pg = g4 + e >= r16 ? pg : 0.f;
              gp = g4 + e > r16 ? gp : 0.f;
            }
            const float gb = bb[mi][e] * gp;
            PGs[mi][yc][e] += pg;
            Gbs[mi][yc][e] += gb;
            grow[e] += pg * QKt[mi][yc][e];
            db3[e] += gp * KKt[mi][yc][e];
            col += pg * QKt[mi][yc][e] + gb * KKt[mi][yc][e];
          }
          col += __shfl_xor(col, 16);
          col += __shfl_xor(col, 32);
          if (lane < 16) redch[(m0 + mi) * C + jj] = col;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          grow[e] = row16_sum(grow[e]);
          db3[e] = row16_sum(db3[e]);
        }
        if (r16 == 0)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 16 * (m0 + mi) + g4 + e;
            redh[R_GROW * RS + cb * C + i] = grow[e];
            redh[R_DB3 * RS + cb * C + i] = db3[e];
          }
      }
    }
    if (aD) {
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        const int i = 16 * (m0 + mi) + r16;  // this lane's row of the chunk
        const float gi = gam[i];
        const float exi = __builtin_amdgcn_exp2f(gn - gi), bxi = __builtin_amdgcn_exp2f(gi), bbi = bet[i];
        float pe = 0.f, pq = 0.f, pr = 0.f;  // partial row sums over this lane's d
#pragma unroll
        for (int y = 0; y < NT; ++y) {
          const f32x4 kv = ld_row4<OT, LD>(sK, i, 16 * (nD + y) + g4);
          const f32x4 qv = ld_row4<OT, LD>(sQ, i, 16 * (nD + y) + g4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pe += XKt[y][mi][e] * kv[e];
            pq += XQt[y][mi][e] * qv[e];
            pr += Yt[y][mi][e] * kv[e];
            dkt[y][mi][e] += exi * XKt[y][mi][e] - bbi * bxi * Yt[y][mi][e];
            dqt[y][mi][e] += sc * bxi * XQt[y][mi][e];
          }
        }
        pe = group4_sum(pe);
        pq = group4_sum(pq);
        pr = group4_sum(pr);
        if (lane < 16) {
          redh[R_EBAR * RS + cb * C + i] = exi * pe;
          redh[R_RQ * RS + cb * C + i] = sc * pq;
          redh[R_RHO * RS + cb * C + i] = -pr;
        }
      }
    }
    float sdot = 0.f;  // the trace of SD
    {
      const int e = r16 - g4;
      if (e >= 0 && e < 4) sdot = pick4(SD, e);
    }
    sdot = wave_sum(sdot);
    if (lane == 0) swv[par][w] = sdot;
    if constexpr (NBH < 2) {  // one block per head: no later block barrier would separate the
                              // finishing wave's reads from the zeroing of these slots two heads on
      lds_barrier();
      if (w == FIN) finish(hh);
    }
  }

  // ---- the key head's products with K and Q on the head sums
  OT* const sPGs = smem;          // sum PG    [C][C]
  OT* const sGbs = smem + C * C;  // sum Gb    [C][C]
  if (aC) {
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int yc = 0; yc < NTC; ++yc)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * (m0 + mi) + g4 + e, jj = 16 * (nC + yc) + r16;
          sPGs[LC::at(i, jj)] = (OT)PGs[mi][yc][e];
          sGbs[LC::at(i, jj)] = (OT)Gbs[mi][yc][e];
        }
  }
  lds_barrier();  // (also: every head's partial sums are complete)
  if constexpr (NBH >= 2)
    if (w == FIN) finish(p.r - 1);
  if (aD) {
    auto fK = [&](int y, int s) { return ld_t<OT, KSC, STD, LD>(sK, 16 * (nD + y), s); };  // K^T rows d
    // dq^T += K^T (sum PG)^T
    wave_mm<OT, C, NT, MT>(dqt, fK, [&](int mi, int s) { return ld_n<OT, KSC, STD, LC>(sPGs, 16 * (m0 + mi), s); });
    // dk^T += Q^T (sum PG) + K^T (sum Gb) + K^T (sum Gb)^T
    wave_mm<OT, C, NT, MT>(dkt, [&](int y, int s) { return ld_t<OT, KSC, STD, LD>(sQ, 16 * (nD + y), s); },
                           [&](int mi, int s) { return ld_t<OT, KSC, STD, LC>(sPGs, 16 * (m0 + mi), s); });
    wave_mm<OT, C, NT, MT>(dkt, fK, [&](int mi, int s) { return ld_t<OT, KSC, STD, LC>(sGbs, 16 * (m0 + mi), s); });
    wave_mm<OT, C, NT, MT>(dkt, fK, [&](int mi, int s) { return ld_n<OT, KSC, STD, LC>(sGbs, 16 * (m0 + mi), s); });
  }
  lds_barrier();
  // dq, dk of the key head: rows through LDS, 16-byte stores
  {
    // rows [2C][D] (dq, then dk) in a swizzled layout: a plain row-major tile would put the
    // 16 rows of a wave's 8-byte writes in the same banks
    using LS = Swz<TI, D>;
    TI* st = (TI*)smem;
    if (aD) {
#pragma unroll
      for (int mi = 0; mi < MT; ++mi)
#pragma unroll
        for (int y = 0; y < NT; ++y) {
          const int i = 16 * (m0 + mi) + r16, d = 16 * (nD + y) + g4;
          store4b(st + LS::at(i, d), dqt[y][mi]);
          store4b(st + LS::at(C + i, d), dkt[y][mi]);
        }
    }
    lds_barrier();
    using V = Vec16<TI>;
    constexpr int VPR = D / V::N;
    const bool l2 = p.sv_qn != nullptr;
    if (l2) {  // x_hat . dx_hat per row of dq, then of dk: PPR lanes per row, one 16-byte
               // piece each, RPW rows per wave and pass
      // The rows' norm factors, one load per row (thread rr: row rr % C of q, then of k), in
      // flight during the dots and written after them (loaded one at a time by one lane, the
      // loads' latencies had added a quarter to the kernel's time)
      float rfv = 0.f;
      const int fr = threadIdx.x;
      if (fr < 2 * C && fr % C < n) rfv = p.sv_r[((int64_t)(ci.t0 + fr % C) * p.Hk + kh) * 2 + (fr < C ? 0 : 1)];
      constexpr int PPR = D / V::N, RPW = 64 / PPR;
      const int sub = lane % PPR;
      for (int r0 = w * RPW; r0 < 2 * C; r0 += NW * RPW) {
        const int rr = r0 + lane / PPR;
        const bool okr = rr < 2 * C;  // (every lane takes part in the group sum)
        const int rc = okr ? rr : 0, i = rc % C;
        const OT* X = rc < C ? sQ : sK;  // the normalised rows
        const typename V::type xv = *reinterpret_cast<const typename V::type*>(X + LD::at(i, sub * V::N));
        const typename V::type dv = *reinterpret_cast<const typename V::type*>(st + LS::at(rc, sub * V::N));
        float x = 0.f;
#pragma unroll
        for (int e = 0; e < V::N; ++e) x += (float)xv[e] * (float)dv[e];
#pragma unroll
        for (int o = 1; o < PPR; o <<= 1) x += __shfl_xor(x, o);
        if (okr && sub == 0) sdot[rr] = x;
      }
      if (fr < 2 * C) srf[fr] = rfv;
      lds_barrier();
    }
    TI* dq = (TI*)p.dq + (int64_t)ci.t0 * p.dq_rs + kh * D;
    TI* dk = (TI*)p.dk + (int64_t)ci.t0 * p.dk_rs + kh * D;
    for (int idx = threadIdx.x; idx < 2 * C * VPR; idx += kThreadsG) {
      const int r = idx / VPR, cc = (idx % VPR) * V::N;
      const int i = r % C;
      if (i < n) {
        TI* dst = r < C ? dq + (int64_t)i * p.dq_rs + cc : dk + (int64_t)i * p.dk_rs + cc;
        typename V::type val = *reinterpret_cast<const typename V::type*>(st + LS::at(r, cc));
        if (l2) {  // dx = r (dx_hat - x_hat (x_hat . dx_hat)), the gradient of the raw row
          const OT* X = r < C ? sQ : sK;
          const typename V::type xv = *reinterpret_cast<const typename V::type*>(X + LD::at(i, cc));
          const float dt = sdot[r], rf = srf[r];
#pragma unroll
          for (int e = 0; e < V::N; ++e) val[e] = (TI)(rf * ((float)val[e] - (float)xv[e] * dt));
        }
        store_nt(reinterpret_cast<typename V::type*>(dst), val);  // non-temporal: slightly faster
      }
    }
    if (p.r <= GRM) {  // dbeta, dg: row i, heads h0 .. h0 + r - 1
      const int nr = n * p.r;
      for (int idx = threadIdx.x; idx < 2 * nr; idx += kThreadsG) {
        const int a = idx >= nr, q = idx - a * nr, i = q / p.r, hh = q - i * p.r;
        float* dst = a ? p.dg : p.dbeta;
        dst[(int64_t)(ci.t0 + i) * p.Hv + h0 + hh] = sgo[a][hh][i];
      }
    }
  }
}

template <typename TI, int C, int D>
static hipError_t bwd_seq(const Prob& p, hipStream_t s) {
  using CF = BwCfg<TI, C, D>;
  // the chunk table is the forward's, saved with the chunk states
  if (p.N > 0)
    traced("k_bwd_sweep", s,
           [&] { k_bwd_sweep<TI, C, D><<<xcd_grid(p.N * p.Hk, p.r), CF::NW * 64, 0, s>>>(p); });
  if (p.nc_max > 0)
    traced("k_bwd_grad", s, [&] {
      if (p.a_log)
        k_bwd_grad<TI, C, D, true><<<p.nc_max * p.Hk, kThreadsG, 0, s>>>(p);
      else
        k_bwd_grad<TI, C, D, false><<<p.nc_max * p.Hk, kThreadsG, 0, s>>>(p);
    });
  return hipGetLastError();
}

template <typename TI, int C>
static hipError_t bwd_d(const Prob& p, hipStream_t s) {
  switch (p.D) {
    case 16: return bwd_seq<TI, C, 16>(p, s);
    case 32: return bwd_seq<TI, C, 32>(p, s);
    case 64:
      if constexpr (sizeof(TI) == 4 && C == 64)
        return hipErrorInvalidValue;  // rejected on the host (LDS)
      else
        return bwd_seq<TI, C, 64>(p, s);
    case 128:
      if constexpr (sizeof(TI) == 4 && C == 64)
        return hipErrorInvalidValue;
      else
        return bwd_seq<TI, C, 128>(p, s);
  }
  return hipErrorInvalidValue;
}

template <typename TI>
static hipError_t bwd_c(const Prob& p, hipStream_t s) {
  return p.C == 16 ? bwd_d<TI, 16>(p, s) : bwd_d<TI, 64>(p, s);
}

hipError_t launch_backward(const Prob& p, int dtype, hipStream_t s) {
  return dtype == 0 ? bwd_c<float>(p, s) : bwd_c<__bf16>(p, s);
}

}  // namespace gdn
