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

template <typename OT, int K, int MT, int NT, class FA, class FB>
__device__ __forceinline__ void wave_mm_cm(f32x4 (&acc)[NT][MT], FA&& fa, FB&& fb) {
  constexpr int KS = ks_of<OT, K>();
  using M = Mf<OT, KS>;
#pragma unroll
  for (int s = 0; s < K / KS; ++s) {
    typename M::frag b[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) b[n] = fb(n, s);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const typename M::frag a = fa(m, s);
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n][m] = M::run(a, b[n], acc[n][m]);
    }
  }
}

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
  using LD = Swz<OT, D>;
  using LC = Swz<OT, C>;
  using FragD = typename Mf<OT, KSD>::frag;
  using FragC = typename Mf<OT, KSC>::frag;
  __shared__ __align__(16) OT sbuf[2][CF::BUF];
  __shared__ __align__(16) float sgb[2][2 * C];
  __shared__ __align__(16) OT stg[C * CF::LSO];  // the chunk's dV rows, all D columns

  int grp, hh;
  if (!xcd_group(blockIdx.x, p.N * p.Hk, p.r, grp, hh)) return;
  const int n = grp / p.Hk, kh = grp % p.Hk, h = kh * p.r + hh;
  const size_t nh = (size_t)n * p.Hv + h;
  const int c0 = p.seq_chunk[n], c1 = p.seq_chunk[n + 1];
  int64_t sa, sb;  // rows of the sequence; chunk c starts at sa + (c - c0) C (as in the chunk table)
  seq_bounds(p, n, sa, sb);
  const int w = wave_id(), l = lane_id(), g4 = (l >> 4) * 4, r16 = l & 15;
  const int v0 = w * WC;

  TileDma<C, D, NW, OT> dmD;         // K, Q, dO
  TileDma<C, C, NW, OT> dmC;         // T, M
  TileDma<1, 2 * C, NW, float> dmG;  // gate record
  dmD.init(w);
  dmC.init(w);
  dmG.init(w);
  auto issue = [&](int c, int buf) {
    const int64_t t0 = sa + (int64_t)(c - c0) * C;
    const int len = (int)(sb - t0 < C ? sb - t0 : C);
    const size_t ch = ch_idx(p, c, h);
    OT* b = sbuf[buf];
    dmD.issue(b + CF::O_K, (const OT*)p.k + t0 * p.k_rs + kh * D, p.k_rs, len, w);
    dmD.issue(b + CF::O_Q, (const OT*)p.q + t0 * p.q_rs + kh * D, p.q_rs, len, w);
    dmD.issue(b + CF::O_O, (const OT*)p.dO + t0 * p.dO_rs + h * D, p.dO_rs, len, w);
    dmC.issue(b + CF::O_T, (const OT*)p.sv_T + ch * C * C, C, C, w);
    dmC.issue(b + CF::O_M, (const OT*)p.sv_M + ch * C * C, C, C, w);
    dmG.issue(sgb[buf], p.sv_gb + ch * 2 * C, 2 * C, 1, w);
  };

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
    const float* gam = sgb[buf];  // log2 units
    const float* bet = gam + C;
    const float gn = gam[C - 1], bn = __builtin_amdgcn_exp2f(gn), sc = p.scale;
    float ex[RT][4], sbx[RT][4], nbb[RT][4];  // e_i, scale b_i, -beta_i b_i
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const f32x4 gv = *reinterpret_cast<const f32x4*>(gam + 16 * t + g4);
      const f32x4 bv = *reinterpret_cast<const f32x4*>(bet + 16 * t + g4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float b = __builtin_amdgcn_exp2f(gv[e]);
        ex[t][e] = __builtin_amdgcn_exp2f(gn - gv[e]);
        sbx[t][e] = sc * b;
        nbb[t][e] = -bv[e] * b;
      }
    }
    // dS_C's fragments (B operand over d) and its saved copy dS^T[v][d]
    FragD dSb[CT][NSD];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int s = 0; s < NSD; ++s) dSb[ct][s] = from_acc<OT, KSD>(dS[ct], s, Ident{});
    save_rows_b<OT, D, CT, DT, NSD>((OT*)p.ws_dS + ch * D * D, v0, dS, dSb);
    // dDelta = e o (K dS) + scale M^T dO
    f32x4 dD[CT][RT];
    {
      f32x4 KdS[RT][CT], MdO[RT][CT];
      zero(KdS);
      zero(MdO);
      wave_mm<OT, D, RT, CT>(KdS, [&](int m, int s) { return ld_n<OT, KSD, ACC, LD>(sK, 16 * m, s); },
                             [&](int j, int s) { return dSb[j][s]; });
      wave_mm<OT, C, RT, CT>(MdO, [&](int m, int s) { return ld_t<OT, KSC, STD, LC>(sM, 16 * m, s); },
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
    // A = T^T dDelta: the gradient kernel's A (saved as A^T[v][i]) and dV = diag(beta) A
    f32x4 Z[CT][RT];
    zero(Z);
    wave_mm_cm<OT, C, RT, CT>(Z, [&](int m, int s) { return ld_t<OT, KSC, ACC, LC>(sT, 16 * m, s); },
                              [&](int j, int s) { return dDb[j][s]; });
    {
      FragC Ab[CT][NSC];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int s = 0; s < NSC; ++s) Ab[ct][s] = from_acc<OT, KSC>(Z[ct], s, Ident{});
      save_rows_b<OT, C, CT, RT, NSC>((OT*)p.ws_At + ch * D * C, v0, Z, Ab);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const f32x4 bv = *reinterpret_cast<const f32x4*>(bet + 16 * t + g4);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e) stg[(16 * t + g4 + e) * CF::LSO + v0 + 16 * ct + r16] = (OT)(bv[e] * Z[ct][t][e]);
      }
    }
    lds_barrier();  // the chunk's dV rows are staged
    {  // full dV rows, 16-byte stores spread over every wave
      using V = Vec16<OT>;
      constexpr int VPR = D / CE;
      TI* dv = (TI*)p.dv + t0 * p.dv_rs + h * D;
#pragma unroll
      for (int idx = threadIdx.x; idx < C * VPR; idx += NW * 64) {
        const int i = idx / VPR, q = idx % VPR;
        if (i < len)
          *reinterpret_cast<typename V::type*>(dv + (int64_t)i * p.dv_rs + q * CE) =
              *reinterpret_cast<const typename V::type*>(stg + i * CF::LSO + q * CE);
      }
    }
    // dS <- b_n dS + Q^T (scale b o dO) - K^T (beta b o Z)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dS[ct][dt] *= bn;
    wave_mm_cm<OT, C, DT, CT>(
        dS, [&](int m, int s) { return ld_t<OT, KSC, ACC, LD>(sQ, 16 * m, s); },
        [&](int j, int s) { return scale_acc<OT, KSC, RT>(ld_t<OT, KSC, ACC, LD>(sO, v0 + 16 * j, s), s, sbx); });
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
// Tile ownership of an R x Cc grid of 16 x 16 tiles over NW waves (R, Cc powers of two,
// R <= NW): wave w owns row tile w % WR and the NT column tiles from (w / WR) NT. Every
// product with the same grid gives a wave the same tiles, so their accumulators combine
// elementwise. cb = w / WR indexes the wave's column block in partial row sums.
template <int R, int Cc, int NW> struct Own {
  static_assert(R <= NW, "one row tile per wave at most");
  static constexpr int WR = R, WCc = NW / R;
  static constexpr int NT = Cc >= WCc ? Cc / WCc : 1;
  __device__ __forceinline__ static bool active(int w) { return (w / WR) * NT < Cc; }
  __device__ __forceinline__ static int m(int w) { return w % WR; }
  __device__ __forceinline__ static int n0(int w) { return (w / WR) * NT; }
  __device__ __forceinline__ static int cb(int w) { return w / WR; }
};

// Row-vector slots of the partial sums in k_bwd_grad (column sums have their own array).
enum { R_EBAR = 0, R_DB1, R_RQ, R_RHO, R_DB3, R_GROW, R_NSLOT };

constexpr int kWavesG = 8;
constexpr int kThreadsG = kWavesG * 64;

template <typename TI, int C, int D> struct GradCfg {
  static constexpr int E = (int)sizeof(TI);
  static constexpr int BV = E == 2 ? (D >= 32 ? 32 : D) : 16;  // value columns per block
  static constexpr int NBH = D / BV;                            // blocks per head
  static constexpr int RT = C / 16;
  static constexpr int NCB = kWavesG / RT;  // column blocks of the partial row sums
  // One block buffer (elements): S0^T and dS^T row blocks [BV][D], Delta^T and A^T row
  // blocks [BV][C], dO and V column blocks [C][BV].
  static constexpr int O_S0 = 0, O_DS = BV * D, O_DL = 2 * BV * D, O_AT = O_DL + BV * C, O_DO = O_AT + BV * C,
                       O_V = O_DO + C * BV, BUF = O_V + C * BV;
  static constexpr int NBUF = 3;  // block buffers: two blocks in flight
  static_assert(NBUF * BUF >= 2 * C * C, "the head-summed C x C matrices must fit the block buffers");
  static_assert(BUF >= 2 * C * D, "dq/dk staging must fit a block buffer");
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

__device__ __forceinline__ void lds_wave_fence_b() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Grid (nc_max, Hk). Gradients of the r value heads of one key head in one chunk.
//
// Phase 1 streams the value dimension in blocks of BV columns (direct loads, the next two
// blocks in flight while the current one is used; one workgroup barrier per block).
// A = T^T dDelta comes from the reverse sweep, which formed it anyway and already wrote
// dV = diag(beta) A. Per block:
//   rowsum(A o V), <S0, dS_C>,
//   XQ += dO S0^T,  XK += Delta dS_C^T,  Y += A S0^T,  P += dO Delta^T,  AD += A Delta^T,
// with dO unscaled (the scale is applied afterwards). Since (I + L) Delta is exactly the
// right factor of dT, dL = -stril(T^T dT T^T) reduces to -stril(A Delta^T) = -stril(AD),
// and the W-path gradient of K is -diag(beta b) Y with rho = -rowsum(Y o K).
// Per head, the rest is elementwise on the wave's tiles: PG = P o Gamma (scaled),
// G' = -stril(AD) o Gamma, Gb = diag(beta) G', and the gate sums
//   rowsum(P o M) = rowsum(PG o Q K^T),  colsum(P o M) = colsum(PG o Q K^T),
//   rowsum(dL o Gamma o K K^T) = rowsum(G' o K K^T),  colsum(beta_i dL o Gamma o K K^T) = colsum(Gb o K K^T),
// with Q K^T and K K^T formed once per key head. The products with K and Q are linear in
// PG and Gb and dq, dk sum over the value heads, so they run once per key head on the
// head sums: dq += (sum PG) K,  dk += (sum PG)^T Q + ((sum Gb) + (sum Gb)^T) K.
template <typename TI, int C, int D>
__global__ __launch_bounds__(kThreadsG) void k_bwd_grad(Prob p) {
  using OT = TI;
  using CF = GradCfg<TI, C, D>;
  constexpr int NW = kWavesG, BV = CF::BV, NBH = CF::NBH, RT = CF::RT, NCB = CF::NCB;
  constexpr int KSC = ks_of<OT, C>(), KSB = ks_of<OT, BV>(), KSD = ks_of<OT, D>();
  constexpr int CE = 16 / (int)sizeof(OT);
  using LD = Swz<OT, D>;
  using LC = Swz<OT, C>;
  using LB = Swz<OT, BV>;
  using OD = Own<RT, D / 16, NW>;    // C x D products
  using OC = Own<RT, C / 16, NW>;    // C x C products
  using OrdD = RowOrd<OT, D>;        // storage order of the saved S^T and dS^T rows
  using OrdC = RowOrd<OT, C>;        // storage order of the saved Delta^T and A^T rows
  constexpr int NTD = OD::NT, NTC = OC::NT, NTB = BV / 16;
  constexpr int RS = NCB * C;  // one partial-sum slot

  __shared__ __align__(16) OT sK[C * D];
  __shared__ __align__(16) OT sQ[C * D];
  __shared__ __align__(16) OT sB[CF::NBUF][CF::BUF];  // block buffers (job j uses sB[j % NBUF])
  __shared__ __align__(16) float sgb[3][2 * C];        // gate records (head hh uses sgb[hh % 3])
  __shared__ float red[2][R_NSLOT * RS];
  __shared__ float redc[2][RT * C];  // column sums of PG o QK^T + Gb o KK^T per row tile
  __shared__ float swv[2][NW];

  const int c = blockIdx.x, kh = blockIdx.y;
  const ChunkInfo ci = p.chunks[c];
  if (ci.seq < 0) return;
  const int n = ci.len;
  const int w = wave_id(), lane = lane_id(), g4 = (lane >> 4) * 4, r16 = lane & 15;

  const int h0 = kh * p.r;
  constexpr int NH = NW / 2;  // the two halves of the waves load different tensors of a block
  TileDma<BV, D, NW, OT> dmS;   // S0^T, dS^T row blocks (every wave)
  TileDma<BV, C, NH, OT> dmB;   // Delta^T (first half) or A^T (second half) row blocks
  TileDma<C, BV, NH, OT> dmV;   // dO (first half) or V (second half) column blocks
  TileDma<C, D, NW, OT> dmD;    // K, Q
  TileDma<1, 2 * C, NW, float> dmG;  // gate record
  const int wh = w % NH;
  dmS.init(w);
  dmB.init(wh);
  dmV.init(wh);
  dmD.init(w);
  dmG.init(w);
  // Job j = (head h0 + j / NBH, block j % NBH) goes into sB[j % NBUF]; the first block of a
  // head also brings the head's gate record. A job's loads are issued in four parts spread
  // over the step two jobs earlier, so that no wave stalls long on a full memory queue.
  auto issue_part = [&](int j, int part) {
    const int h = h0 + j / NBH, v0 = (j % NBH) * BV;
    const size_t ch = ch_idx(p, c, h);
    OT* b = sB[j % CF::NBUF];
    if (part == 0) {
      dmS.issue(b + CF::O_S0, (const OT*)p.sv_S + ch * D * D + (size_t)v0 * D, D, BV, w);
      if (j % NBH == 0) dmG.issue(sgb[(j / NBH) % 3], p.sv_gb + ch * 2 * C, 2 * C, 1, w);
    } else if (part == 1) {
      dmS.issue(b + CF::O_DS, (const OT*)p.ws_dS + ch * D * D + (size_t)v0 * D, D, BV, w);
    } else if (part == 2) {
      if (w < NH)
        dmB.issue(b + CF::O_DL, (const OT*)p.sv_Dt + ch * D * C + (size_t)v0 * C, C, BV, wh);
      else
        dmB.issue(b + CF::O_AT, (const OT*)p.ws_At + ch * D * C + (size_t)v0 * C, C, BV, wh);
    } else {
      if (w < NH)
        dmV.issue(b + CF::O_DO, (const OT*)p.dO + (int64_t)ci.t0 * p.dO_rs + h * D + v0, p.dO_rs, n, wh);
      else
        dmV.issue(b + CF::O_V, (const OT*)p.v + (int64_t)ci.t0 * p.v_rs + h * D + v0, p.v_rs, n, wh);
    }
  };
  auto issue_block = [&](int j) {
    for (int part = 0; part < 4; ++part) issue_part(j, part);
  };
  // This wave's load instructions of job j.
  auto job_loads = [&](int j) {
    return 2 * dmS.count(w) + dmB.count(wh) + dmV.count(wh) + (j % NBH == 0 ? dmG.count(w) : 0);
  };
  dmD.issue(sK, (const OT*)p.k + (int64_t)ci.t0 * p.k_rs + kh * D, p.k_rs, n, w);
  dmD.issue(sQ, (const OT*)p.q + (int64_t)ci.t0 * p.q_rs + kh * D, p.q_rs, n, w);
  issue_block(0);
  if (1 < p.r * NBH) issue_block(1);

  const bool aD = OD::active(w), aC = OC::active(w);
  const int mt = OD::m(w);  // the wave's row tile (the same in every grid)
  const int nD = OD::n0(w), nC = OC::n0(w), cbD = OD::cb(w), cbC = OC::cb(w);
  // rowsum(A o V) is the diagonal of A V^T: the wave holding the diagonal C x C tile of its
  // row tile accumulates that tile of A V^T (one MFMA per block) and reads the diagonal.
  const bool dgw = aC && nC <= mt && mt < nC + NTC;
  constexpr int FIN = NW - 1;  // the wave that finishes each head's per-row gate gradients

  f32x4 dqf[NTD], dkf[NTD];  // dq, dk of the key head, summed over its value heads in order
#pragma unroll
  for (int y = 0; y < NTD; ++y) dqf[y] = dkf[y] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 QKt[NTC], KKt[NTC], PGs[NTC], Gbs[NTC];  // Q K^T, K K^T, sum PG, sum Gb on the C x C tiles
#pragma unroll
  for (int y = 0; y < NTC; ++y) QKt[y] = KKt[y] = PGs[y] = Gbs[y] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int njobs = p.r * NBH;
  for (int hh = 0; hh < p.r; ++hh) {
    const int h = h0 + hh, par = hh & 1;
    const float* gam = sgb[hh % 3];  // log2 units
    const float* bet = gam + C;
    float* redh = red[par];
    float* redch = redc[par];
    for (int i = threadIdx.x; i < R_NSLOT * RS; i += kThreadsG) redh[i] = 0.f;
    for (int i = threadIdx.x; i < RT * C; i += kThreadsG) redch[i] = 0.f;

    // ---- phase 1: stream the value dimension
    f32x4 XQ[NTD], XK[NTD], Y[NTD], P[NTC], AD[NTC], AV[1][1] = {{f32x4{0.f, 0.f, 0.f, 0.f}}};
#pragma unroll
    for (int y = 0; y < NTD; ++y) XQ[y] = XK[y] = Y[y] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int y = 0; y < NTC; ++y) P[y] = AD[y] = f32x4{0.f, 0.f, 0.f, 0.f};
    float sdot = 0.f;
    for (int b = 0; b < NBH; ++b) {
      const int j = hh * NBH + b;
      const OT* cur = sB[j % CF::NBUF];
      dma_wait_keep(j + 1 < njobs ? job_loads(j + 1) : 0);  // job j's loads (and all before) are done
      lds_barrier();  // job j (and K, Q, gates with it) is in LDS; every wave is done with job j - 1
      const bool nxt2 = j + 2 < njobs;
      if (nxt2) issue_part(j + 2, 0);
      if (j == 0 && aC) {  // Q K^T and K K^T of the key head on this wave's C x C tiles
        f32x4 G2[2][NTC];
#pragma unroll
        for (int y = 0; y < NTC; ++y) G2[0][y] = G2[1][y] = f32x4{0.f, 0.f, 0.f, 0.f};
        wave_mm<OT, D, 2, NTC>(G2, [&](int m, int s) { return ld_n<OT, KSD, STD, LD>(m == 0 ? sQ : sK, 16 * mt, s); },
                               [&](int y, int s) { return ld_n<OT, KSD, STD, LD>(sK, 16 * (nC + y), s); });
#pragma unroll
        for (int y = 0; y < NTC; ++y) {
          QKt[y] = G2[0][y];
          KKt[y] = G2[1][y];
        }
      }
      const OT* sS0 = cur + CF::O_S0;
      const OT* sDS = cur + CF::O_DS;
      const OT* sDL = cur + CF::O_DL;
      const OT* sAt = cur + CF::O_AT;
      const OT* sDO = cur + CF::O_DO;
      const OT* sV = cur + CF::O_V;
      {
        using V = Vec16<OT>;
        for (int idx = threadIdx.x; idx < D * BV / V::N; idx += kThreadsG) {  // same layout: index-wise product
          const typename V::type a = reinterpret_cast<const typename V::type*>(sS0)[idx];
          const typename V::type d = reinterpret_cast<const typename V::type*>(sDS)[idx];
#pragma unroll
          for (int e = 0; e < V::N; ++e) sdot += (float)a[e] * (float)d[e];
        }
      }
      if (nxt2) issue_part(j + 2, 1);  // every wave issues every part (the wait counts rely on it)
      if (aD) {
        f32x4 XY[2][NTD];  // dO S0^T and A S0^T share the S0 fragments
#pragma unroll
        for (int y = 0; y < NTD; ++y) {
          XY[0][y] = XQ[y];
          XY[1][y] = Y[y];
        }
        wave_mm<OT, BV, 2, NTD>(XY,
                                [&](int m, int s) {
                                  return m == 0 ? ld_n<OT, KSB, STD, LB>(sDO, 16 * mt, s)
                                                : ld_t<OT, KSB, STD, LC, OrdC>(sAt, 16 * mt, s);
                                },
                                [&](int y, int s) { return ld_t<OT, KSB, STD, LD, OrdD>(sS0, 16 * (nD + y), s); });
        f32x4 XKa[1][NTD];
#pragma unroll
        for (int y = 0; y < NTD; ++y) XKa[0][y] = XK[y];
        wave_mm<OT, BV, 1, NTD>(XKa, [&](int, int s) { return ld_t<OT, KSB, STD, LC, OrdC>(sDL, 16 * mt, s); },
                                [&](int y, int s) { return ld_t<OT, KSB, STD, LD, OrdD>(sDS, 16 * (nD + y), s); });
#pragma unroll
        for (int y = 0; y < NTD; ++y) {
          XQ[y] = XY[0][y];
          Y[y] = XY[1][y];
          XK[y] = XKa[0][y];
        }
      }
      if (nxt2) issue_part(j + 2, 2);
      if (aC) {
        f32x4 PA[2][NTC];  // dO Delta^T and A Delta^T share the Delta fragments
#pragma unroll
        for (int y = 0; y < NTC; ++y) {
          PA[0][y] = P[y];
          PA[1][y] = AD[y];
        }
        wave_mm<OT, BV, 2, NTC>(PA,
                                [&](int m, int s) {
                                  return m == 0 ? ld_n<OT, KSB, STD, LB>(sDO, 16 * mt, s)
                                                : ld_t<OT, KSB, STD, LC, OrdC>(sAt, 16 * mt, s);
                                },
                                [&](int y, int s) { return ld_t<OT, KSB, STD, LC, OrdC>(sDL, 16 * (nC + y), s); });
#pragma unroll
        for (int y = 0; y < NTC; ++y) {
          P[y] = PA[0][y];
          AD[y] = PA[1][y];
        }
      }
      if (nxt2) issue_part(j + 2, 3);
      if (dgw)  // A V^T on the diagonal tile of row tile mt
        wave_mm<OT, BV, 1, 1>(AV, [&](int, int s) { return ld_t<OT, KSB, STD, LC, OrdC>(sAt, 16 * mt, s); },
                              [&](int, int s) { return ld_n<OT, KSB, STD, LB>(sV, 16 * mt, s); });
    }

    // ---- phase 2 of the head: elementwise on the wave's tiles
    const float sc = p.scale, gn = gam[C - 1];
    float bx[4], ex[4], bb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * mt + g4 + e;
      bx[e] = __builtin_amdgcn_exp2f(gam[i]);
      ex[e] = __builtin_amdgcn_exp2f(gn - gam[i]);
      bb[e] = bet[i];
    }
    if (dgw) {  // lane (g, r) holds (A V^T)[4 g + e][r]: the diagonal is e = r - 4 g
      const int e = r16 - g4;
      if (e >= 0 && e < 4) redh[R_DB1 * RS + 16 * mt + r16] = AV[0][0][e];
    }
    if (aC) {
      float grow[4] = {0.f, 0.f, 0.f, 0.f}, db3[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int y = 0; y < NTC; ++y) {
        float col = 0.f;
        const int jj = 16 * (nC + y) + r16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * mt + g4 + e;
          const float gd = __builtin_amdgcn_exp2f(gam[i] - gam[jj]);
          const float pg = i >= jj ? sc * P[y][e] * gd : 0.f;
          const float gp = i > jj ? -AD[y][e] * gd : 0.f;
          const float gb = bb[e] * gp;
          PGs[y][e] += pg;
          Gbs[y][e] += gb;
          grow[e] += pg * QKt[y][e];
          db3[e] += gp * KKt[y][e];
          col += pg * QKt[y][e] + gb * KKt[y][e];
        }
        col += __shfl_xor(col, 16);
        col += __shfl_xor(col, 32);
        if (lane < 16) redch[mt * C + jj] = col;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        grow[e] = row16_sum(grow[e]);
        db3[e] = row16_sum(db3[e]);
      }
      if (r16 == 0)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          redh[R_GROW * RS + cbC * C + 16 * mt + g4 + e] = grow[e];
          redh[R_DB3 * RS + cbC * C + 16 * mt + g4 + e] = db3[e];
        }
    }
    if (aD) {
      f32x4 Kc[NTD], Qc[NTD];  // K and Q at this wave's accumulator positions
#pragma unroll
      for (int y = 0; y < NTD; ++y) {
        Kc[y] = ld_col4<OT, LD>(sK, 16 * mt + g4, 16 * (nD + y));
        Qc[y] = ld_col4<OT, LD>(sQ, 16 * mt + g4, 16 * (nD + y));
      }
      acc_rowsum<NTD>(XK, mt, [&](int y, int e, float x) { return ex[e] * x * Kc[y][e]; }, redh + R_EBAR * RS + cbD * C);
      acc_rowsum<NTD>(XQ, mt, [&](int y, int e, float x) { return sc * x * Qc[y][e]; }, redh + R_RQ * RS + cbD * C);
      acc_rowsum<NTD>(Y, mt, [&](int y, int e, float x) { return -x * Kc[y][e]; }, redh + R_RHO * RS + cbD * C);
#pragma unroll
      for (int y = 0; y < NTD; ++y)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dkf[y][e] += ex[e] * XK[y][e] - bb[e] * bx[e] * Y[y][e];
          dqf[y][e] += sc * bx[e] * XQ[y][e];
        }
    }
    sdot = wave_sum(sdot);
    if (lane == 0) swv[par][w] = sdot;
    lds_barrier();  // the head's partial sums are complete
    if (w == FIN) {  // per-row gate gradients of head h (the other waves move on)
      const int i = lane;
      const bool ok = i < C;
      float rv[R_NSLOT], gcol = 0.f;
#pragma unroll
      for (int sl = 0; sl < R_NSLOT; ++sl) {
        float a = 0.f;
        if (ok)
          for (int b = 0; b < NCB; ++b) a += redh[sl * RS + b * C + i];
        rv[sl] = a;
      }
      if (ok)
        for (int m = 0; m < RT; ++m) gcol += redch[m * C + i];
      const float bi = ok ? __builtin_amdgcn_exp2f(gam[i]) : 0.f, be = ok ? bet[i] : 0.f;
      float dgam = 0.f;
      if (ok) dgam = bi * rv[R_RQ] + be * bi * rv[R_RHO] - rv[R_EBAR] + rv[R_GROW] + be * rv[R_DB3] - gcol;
      const float ebsum = wave_sum(rv[R_EBAR]);
      if (i == n - 1) {
        float st = 0.f;
        for (int k = 0; k < NW; ++k) st += swv[par][k];
        dgam += __builtin_amdgcn_exp2f(gn) * st + ebsum;
      }
      const float dlg = wave_rscan_incl(dgam);
      if (i < n) {
        const int64_t row = (int64_t)(ci.t0 + i) * p.Hv + h;
        p.dbeta[row] = rv[R_DB1] + bi * rv[R_RHO] + rv[R_DB3];
        // dg = dlog g / g, with 1 / g_i = 2^(gamma_{i-1} - gamma_i) from the record
        p.dg[row] = dlg * __builtin_amdgcn_exp2f((i > 0 ? gam[i - 1] : 0.f) - gam[i]);
      }
    }
  }

  // ---- the key head's products with K and Q on the head sums
  OT* const sPGs = sB[0];         // sum PG    [C][C]
  OT* const sGbs = sB[0] + C * C;  // sum Gb   [C][C]
  if (aC) {
#pragma unroll
    for (int y = 0; y < NTC; ++y)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * mt + g4 + e, jj = 16 * (nC + y) + r16;
        sPGs[LC::at(i, jj)] = (OT)PGs[y][e];
        sGbs[LC::at(i, jj)] = (OT)Gbs[y][e];
      }
  }
  lds_barrier();
  if (aD) {
    auto fK = [&](int y, int s) { return ld_t<OT, KSC, STD, LD>(sK, 16 * (nD + y), s); };
    {  // dq += (sum PG) K
      f32x4 Z[1][NTD];
      zero(Z);
      wave_mm<OT, C, 1, NTD>(Z, [&](int, int s) { return ld_n<OT, KSC, STD, LC>(sPGs, 16 * mt, s); }, fK);
#pragma unroll
      for (int y = 0; y < NTD; ++y) dqf[y] += Z[0][y];
    }
    {  // dk += (sum PG)^T Q + (sum Gb)^T K + (sum Gb) K
      f32x4 Z[1][NTD];
      zero(Z);
      wave_mm<OT, C, 1, NTD>(Z, [&](int, int s) { return ld_t<OT, KSC, STD, LC>(sPGs, 16 * mt, s); },
                             [&](int y, int s) { return ld_t<OT, KSC, STD, LD>(sQ, 16 * (nD + y), s); });
      wave_mm<OT, C, 1, NTD>(Z, [&](int, int s) { return ld_t<OT, KSC, STD, LC>(sGbs, 16 * mt, s); }, fK);
      wave_mm<OT, C, 1, NTD>(Z, [&](int, int s) { return ld_n<OT, KSC, STD, LC>(sGbs, 16 * mt, s); }, fK);
#pragma unroll
      for (int y = 0; y < NTD; ++y) dkf[y] += Z[0][y];
    }
  }
  lds_barrier();
  // dq, dk of the key head: rows through LDS (the first block buffer), 16-byte stores
  {
    TI* st = (TI*)sB[0];
    if (aD) {
#pragma unroll
      for (int y = 0; y < NTD; ++y)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * mt + g4 + e, d = 16 * (nD + y) + r16;
          st[i * D + d] = (TI)dqf[y][e];
          st[(C + i) * D + d] = (TI)dkf[y][e];
        }
    }
    lds_barrier();
    using V = Vec16<TI>;
    constexpr int VPR = D / V::N;
    TI* dq = (TI*)p.dq + (int64_t)ci.t0 * p.dq_rs + kh * D;
    TI* dk = (TI*)p.dk + (int64_t)ci.t0 * p.dk_rs + kh * D;
    for (int idx = threadIdx.x; idx < 2 * C * VPR; idx += kThreadsG) {
      const int r = idx / VPR, cc = (idx % VPR) * V::N;
      const int i = r % C;
      if (i < n) {
        TI* dst = r < C ? dq + (int64_t)i * p.dq_rs + cc : dk + (int64_t)i * p.dk_rs + cc;
        *reinterpret_cast<typename V::type*>(dst) = *reinterpret_cast<const typename V::type*>(st + r * D + cc);
      }
    }
  }
}

template <typename TI, int C, int D>
static hipError_t bwd_seq(const Prob& p, hipStream_t s) {
  using CF = BwCfg<TI, C, D>;
  traced("k_table", s, [&] { k_table<C><<<1, NTHREADS, 0, s>>>(p); });
  if (p.N > 0)
    traced("k_bwd_sweep", s,
           [&] { k_bwd_sweep<TI, C, D><<<xcd_grid(p.N * p.Hk, p.r), CF::NW * 64, 0, s>>>(p); });
  if (p.nc_max > 0)
    traced("k_bwd_grad", s, [&] { k_bwd_grad<TI, C, D><<<dim3(p.nc_max, p.Hk), kThreadsG, 0, s>>>(p); });
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
