// gdn_bwd.hip -- chunked reverse-mode backward of the gated delta rule on gfx950.
//
// Per-token form: lattice-inference gdn_backward.rs, gdn_backward steps 4a-4d (output,
// state update, delta, retrieval), with the state adjoint dS carried in reverse time.
// Chunk form (derived here; the pages give none), with dO~ = scale dO, e = exp(gamma_n -
// gamma) and dS_C the adjoint flowing into the end of a chunk:
//   dDelta = M^T dO~ + diag(e) K dS_C                     (M = Gamma o Q K^T, lower incl.)
//   dS_0   = b_n dS_C + (diag(b) Q)^T dO~ - W^T dDelta    (carried to the previous chunk)
//   XQ = dO~ S0^T,  XW = dDelta S0^T,  XK = Delta dS_C^T,  P = tril(dO~ Delta^T)
//   dQ     = diag(b) XQ + (P o Gamma) K
//   dV     = diag(beta) T^T dDelta;  dK_beta_b = -T^T XW = -(T^T dDelta) S0^T
//   dT     = dDelta (diag(beta) V)^T - XW (diag(beta b) K)^T;  dL = strictly_lower(-T^T dT T^T)
//   dK     = (P o Gamma)^T Q + diag(e) XK + diag(beta b) dK_beta_b + G K + G^T K,
//            G = dL o (beta_i Gamma_ij)
//   dbeta  = rowsum(dV / beta o V) + b o rho + rowsum(dL o Gamma o K K^T),
//            rho = rowsum(dK_beta_b o K) = -colsum(T o (XW K^T))
//   dgamma = b o rowsum(Q o XQ) + beta b rho - ebar + rowsum(Gbar o Gamma) - colsum(Gbar o Gamma),
//            ebar = e o rowsum(K o XK), Gbar o Gamma = P o M + dL o beta_i K K^T o Gamma,
//            and the last valid row also gets b_n <S0, dS_C> + sum(ebar)
//   dlog g = reverse cumulative sum of dgamma within the chunk;  dg = dlog g / g.
//
// Kernels after the chunk table:
//  k_bwd_sweep (sequence x value head, 16 waves): the reverse chunk-serial pass; the
//      adjoint lives in float32 MFMA accumulators; saves dS_C, dDelta and dDelta^T.
//  k_bwd_grad  (chunk x key head, 16 waves): all remaining gradients for the r value
//      heads of the key head, one head after the other. Every operand arrives in the
//      layout its product reads (no transposes while staging). dq and dk of the key
//      head are summed over its value heads in ascending order in registers and stored
//      once: no atomics, every run is bit-identical. Row sums go through partial arrays
//      indexed by tile column block and are added in a fixed order.
#include "gdn_common.h"
#include "gdn_mma.h"

namespace gdn {

constexpr int kWavesB = 16;
constexpr int kWavesG = 8;  // k_bwd_grad
constexpr int kThreadsG = kWavesG * 64;
constexpr int kThreadsB = kWavesB * 64;

__host__ __device__ constexpr int bblk2(int x) { return x >= 32 ? 2 : 1; }

// Row sums of f(i, j, x) over an accumulator tile, added into red[column block][M].
// Each (row block, column block) belongs to one wave, so no two waves touch the same
// entry; the caller adds the column-block partials in order after a barrier.
template <int M, int N, int TM, int TN, int NWV, class F>
__device__ __forceinline__ void acc_rowsum(Tile<M, N, TM, TN, NWV>& t, F&& f, float* red) {
  using B = Blk<M, N, TM, TN, NWV>;
  const int w = threadIdx.x / 64, l = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < B::PER; ++q) {
    const int b = w + q * NWV;
    if (b < B::NB) {
      const int cb = b % B::BN, bi = (b / B::BN) * 16 * TM, bj = cb * 16 * TN;
#pragma unroll
      for (int x = 0; x < TM; ++x) {
        const int i0 = bi + x * 16 + (l >> 4) * 4;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int y = 0; y < TN; ++y) {
          const int j = bj + y * 16 + (l & 15);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += f(i0 + e, j, t.a[q][x][y][e]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = row16_sum(v[e]);
        if ((l & 15) == 0)
#pragma unroll
          for (int e = 0; e < 4; ++e) red[cb * M + i0 + e] += v[e];
      }
    }
  }
}

// Column sums, added into red[row block][N].
template <int M, int N, int TM, int TN, int NWV, class F>
__device__ __forceinline__ void acc_colsum(Tile<M, N, TM, TN, NWV>& t, F&& f, float* red) {
  using B = Blk<M, N, TM, TN, NWV>;
  const int w = threadIdx.x / 64, l = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < B::PER; ++q) {
    const int b = w + q * NWV;
    if (b < B::NB) {
      const int rb = b / B::BN, bi = rb * 16 * TM, bj = (b % B::BN) * 16 * TN;
#pragma unroll
      for (int y = 0; y < TN; ++y) {
        const int j = bj + y * 16 + (l & 15);
        float v = 0.f;
#pragma unroll
        for (int x = 0; x < TM; ++x)
#pragma unroll
          for (int e = 0; e < 4; ++e) v += f(bi + x * 16 + (l >> 4) * 4 + e, j, t.a[q][x][y][e]);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (l < 16) red[rb * N + j] += v;
      }
    }
  }
}

// ---------------------------------------------------------------------------- sweep
// Grid (N, Hv). Reverse chunk-serial pass over one sequence and one value head.
template <typename TI, int C, int D>
__global__ __launch_bounds__(kThreadsB) void k_bwd_sweep(Prob p) {
  using OT = TI;
  constexpr int NT = kThreadsB, NWV = kWavesB, LDO = D + 8, LCO = C + 8;
  constexpr int SM = bblk2(D), DN = bblk2(D);
  __shared__ __align__(16) OT sMt[C * LCO];   // M^T
  __shared__ __align__(16) OT sOt[D * LCO];   // dO~^T
  __shared__ __align__(16) OT sK[C * LDO];    // K
  __shared__ __align__(16) OT sQbt[D * LCO];  // (diag(b) Q)^T
  __shared__ __align__(16) OT sWt[D * LCO];   // -W^T
  __shared__ __align__(16) OT sdSt[D * LDO];  // dS^T: [v][d]
  __shared__ __align__(16) OT sdDt[D * LCO];  // dDelta^T: [v][i]
  __shared__ float sg[C], se[C];
  typedef OT o4 __attribute__((ext_vector_type(4)));

  const int n = blockIdx.x, h = blockIdx.y, kh = h / p.r;
  const size_t nh = (size_t)n * p.Hv + h;
  const int c0 = p.seq_chunk[n], c1 = p.seq_chunk[n + 1];
  using TS = Tile<D, D, SM, SM, NWV>;
  using TD = Tile<C, D, 1, DN, NWV>;
  TS dS;
  if (p.dST) {
    const float* s = p.dST + nh * D * D;
    dS.each([&](int d, int v, float& x) { x = s[d * D + v]; });
  } else {
    dS.zero();
  }

  Stage<C, C, NT, OT> nM;
  Stage<C, D, NT, TI> nO, nK;
  Stage<D, C, NT, OT> nQb;
  Stage<C, D, NT, OT> nW;
  float ng = 0.f;
  auto issue = [&](int c) {
    const ChunkInfo ci = p.chunks[c];
    const size_t ch = ch_idx(p, c, h);
    nM.issue((const OT*)p.sv_M + ch * C * C, C, C);
    nO.issue((const TI*)p.dO + (int64_t)ci.t0 * p.dO_rs + h * D, p.dO_rs, ci.len);
    nK.issue((const TI*)p.k + (int64_t)ci.t0 * p.k_rs + kh * D, p.k_rs, ci.len);
    nQb.issue((const OT*)p.sv_Qbt + ch * D * C, C, D);
    nW.issue((const OT*)p.sv_W + ch * C * D, D, C);
    if (threadIdx.x < C) ng = p.sv_gam[ch * C + threadIdx.x];
  };
  auto commit = [&]() {
    nM.template to_cols<LCO>(sMt);
    nO.template to_cols<LCO>(sOt, nullptr, p.scale);
    nK.template to_rows_raw<LDO>(sK);
    nQb.template to_rows_raw<LCO>(sQbt);
    nW.template to_cols<LCO>(sWt, nullptr, -1.f);
    if (threadIdx.x < C) sg[threadIdx.x] = ng;
  };
  auto adj_to_lds = [&]() {
    dS.each4([&](int d0, int v, f32x4& x) {
      *reinterpret_cast<o4*>(sdSt + v * LDO + d0) = o4{(OT)x[0], (OT)x[1], (OT)x[2], (OT)x[3]};
    });
  };

  if (c0 < c1) {
    issue(c1 - 1);
    commit();
  }
  adj_to_lds();
  lds_barrier();
  for (int c = c1 - 1; c >= c0; --c) {
    const size_t ch = ch_idx(p, c, h);
    lds_to_global_t<D, D, LDO, NT>((OT*)p.ws_dS + ch * D * D, sdSt);  // dS_C, key-major
    if (threadIdx.x < C) se[threadIdx.x] = expf(sg[C - 1] - sg[threadIdx.x]);
    const float bn = expf(sg[C - 1]);
    if (c - 1 >= c0) issue(c - 1);
    TD dD;
    dD.zero();
    gemm_nt<OT, C, D, D, 1, DN, NWV, LDO, LDO>(dD, sK, sdSt);  // K dS
    dS.each([&](int, int, float& x) { x *= bn; });
    gemm_nt<OT, D, D, C, SM, SM, NWV, LCO, LCO>(dS, sQbt, sOt);  // + (diag(b) Q)^T dO~
    lds_barrier();  // se visible
    dD.each([&](int i, int, float& x) { x *= se[i]; });
    gemm_nt<OT, C, D, C, 1, DN, NWV, LCO, LCO>(dD, sMt, sOt);  // + M^T dO~
    dD.each4([&](int i0, int v, f32x4& x) {
      *reinterpret_cast<o4*>(sdDt + v * LCO + i0) = o4{(OT)x[0], (OT)x[1], (OT)x[2], (OT)x[3]};
    });
    lds_barrier();
    gemm_nt<OT, D, D, C, SM, SM, NWV, LCO, LCO>(dS, sWt, sdDt);  // - W^T dDelta
    lds_to_global<D, C, LCO, NT>((OT*)p.ws_dDt + ch * D * C, sdDt);
    lds_barrier();
    adj_to_lds();
    if (c - 1 >= c0) commit();
    lds_barrier();
  }
  if (p.dS0) {
    float* s = p.dS0 + nh * D * D;
    dS.each([&](int d, int v, float& x) { s[d * D + v] = x; });
  }
}

// ---------------------------------------------------------------------------- grad
// Row-vector slots of the partial sums in k_bwd_grad.
enum { R_EBAR = 0, R_DB1, R_RQ, R_RHO, R_DB3, R_GROW, R_GCOL, R_NSLOT };
constexpr int kRedBlocks = 4;  // column blocks per partial-sum slot

template <typename TI, int C, int D> struct GradCfg {
  static constexpr int E = (int)sizeof(TI);
  static constexpr int BV = E == 2 ? (D >= 32 ? 32 : D) : 16;  // value columns per block
  static constexpr int NBH = D / BV;                            // blocks per head
  static constexpr bool DBUF = NBH % 2 == 0;  // blocks alternate between two buffers
  // One block buffer (element offsets): S0 and dS_C column blocks [D][BV] (key-major),
  // Delta, dO, V and A = T^T dDelta column blocks [C][BV], dDelta^T row block [BV][C].
  static constexpr int O_S0 = 0, O_DS = D * BV, O_DL = 2 * D * BV, O_DO = O_DL + C * BV, O_V = O_DO + C * BV,
                       O_A = O_V + C * BV, O_DDT = O_A + C * BV, BUF = O_DDT + BV * C;
  // Scratch of the second phase (padded rows of LC = C + 8): P o Gamma, its transpose,
  // G' = dL o Gamma, and G^T = (diag(beta) G')^T.
  static constexpr int LC = C + 8, SCR = 4 * C * LC;
  // With two buffers the scratch shares the second one (free once the head's last block,
  // which always sits there, is consumed); otherwise it has its own array.
  static constexpr int BUFY = DBUF ? (BUF > SCR ? BUF : SCR) : 16;
  static constexpr int SCRZ = DBUF ? 16 : SCR;
  static_assert(BUF >= 2 * C * D, "dq/dk staging must fit the first buffer");
};

// Grid (nc_max, Hk). Gradients of the r value heads of one key head in one chunk, one head
// after the other; dq and dk of the key head stay in registers across its value heads.
//
// Phase 1 streams the value dimension in blocks of BV columns (global -> LDS by direct
// loads, the next block in flight while the current one is used) and accumulates
//   A = T^T dDelta (per block, to LDS), dV = diag(beta) A, rowsum(A o V), <S0, dS_C>,
//   XQ += dO S0^T,  XK += Delta dS_C^T,  Y += A S0^T,  P += dO Delta^T,  AD += A Delta^T,
// with dO unscaled (the scale is applied afterwards). Since (I + L) Delta is exactly the
// right factor of dT, dL = -stril(T^T dT T^T) reduces to -stril(A Delta^T) = -stril(AD),
// and the W-path gradient of K is -diag(beta b) Y with rho = -rowsum(Y o K).
// Phase 2 forms Zq = (P o Gamma) K, Zk = (P o Gamma)^T Q, Z1 = G' K and Z2 = G^T K on MFMA
// and folds them into dq and dk. The row and column sums of Gbar o Gamma that the gate
// gradient needs are row sums against Q and K of these same products:
//   rowsum(P o M) = rowsum(Q o Zq),   colsum(P o M) = rowsum(K o Zk),
//   rowsum(dL o Gamma o K K^T) = rowsum(K o Z1),   colsum(beta_i dL o Gamma o K K^T) = rowsum(K o Z2),
// so neither K K^T nor M is needed here.
template <typename TI, int C, int D>
__global__ __launch_bounds__(kThreadsG) void k_bwd_grad(Prob p) {
  using OT = TI;
  using CF = GradCfg<TI, C, D>;
  constexpr int NT = kThreadsG, NWV = kWavesG, BV = CF::BV, NBH = CF::NBH;
  constexpr int DN = bblk2(D), RS = kRedBlocks * C;
  using LC = Swz<OT, C>;        // rows of C: K^T, Q^T, T^T, dDelta^T
  using LB = Swz<OT, BV>;       // rows of BV: the column blocks
  using LP = Pad<CF::LC>;       // scratch
  using TCC = Tile<C, C, 1, 1, NWV>;
  using TCD = Tile<C, D, 1, DN, NWV>;
  using TCB = Tile<C, BV, 1, 1, NWV>;
  static_assert(TCD::B::BN <= kRedBlocks && TCB::B::BN <= kRedBlocks, "partial-sum slots too small");

  __shared__ __align__(16) OT sKt[D * C];
  __shared__ __align__(16) OT sQt[D * C];
  __shared__ __align__(16) OT sTt[C * C];
  __shared__ __align__(16) OT sX[CF::BUF];
  __shared__ __align__(16) OT sY[CF::BUFY];
  __shared__ __align__(16) OT sZ[CF::SCRZ];
  __shared__ float red[R_NSLOT * RS];
  __shared__ float rowv[R_NSLOT * C];
  __shared__ float sg[C], sb[C], se[C], sbeta[C], sgate[C], swv[NWV];

  const int c = blockIdx.x, kh = blockIdx.y;
  const ChunkInfo ci = p.chunks[c];
  if (ci.seq < 0) return;
  const int n = ci.len;
  const int w = threadIdx.x / 64, lane = threadIdx.x & 63;
  const size_t ck = (size_t)c * p.Hk + kh;
  OT* const scr = CF::DBUF ? sY : sZ;
  OT* const sPG = scr;
  OT* const sPGt = scr + C * CF::LC;
  OT* const sGp = scr + 2 * C * CF::LC;
  OT* const sGt = scr + 3 * C * CF::LC;

  auto issue_block = [&](OT* buf, int h, int blk) {
    const size_t ch = ch_idx(p, c, h);
    const int v0 = blk * BV;
    dma_tile<D, BV, NT>(buf + CF::O_S0, (const OT*)p.sv_S + ch * D * D + v0, D, D);
    dma_tile<D, BV, NT>(buf + CF::O_DS, (const OT*)p.ws_dS + ch * D * D + v0, D, D);
    dma_tile<C, BV, NT>(buf + CF::O_DL, (const OT*)p.sv_Dl + ch * C * D + v0, D, C);
    dma_tile<C, BV, NT>(buf + CF::O_DO, (const TI*)p.dO + (int64_t)ci.t0 * p.dO_rs + h * D + v0, p.dO_rs, n);
    dma_tile<C, BV, NT>(buf + CF::O_V, (const TI*)p.v + (int64_t)ci.t0 * p.v_rs + h * D + v0, p.v_rs, n);
    dma_tile<BV, C, NT>(buf + CF::O_DDT, (const OT*)p.ws_dDt + ch * D * C + (size_t)v0 * C, C, BV);
  };
  float ngam = 0.f, nbeta = 0.f, ngate = 1.f;
  auto issue_head = [&](int h) {  // T^T and the per-row gate values of value head h
    const size_t ch = ch_idx(p, c, h);
    dma_tile<C, C, NT>(sTt, (const OT*)p.sv_Tt + ch * C * C, C, C);
    if (threadIdx.x < C) {
      const int i = threadIdx.x;
      ngam = p.sv_gam[ch * C + i];
      nbeta = i < n ? p.beta[(int64_t)(ci.t0 + i) * p.Hv + h] : 0.f;
      ngate = i < n ? p.g[(int64_t)(ci.t0 + i) * p.Hv + h] : 1.f;
    }
  };
  const int h0 = kh * p.r;
  dma_tile<D, C, NT>(sKt, (const OT*)p.sv_Kt + ck * D * C, C, D);
  dma_tile<D, C, NT>(sQt, (const OT*)p.sv_Qt + ck * D * C, C, D);
  issue_head(h0);
  issue_block(sX, h0, 0);

  TCD dqf, dkf;  // dq, dk of the key head, summed over its value heads in order
  dqf.zero();
  dkf.zero();

  for (int hh = 0; hh < p.r; ++hh) {
    const int h = h0 + hh;
    TI* dV = (TI*)p.dv + (int64_t)ci.t0 * p.dv_rs + h * D;
    if (threadIdx.x < C) {
      sg[threadIdx.x] = ngam;
      sbeta[threadIdx.x] = nbeta;
      sgate[threadIdx.x] = ngate;
    }
    for (int i = threadIdx.x; i < R_NSLOT * RS; i += NT) red[i] = 0.f;

    // ---- phase 1
    TCD XQ, XK, Y;
    TCC P, AD;
    XQ.zero();
    XK.zero();
    Y.zero();
    P.zero();
    AD.zero();
    float sdot = 0.f;
    auto block = [&](OT* cur, OT* nxt, int b) {
      dma_wait();
      lds_barrier();  // block b (and everything issued with it) is in LDS
      if (b == 0 && threadIdx.x < C) {
        sb[threadIdx.x] = expf(sg[threadIdx.x]);
        se[threadIdx.x] = expf(sg[C - 1] - sg[threadIdx.x]);
      }
      if (b + 1 < NBH) issue_block(nxt, h, b + 1);
      const int v0 = b * BV;
      {
        TCB A;
        A.zero();
        gemm_l<OT, C, BV, C, 1, 1, NWV, LC, LC>(A, sTt, cur + CF::O_DDT);
        A.each([&](int i, int j, float& x) {
          if (i < n) dV[(int64_t)i * p.dv_rs + v0 + j] = (TI)(sbeta[i] * x);
          cur[CF::O_A + LB::at(i, j)] = (OT)x;
        });
        acc_rowsum(A, [&](int i, int j, float x) { return x * (float)cur[CF::O_V + LB::at(i, j)]; },
                   red + R_DB1 * RS);
      }
      {
        using V = Vec16<OT>;
        for (int idx = threadIdx.x; idx < D * BV / V::N; idx += NT) {  // same layout: index-wise product
          const typename V::type a = reinterpret_cast<const typename V::type*>(cur + CF::O_S0)[idx];
          const typename V::type d = reinterpret_cast<const typename V::type*>(cur + CF::O_DS)[idx];
#pragma unroll
          for (int e = 0; e < V::N; ++e) sdot += (float)a[e] * (float)d[e];
        }
      }
      lds_barrier();  // A visible
      gemm_l<OT, C, D, BV, 1, DN, NWV, LB, LB>(XQ, cur + CF::O_DO, cur + CF::O_S0);
      gemm_l<OT, C, D, BV, 1, DN, NWV, LB, LB>(XK, cur + CF::O_DL, cur + CF::O_DS);
      gemm_l<OT, C, D, BV, 1, DN, NWV, LB, LB>(Y, cur + CF::O_A, cur + CF::O_S0);
      gemm_l<OT, C, C, BV, 1, 1, NWV, LB, LB>(P, cur + CF::O_DO, cur + CF::O_DL);
      gemm_l<OT, C, C, BV, 1, 1, NWV, LB, LB>(AD, cur + CF::O_A, cur + CF::O_DL);
    };
    if constexpr (CF::DBUF) {
      for (int b = 0; b < NBH; b += 2) {
        block(sX, sY, b);
        block(sY, sX, b + 1);
      }
    } else {
      block(sX, sX, 0);
    }
    lds_barrier();  // the last block and T^T are consumed
    const bool more = hh + 1 < p.r;
    if (more) {
      issue_head(h + 1);
      issue_block(sX, h + 1, 0);
    }

    // ---- phase 2
    const float sc = p.scale;
    P.each([&](int i, int j, float& x) {
      const float pg = i >= j ? sc * x * expf(sg[i] - sg[j]) : 0.f;
      sPG[LP::at(i, j)] = (OT)pg;
      sPGt[LP::at(j, i)] = (OT)pg;
    });
    AD.each([&](int i, int j, float& x) {  // dL = -stril(AD); G' = dL o Gamma
      const float gp = i > j ? -x * expf(sg[i] - sg[j]) : 0.f;
      sGp[LP::at(i, j)] = (OT)gp;
      sGt[LP::at(j, i)] = (OT)(sbeta[i] * gp);
    });
    acc_rowsum(XK, [&](int i, int d, float x) { return se[i] * x * (float)sKt[LC::at(d, i)]; }, red + R_EBAR * RS);
    dkf.each_with(XK, [&](int i, int, float& a, float& x) { a += se[i] * x; });
    acc_rowsum(XQ, [&](int i, int d, float x) { return sc * x * (float)sQt[LC::at(d, i)]; }, red + R_RQ * RS);
    dqf.each_with(XQ, [&](int i, int, float& a, float& x) { a += sc * sb[i] * x; });
    acc_rowsum(Y, [&](int i, int d, float x) { return -x * (float)sKt[LC::at(d, i)]; }, red + R_RHO * RS);
    dkf.each_with(Y, [&](int i, int, float& a, float& y) { a -= sbeta[i] * sb[i] * y; });
    sdot = wave_sum(sdot);
    if (lane == 0) swv[w] = sdot;
    lds_barrier();  // scratch written
    {
      TCD Z;
      Z.zero();
      gemm_l<OT, C, D, C, 1, DN, NWV, LP, LC>(Z, sPG, sKt);  // (P o Gamma) K
      acc_rowsum(Z, [&](int i, int d, float x) { return x * (float)sQt[LC::at(d, i)]; }, red + R_GROW * RS);
      dqf.each_with(Z, [&](int, int, float& a, float& z) { a += z; });
    }
    {
      TCD Z;
      Z.zero();
      gemm_l<OT, C, D, C, 1, DN, NWV, LP, LC>(Z, sPGt, sQt);  // (P o Gamma)^T Q
      gemm_l<OT, C, D, C, 1, DN, NWV, LP, LC>(Z, sGt, sKt);   // + G^T K
      acc_rowsum(Z, [&](int i, int d, float x) { return x * (float)sKt[LC::at(d, i)]; }, red + R_GCOL * RS);
      dkf.each_with(Z, [&](int, int, float& a, float& z) { a += z; });
    }
    {
      TCD Z;
      Z.zero();
      gemm_l<OT, C, D, C, 1, DN, NWV, LP, LC>(Z, sGp, sKt);  // G' K
      acc_rowsum(Z, [&](int i, int d, float x) { return x * (float)sKt[LC::at(d, i)]; }, red + R_DB3 * RS);
      dkf.each_with(Z, [&](int i, int, float& a, float& z) { a += sbeta[i] * z; });
    }
    lds_barrier();
    if (threadIdx.x < C) {
      const int i = threadIdx.x;
      for (int s = 0; s < R_NSLOT; ++s) {
        float a = 0.f;
        for (int b = 0; b < kRedBlocks; ++b) a += red[s * RS + b * C + i];
        rowv[s * C + i] = a;
      }
    }
    lds_barrier();
    if (threadIdx.x < 64) {
      const int i = threadIdx.x;
      const bool ok = i < C;
      const float ebar = ok ? rowv[R_EBAR * C + i] : 0.f;
      const float rho = ok ? rowv[R_RHO * C + i] : 0.f;
      const float db3 = ok ? rowv[R_DB3 * C + i] : 0.f;
      float dgam = 0.f;
      if (ok)
        dgam = sb[i] * rowv[R_RQ * C + i] + sbeta[i] * sb[i] * rho - ebar + rowv[R_GROW * C + i] +
               sbeta[i] * db3 - rowv[R_GCOL * C + i];
      const float ebsum = wave_sum(ebar);
      if (i == n - 1) {
        float st = 0.f;
        for (int k = 0; k < NWV; ++k) st += swv[k];
        dgam += expf(sg[C - 1]) * st + ebsum;
      }
      const float dlg = wave_rscan_incl(dgam);
      if (i < n) {
        const int64_t row = (int64_t)(ci.t0 + i) * p.Hv + h;
        p.dbeta[row] = rowv[R_DB1 * C + i] + sb[i] * rho + db3;
        p.dg[row] = dlg / sgate[i];
      }
    }
    lds_barrier();
  }
  // dq, dk of the key head: rows through LDS (the first block buffer), 16-byte stores
  {
    TI* st = (TI*)sX;
    dqf.each([&](int i, int d, float& x) { st[i * D + d] = (TI)x; });
    dkf.each([&](int i, int d, float& x) { st[(C + i) * D + d] = (TI)x; });
    lds_barrier();
    using V = Vec16<TI>;
    constexpr int VPR = D / V::N;
    TI* dq = (TI*)p.dq + (int64_t)ci.t0 * p.dq_rs + kh * D;
    TI* dk = (TI*)p.dk + (int64_t)ci.t0 * p.dk_rs + kh * D;
    for (int idx = threadIdx.x; idx < 2 * C * VPR; idx += NT) {
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
  traced("k_table", s, [&] { k_table<C><<<1, NTHREADS, 0, s>>>(p); });
  if (p.N > 0) traced("k_bwd_sweep", s, [&] { k_bwd_sweep<TI, C, D><<<dim3(p.N, p.Hv), kThreadsB, 0, s>>>(p); });
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
