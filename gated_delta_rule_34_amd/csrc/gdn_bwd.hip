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
      for (int x = 0; x < TM; ++x)
#pragma unroll
        for (int y = 0; y < TN; ++y) {
          const int i0 = bi + x * 16 + (l >> 4) * 4, j = bj + y * 16 + (l & 15);
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = f(i0 + e, j, t.a[q][x][y][e]);
#pragma unroll
          for (int m = 1; m < 16; m <<= 1)
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += __shfl_xor(v[e], m);
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
      for (int x = 0; x < TM; ++x)
#pragma unroll
        for (int y = 0; y < TN; ++y) {
          const int i0 = bi + x * 16 + (l >> 4) * 4, j = bj + y * 16 + (l & 15);
          float v = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) v += f(i0 + e, j, t.a[q][x][y][e]);
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
  __syncthreads();
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
    __syncthreads();  // se visible
    dD.each([&](int i, int, float& x) { x *= se[i]; });
    gemm_nt<OT, C, D, C, 1, DN, NWV, LCO, LCO>(dD, sMt, sOt);  // + M^T dO~
    dD.each4([&](int i0, int v, f32x4& x) {
      *reinterpret_cast<o4*>(sdDt + v * LCO + i0) = o4{(OT)x[0], (OT)x[1], (OT)x[2], (OT)x[3]};
    });
    __syncthreads();
    gemm_nt<OT, D, D, C, SM, SM, NWV, LCO, LCO>(dS, sWt, sdDt);  // - W^T dDelta
    lds_to_global<D, C, LCO, NT>((OT*)p.ws_dDt + ch * D * C, sdDt);
    lds_to_global_t<D, C, LCO, NT>((OT*)p.ws_dD + ch * C * D, sdDt);
    __syncthreads();
    adj_to_lds();
    if (c - 1 >= c0) commit();
    __syncthreads();
  }
  if (p.dS0) {
    float* s = p.dS0 + nh * D * D;
    dS.each([&](int d, int v, float& x) { s[d * D + v] = x; });
  }
}

// ---------------------------------------------------------------------------- grad
// Row-vector slots of the partial sums in k_bwd_grad.
enum { R_EBAR = 0, R_DB1, R_RQ, R_RHO, R_DB3, R_GROW, R_GCOL, R_NSLOT };
constexpr int kRedBlocks = 4;  // column (row) blocks per partial-sum slot

template <typename TI, int C, int D> struct GradCfg {
  static constexpr int LDO = D + 8, LCO = C + 8;
  static constexpr int BV = sizeof(TI) == 2 ? (D < 64 ? D : 64) : 16, LBO = BV + 8;
  // phase 1 (one block of BV value columns): S0 and dS_C (key-major), dO, Delta,
  // dDelta, V, -beta b o dVbeta (row-major), dDelta^T
  static constexpr int G1 = 2 * D * LBO + 5 * C * LBO + BV * LCO;
  // phase 2: XW rows, K^T, Q^T, dT (later G^T), Z^T (later G), P o Gamma, its transpose
  static constexpr int G2 = C * LDO + 2 * D * LCO + 4 * C * LCO;
  static constexpr int GR = G1 > G2 ? G1 : G2;
};

// Grid (nc_max, Hk). Gradients of the r value heads of one key head in one chunk.
// Phase 1 streams blocks of value columns and accumulates
//   XQ += dO S0^T    XW += dDelta S0^T    XK += Delta dS_C^T    dk += (-beta b o T^T dDelta) S0^T
//   P += dO Delta^T  dT1 += dDelta V^T    (the scale of dO~ is applied afterwards)
// plus dV = beta o T^T dDelta and the row sums of dVbeta o V and <S0, dS_C>. Phase 2
// finishes dq, dT, dL, the rest of dk and the gate gradients.
template <typename TI, int C, int D>
__global__ __launch_bounds__(kThreadsG) void k_bwd_grad(Prob p) {
  using OT = TI;
  using CF = GradCfg<TI, C, D>;
  constexpr int NT = kThreadsG, NWV = kWavesG, LDO = CF::LDO, LCO = CF::LCO;
  constexpr int BV = CF::BV, LBO = CF::LBO;
  constexpr int DN = bblk2(D);
  constexpr int RS = kRedBlocks * C;  // floats per partial-sum slot
  typedef OT o4 __attribute__((ext_vector_type(4)));

  using TCC = Tile<C, C, 1, 1, NWV>;
  using TCD = Tile<C, D, 1, DN, NWV>;
  using TCB = Tile<C, BV, 1, 1, NWV>;
  static_assert(TCD::B::BN <= kRedBlocks && TCC::B::BN <= kRedBlocks && TCC::B::BM <= kRedBlocks &&
                    TCB::B::BN <= kRedBlocks,
                "partial-sum slots too small");

  __shared__ __align__(16) OT sK[C * LDO];  // K rows
  __shared__ __align__(16) OT sT[C * LCO];  // T rows
  __shared__ __align__(16) OT sTt[C * LCO]; // T^T rows
  __shared__ __align__(16) OT sR[CF::GR];
  __shared__ float red[R_NSLOT * RS];
  __shared__ float rowv[R_NSLOT * C];
  __shared__ float sg[C], sb[C], se[C], sbeta[C], swv[NWV];

  const int c = blockIdx.x, kh = blockIdx.y;
  const ChunkInfo ci = p.chunks[c];
  if (ci.seq < 0) return;
  const int n = ci.len;
  const int w = threadIdx.x / 64, lane = threadIdx.x & 63;
  const size_t ck = (size_t)c * p.Hk + kh;

  // phase-1 buffers
  OT* sS0k = sR;              // [D][LBO]  S0 block, key-major
  OT* sdSk = sS0k + D * LBO;  // [D][LBO]  dS_C block, key-major
  OT* sO = sdSk + D * LBO;    // [C][LBO]  dO
  OT* sDl = sO + C * LBO;     // [C][LBO]  Delta
  OT* sdD = sDl + C * LBO;    // [C][LBO]  dDelta
  OT* sV = sdD + C * LBO;     // [C][LBO]  V
  OT* sdVb = sV + C * LBO;    // [C][LBO]  -beta b o dVbeta
  OT* sdDt = sdVb + C * LBO;  // [BV][LCO] dDelta^T
  // phase-2 buffers
  OT* sXW = sR;               // [C][LDO]
  OT* sKt = sXW + C * LDO;    // [D][LCO]
  OT* sQt = sKt + D * LCO;    // [D][LCO]
  OT* sdT = sQt + D * LCO;    // [C][LCO]  dT, then G^T
  OT* sZt = sdT + C * LCO;    // [C][LCO]  Z^T, then G
  OT* sPG = sZt + C * LCO;    // [C][LCO]
  OT* sPGt = sPG + C * LCO;   // [C][LCO]
  OT* sGt = sdT;
  OT* sG = sZt;

  {
    Stage<C, D, NT, TI> gk;
    gk.issue((const TI*)p.k + (int64_t)ci.t0 * p.k_rs + kh * D, p.k_rs, n);
    gk.template to_rows_raw<LDO>(sK);
  }
  TCD dqf, dkf;  // dq, dk of the key head, summed over its value heads in order
  dqf.zero();
  dkf.zero();
  __syncthreads();

  Stage<C, C, NT, OT> nT, nTt;
  float ngam = 0.f, nbeta = 0.f;
  auto issue_head = [&](int h) {
    const size_t ch = ch_idx(p, c, h);
    nT.issue((const OT*)p.sv_T + ch * C * C, C, C);
    nTt.issue((const OT*)p.sv_Tt + ch * C * C, C, C);
    if (threadIdx.x < C) {
      ngam = p.sv_gam[ch * C + threadIdx.x];
      nbeta = threadIdx.x < n ? p.beta[(int64_t)(ci.t0 + threadIdx.x) * p.Hv + h] : 0.f;
    }
  };
  issue_head(kh * p.r);

  for (int hh = 0; hh < p.r; ++hh) {
    const int h = kh * p.r + hh;
    const size_t ch = ch_idx(p, c, h);
    const OT* S0k = (const OT*)p.sv_S + ch * D * D;
    const OT* dSk = (const OT*)p.ws_dS + ch * D * D;
    const OT* Dl = (const OT*)p.sv_Dl + ch * C * D;
    const OT* dD = (const OT*)p.ws_dD + ch * C * D;
    const OT* dDt = (const OT*)p.ws_dDt + ch * D * C;
    const TI* dO = (const TI*)p.dO + (int64_t)ci.t0 * p.dO_rs + h * D;
    const TI* V = (const TI*)p.v + (int64_t)ci.t0 * p.v_rs + h * D;
    TI* dV = (TI*)p.dv + (int64_t)ci.t0 * p.dv_rs + h * D;

    // ---- set-up: T, T^T, gates, M (in the accumulator layout), zeroed partial sums
    nT.template to_rows_raw<LCO>(sT);
    nTt.template to_rows_raw<LCO>(sTt);
    if (threadIdx.x < C) {
      sg[threadIdx.x] = ngam;
      sbeta[threadIdx.x] = nbeta;
    }
    for (int i = threadIdx.x; i < R_NSLOT * RS; i += NT) red[i] = 0.f;
    Stage<D, BV, NT, OT> gs, gd;
    Stage<C, BV, NT, OT> gdl, gdd;
    Stage<BV, C, NT, OT> gdt;
    Stage<C, BV, NT, TI> go, gv;
    auto issue_blk = [&](int v0) {
      gs.issue(S0k + v0, D, D);
      gd.issue(dSk + v0, D, D);
      gdl.issue(Dl + v0, D, C);
      gdd.issue(dD + v0, D, C);
      gdt.issue(dDt + (size_t)v0 * C, C, BV);
      go.issue(dO + v0, p.dO_rs, n);
      gv.issue(V + v0, p.v_rs, n);
    };
    issue_blk(0);
    __syncthreads();
    if (threadIdx.x < C) {
      sb[threadIdx.x] = expf(sg[threadIdx.x]);
      se[threadIdx.x] = expf(sg[C - 1] - sg[threadIdx.x]);
    }

    // ---- phase 1
    TCD XQ, XW, XK;
    TCC PP, dT1;
    XQ.zero();
    XW.zero();
    XK.zero();
    PP.zero();
    dT1.zero();
    float sdot = 0.f;
    for (int v0 = 0; v0 < D; v0 += BV) {
      gs.template to_rows_raw<LBO>(sS0k);
      gd.template to_rows_raw<LBO>(sdSk);
      gdl.template to_rows_raw<LBO>(sDl);
      gdd.template to_rows_raw<LBO>(sdD);
      gdt.template to_rows_raw<LCO>(sdDt);
      go.template to_rows_raw<LBO>(sO);
      gv.template to_rows_raw<LBO>(sV);
      __syncthreads();
      if (v0 + BV < D) issue_blk(v0 + BV);
      {
        TCB dvb;
        dvb.zero();
        gemm_nt<OT, C, BV, C, 1, 1, NWV, LCO, LCO>(dvb, sTt, sdDt);  // T^T dDelta
        dvb.each([&](int i, int j, float& x) {
          if (i < n) dV[(int64_t)i * p.dv_rs + v0 + j] = (TI)(sbeta[i] * x);
          sdVb[i * LBO + j] = (OT)(-sbeta[i] * sb[i] * x);
        });
        acc_rowsum(dvb, [&](int i, int j, float x) { return x * (float)sV[i * LBO + j]; }, red + R_DB1 * RS);
      }
      for (int idx = threadIdx.x; idx < D * BV; idx += NT) {
        const int d = idx / BV, vv = idx % BV;
        sdot += (float)sS0k[d * LBO + vv] * (float)sdSk[d * LBO + vv];
      }
      __syncthreads();  // sdVb visible
      gemm_nt<OT, C, D, BV, 1, DN, NWV, LBO, LBO>(XQ, sO, sS0k);
      gemm_nt<OT, C, D, BV, 1, DN, NWV, LBO, LBO>(XW, sdD, sS0k);
      gemm_nt<OT, C, D, BV, 1, DN, NWV, LBO, LBO>(XK, sDl, sdSk);
      gemm_nt<OT, C, D, BV, 1, DN, NWV, LBO, LBO>(dkf, sdVb, sS0k);
      gemm_nt<OT, C, C, BV, 1, 1, NWV, LBO, LBO>(PP, sO, sDl);
      gemm_nt<OT, C, C, BV, 1, 1, NWV, LBO, LBO>(dT1, sdD, sV);
      __syncthreads();  // block buffers free
    }
    if (hh + 1 < p.r) issue_head(h + 1);

    // ---- phase 2
    {
      Stage<D, C, NT, OT> gkt, gqt;
      gkt.issue((const OT*)p.sv_Kt + ck * D * C, C, D);
      gqt.issue((const OT*)p.sv_Qt + ck * D * C, C, D);
      gkt.template to_rows_raw<LCO>(sKt);
      gqt.template to_rows_raw<LCO>(sQt);
    }
    const float sc = p.scale;
    XW.each([&](int i, int d, float& x) { sXW[i * LDO + d] = (OT)x; });
    PP.each([&](int i, int j, float& x) {
      x = i >= j ? x * sc : 0.f;
      const float pg = i >= j ? x * expf(sg[i] - sg[j]) : 0.f;
      sPG[i * LCO + j] = (OT)pg;
      sPGt[j * LCO + i] = (OT)pg;
    });
    acc_rowsum(XK, [&](int i, int d, float x) { return se[i] * x * (float)sK[i * LDO + d]; }, red + R_EBAR * RS);
    dkf.each_with(XK, [&](int i, int, float& a, float& x) { a += se[i] * x; });
    __syncthreads();
    acc_rowsum(XQ, [&](int i, int d, float x) { return sc * x * (float)sQt[d * LCO + i]; }, red + R_RQ * RS);
    dqf.each_with(XQ, [&](int i, int, float& a, float& x) { a += sc * sb[i] * x; });
    gemm_nt<OT, C, D, C, 1, DN, NWV, LCO, LCO>(dqf, sPG, sKt);  // (P o Gamma) K
    {
      TCC XWK;
      XWK.zero();
      gemm_nt<OT, C, C, D, 1, 1, NWV, LDO, LDO>(XWK, sXW, sK);  // XW K^T
      // rho_i = -sum_j T[j][i] XWK[j][i]: column sums of T o XWK
      acc_colsum(XWK, [&](int j, int i, float x) { return -(float)sT[j * LCO + i] * x; }, red + R_RHO * RS);
      XWK.each_with(dT1, [&](int, int j, float& xk, float& t1) { xk = sbeta[j] * (t1 - sb[j] * xk); });
      XWK.each([&](int i, int j, float& x) { sdT[i * LCO + j] = (OT)x; });
    }
    __syncthreads();
    {
      TCC Z;
      Z.zero();
      gemm_nt<OT, C, C, C, 1, 1, NWV, LCO, LCO>(Z, sdT, sT);  // dT T^T
      Z.each4([&](int i0, int m, f32x4& x) {
        *reinterpret_cast<o4*>(sZt + m * LCO + i0) = o4{(OT)x[0], (OT)x[1], (OT)x[2], (OT)x[3]};
      });
    }
    __syncthreads();
    TCC dL;
    dL.zero();
    gemm_nt<OT, C, C, C, 1, 1, NWV, LCO, LCO>(dL, sTt, sZt);  // T^T Z
    __syncthreads();  // sdT and sZt free: G and G^T take their place
    dL.each([&](int i, int j, float& x) {
      x = i > j ? -x : 0.f;
      const float gv = i > j ? x * sbeta[i] * expf(sg[i] - sg[j]) : 0.f;
      sG[i * LCO + j] = (OT)gv;
      sGt[j * LCO + i] = (OT)gv;
    });
    __syncthreads();
    gemm_nt<OT, C, D, C, 1, DN, NWV, LCO, LCO>(dkf, sPGt, sQt);  // (P o Gamma)^T Q
    gemm_nt<OT, C, D, C, 1, DN, NWV, LCO, LCO>(dkf, sG, sKt);    // G K
    gemm_nt<OT, C, D, C, 1, DN, NWV, LCO, LCO>(dkf, sGt, sKt);   // G^T K
    // Gbar o Gamma = P o M + dL o beta_i K K^T o Gamma, and dbeta's K K^T term
    {
      TCC gb = PP;
      {
        const OT* M = (const OT*)p.sv_M + ch * C * C;
        gb.each([&](int i, int j, float& x) { x *= (float)M[i * C + j]; });
      }
      TCC KK;
      KK.zero();
      gemm_nt<OT, C, C, D, 1, 1, NWV, LDO, LDO>(KK, sK, sK);
      dL.each_with(KK, [&](int i, int j, float& x, float& kk) { x = i > j ? x * expf(sg[i] - sg[j]) * kk : 0.f; });
      gb.each_with(dL, [&](int i, int, float& x, float& t) { x += sbeta[i] * t; });
      acc_rowsum(dL, [&](int, int, float x) { return x; }, red + R_DB3 * RS);
      acc_rowsum(gb, [&](int, int, float x) { return x; }, red + R_GROW * RS);
      acc_colsum(gb, [&](int, int, float x) { return x; }, red + R_GCOL * RS);
    }
    sdot = wave_sum(sdot);
    if (lane == 0) swv[w] = sdot;
    __syncthreads();
    if (threadIdx.x < C) {
      const int i = threadIdx.x;
      for (int s = 0; s < R_NSLOT; ++s) {
        float a = 0.f;
        for (int b = 0; b < kRedBlocks; ++b) a += red[s * RS + b * C + i];
        rowv[s * C + i] = a;
      }
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      const int i = threadIdx.x;
      const bool ok = i < C;
      const float ebar = ok ? rowv[R_EBAR * C + i] : 0.f;
      const float rho = ok ? rowv[R_RHO * C + i] : 0.f;
      float dgam = 0.f;
      if (ok)
        dgam = sb[i] * rowv[R_RQ * C + i] + sbeta[i] * sb[i] * rho - ebar + rowv[R_GROW * C + i] -
               rowv[R_GCOL * C + i];
      const float ebsum = wave_sum(ebar);
      if (i == n - 1) {
        float st = 0.f;
        for (int k = 0; k < NWV; ++k) st += swv[k];
        dgam += expf(sg[C - 1]) * st + ebsum;
      }
      const float dlg = wave_rscan_incl(dgam);
      if (i < n) {
        const int64_t row = (int64_t)(ci.t0 + i) * p.Hv + h;
        p.dbeta[row] = rowv[R_DB1 * C + i] + sb[i] * rho + rowv[R_DB3 * C + i];
        p.dg[row] = dlg / p.g[row];
      }
    }
    __syncthreads();
  }
  // dq, dk of the key head: stage rows through LDS, then 16-byte stores
  {
    TI* st = (TI*)sR;
    dqf.each([&](int i, int d, float& x) { st[i * LDO + d] = (TI)x; });
    dkf.each([&](int i, int d, float& x) { st[(C + i) * LDO + d] = (TI)x; });
    __syncthreads();
    using V = Vec16<TI>;
    constexpr int VPR = D / V::N;
    TI* dq = (TI*)p.dq + (int64_t)ci.t0 * p.dq_rs + kh * D;
    TI* dk = (TI*)p.dk + (int64_t)ci.t0 * p.dk_rs + kh * D;
    for (int idx = threadIdx.x; idx < 2 * C * VPR; idx += NT) {
      const int r = idx / VPR, cc = (idx % VPR) * V::N;
      const int i = r % C;
      if (i < n) {
        TI* dst = r < C ? dq + (int64_t)i * p.dq_rs + cc : dk + (int64_t)i * p.dk_rs + cc;
        *reinterpret_cast<typename V::type*>(dst) = *reinterpret_cast<const typename V::type*>(st + r * LDO + cc);
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
