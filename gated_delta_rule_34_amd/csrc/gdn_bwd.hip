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
//   dV     = diag(beta) T^T dDelta;  dK_beta_b = -T^T XW
//   dT     = dDelta (diag(beta) V)^T - XW (diag(beta b) K)^T;  dL = strictly_lower(-T^T dT T^T)
//   dK     = (P o Gamma)^T Q + diag(e) XK + diag(beta b) dK_beta_b + G K + G^T K,
//            G = dL o (beta_i Gamma_ij)
//   dbeta  = rowsum(dV / beta o V) + b o rho + rowsum(dL o Gamma o K K^T),
//            rho = rowsum(dK_beta_b o K)
//   dgamma = b o rowsum(Q o XQ) + beta b rho - ebar + rowsum(Gbar o Gamma) - colsum(Gbar o Gamma),
//            ebar = e o rowsum((K dS_C) o Delta), Gbar o Gamma = P o M + dL o beta_i K K^T o Gamma,
//            and the last valid row also gets b_n <S0, dS_C> + sum(ebar)
//   dlog g = reverse cumulative sum of dgamma within the chunk;  dg = dlog g / g.
//
// Kernels after the chunk table:
//  k_bwd_sweep (sequence x value head, 8 waves): the reverse chunk-serial pass; the
//      adjoint lives in float32 MFMA accumulators; saves dS_C and dDelta per chunk.
//  k_bwd_grad  (chunk x key head, 8 waves): all remaining gradients for the r value
//      heads of the key head, one head after the other. dq and dk of the key head are
//      summed over its value heads in ascending order in registers and stored once:
//      no atomics anywhere, every run is bit-identical. Row sums go through per-wave
//      partial arrays added in a fixed order.
#include "gdn_common.h"
#include "gdn_mma.h"

namespace gdn {

constexpr int kWavesB = 8;
constexpr int kThreadsB = kWavesB * 64;

__host__ __device__ constexpr int bblk2(int x) { return x >= 32 ? 2 : 1; }

template <int R, int Cn, int LD, int NT, typename OT>
__device__ __forceinline__ void lds_rows_to_global(OT* __restrict__ dst, const OT* src) {
  using V = Vec16<OT>;
  constexpr int VPR = Cn / V::N;
  for (int idx = threadIdx.x; idx < R * VPR; idx += NT) {
    const int r = idx / VPR, c = (idx % VPR) * V::N;
    *reinterpret_cast<typename V::type*>(dst + (size_t)r * Cn + c) =
        *reinterpret_cast<const typename V::type*>(src + r * LD + c);
  }
}

// Row sums of f(i, j, x) over the elements of an accumulator tile, added into the
// per-wave partial array red[wave][M] (no barrier; the caller sums the NWV partials
// in wave order after a barrier).
template <int M, int N, int TM, int TN, int NWV, class F>
__device__ __forceinline__ void acc_rowsum(Tile<M, N, TM, TN, NWV>& t, F&& f, float* red) {
  const int w = threadIdx.x / 64, l = threadIdx.x & 63;
  t.each4([&](int i0, int j, f32x4& x) {
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = f(i0 + e, j, x[e]);
#pragma unroll
    for (int m = 1; m < 16; m <<= 1)
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += __shfl_xor(v[e], m);
    if ((l & 15) == 0)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[w * M + i0 + e] += v[e];
  });
}

// Column sums, same conventions (red[wave][N]).
template <int M, int N, int TM, int TN, int NWV, class F>
__device__ __forceinline__ void acc_colsum(Tile<M, N, TM, TN, NWV>& t, F&& f, float* red) {
  const int w = threadIdx.x / 64, l = threadIdx.x & 63;
  t.each4([&](int i0, int j, f32x4& x) {
    float v = f(i0, j, x[0]) + f(i0 + 1, j, x[1]) + f(i0 + 2, j, x[2]) + f(i0 + 3, j, x[3]);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    if (l < 16) red[w * N + j] += v;
  });
}

// ---------------------------------------------------------------------------- sweep
// Grid (N, Hv). Reverse chunk-serial pass over one sequence and one value head.
template <typename TI, int C, int D>
__global__ __launch_bounds__(kThreadsB) void k_bwd_sweep(Prob p) {
  using OT = TI;
  constexpr int NT = kThreadsB, LDO = D + 8, LCO = C + 8;
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
  using TS = Tile<D, D, SM, SM, kWavesB>;
  using TD = Tile<C, D, 1, DN, kWavesB>;
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
    nK.template to_rows<LDO>(sK);
    nQb.template to_rows<LCO>(sQbt);
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
    lds_rows_to_global<D, D, LDO, NT>((OT*)p.ws_dS + ch * D * D, sdSt);  // dS_C, value-major
    if (threadIdx.x < C) se[threadIdx.x] = expf(sg[C - 1] - sg[threadIdx.x]);
    const float bn = expf(sg[C - 1]);
    if (c - 1 >= c0) issue(c - 1);
    TD dD;
    dD.zero();
    gemm_nt<OT, C, D, D, 1, DN, kWavesB, LDO, LDO>(dD, sK, sdSt);  // K dS
    dS.each([&](int, int, float& x) { x *= bn; });
    gemm_nt<OT, D, D, C, SM, SM, kWavesB, LCO, LCO>(dS, sQbt, sOt);  // + (diag(b) Q)^T dO~
    __syncthreads();  // se visible
    dD.each([&](int i, int, float& x) { x *= se[i]; });
    gemm_nt<OT, C, D, C, 1, DN, kWavesB, LCO, LCO>(dD, sMt, sOt);  // + M^T dO~
    dD.each4([&](int i0, int v, f32x4& x) {
      *reinterpret_cast<o4*>(sdDt + v * LCO + i0) = o4{(OT)x[0], (OT)x[1], (OT)x[2], (OT)x[3]};
    });
    __syncthreads();
    gemm_nt<OT, D, D, C, SM, SM, kWavesB, LCO, LCO>(dS, sWt, sdDt);  // - W^T dDelta
    lds_rows_to_global<D, C, LCO, NT>((OT*)p.ws_dDt + ch * D * C, sdDt);
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
// Row-vector slots of the per-wave partial sums in k_bwd_grad.
enum { R_EBAR = 0, R_DB1, R_RQ, R_RHO, R_DB3, R_GROW, R_GCOL, R_NSLOT };

template <typename TI, int C, int D> struct GradCfg {
  static constexpr int LDO = D + 8, LCO = C + 8, BV = D < 32 ? D : 32, LBO = BV + 8;
  // phase 1 (one value-column block): S0 and dS_C key-major, dS_C value-major,
  // dO, Delta, dDelta, V row blocks, dDelta^T
  static constexpr int G1 = 2 * D * LBO + BV * LDO + 4 * C * LBO + BV * LCO;
  // phase 2: XW^T (later Z^T), XW (later G), P o Gamma, its transpose, dT (later G^T)
  static constexpr int G2 = D * LCO + C * LDO + 3 * C * LCO;
  static constexpr int GR = G1 > G2 ? G1 : G2;
};

// Grid (nc_max, Hk).
template <typename TI, int C, int D>
__global__ __launch_bounds__(kThreadsB) void k_bwd_grad(Prob p) {
  using OT = TI;
  using CF = GradCfg<TI, C, D>;
  constexpr int NT = kThreadsB, NWV = kWavesB, LDO = CF::LDO, LCO = CF::LCO;
  constexpr int BV = CF::BV, LBO = CF::LBO;
  constexpr int DN = bblk2(D), BN = bblk2(BV);
  typedef OT o4 __attribute__((ext_vector_type(4)));

  __shared__ __align__(16) OT sK[C * LDO];   // K rows (shared by the value heads)
  __shared__ __align__(16) OT sKt[D * LCO];  // K^T
  __shared__ __align__(16) OT sQt[D * LCO];  // Q^T
  __shared__ __align__(16) OT sT[C * LCO];   // T rows (per value head)
  __shared__ __align__(16) OT sTt[C * LCO];  // T^T
  __shared__ __align__(16) OT sR[CF::GR];
  __shared__ float red[R_NSLOT * NWV * C];
  __shared__ float rowv[R_NSLOT * C];
  __shared__ float sg[C], sb[C], se[C], sbeta[C], sdg[C], sred[NT];

  const int c = blockIdx.x, kh = blockIdx.y;
  const ChunkInfo ci = p.chunks[c];
  if (ci.seq < 0) return;
  const int n = ci.len;

  {
    Stage<C, D, NT, TI> gk, gq;
    gk.issue((const TI*)p.k + (int64_t)ci.t0 * p.k_rs + kh * D, p.k_rs, n);
    gq.issue((const TI*)p.q + (int64_t)ci.t0 * p.q_rs + kh * D, p.q_rs, n);
    gk.template to_rows<LDO>(sK);
    gk.template to_cols<LCO>(sKt);
    gq.template to_cols<LCO>(sQt);
  }
  __syncthreads();
  using TCC = Tile<C, C, 1, 1, NWV>;
  using TCD = Tile<C, D, 1, DN, NWV>;
  using TCB = Tile<C, BV, 1, BN, NWV>;
  TCC KK;
  KK.zero();
  gemm_nt<OT, C, C, D, 1, 1, NWV, LDO, LDO>(KK, sK, sK);
  TCD dqf, dkf;  // dq, dk of the key head, summed over its value heads
  dqf.zero();
  dkf.zero();

  for (int hh = 0; hh < p.r; ++hh) {
    const int h = kh * p.r + hh;
    const size_t ch = ch_idx(p, c, h);
    // ---- per-head set-up
    {
      Stage<C, C, NT, OT> gt;
      gt.issue((const OT*)p.sv_T + ch * C * C, C, C);
      gt.template to_rows<LCO>(sT);
      gt.template to_cols<LCO>(sTt);
    }
    for (int i = threadIdx.x; i < C; i += NT) {
      sg[i] = p.sv_gam[ch * C + i];
      sbeta[i] = i < n ? p.beta[(int64_t)(ci.t0 + i) * p.Hv + h] : 0.f;
    }
    for (int i = threadIdx.x; i < R_NSLOT * NWV * C; i += NT) red[i] = 0.f;
    __syncthreads();
    for (int i = threadIdx.x; i < C; i += NT) {
      sb[i] = expf(sg[i]);
      se[i] = expf(sg[C - 1] - sg[i]);
    }
    // ---- phase 1: everything that needs S0 or dS_C, streamed over value-column blocks
    OT* sS0k = sR;              // [D][LBO]  S0 block, key-major
    OT* sdSk = sS0k + D * LBO;  // [D][LBO]  dS_C block, key-major
    OT* sdSv = sdSk + D * LBO;  // [BV][LDO] dS_C block, value-major
    OT* sO = sdSv + BV * LDO;   // [C][LBO]  dO (scale applied to the products)
    OT* sDl = sO + C * LBO;     // [C][LBO]  Delta
    OT* sdD = sDl + C * LBO;    // [C][LBO]  dDelta
    OT* sV = sdD + C * LBO;     // [C][LBO]  V
    OT* sdDt = sV + C * LBO;    // [BV][LCO] dDelta^T
    TCD XQ, XW, XK;
    TCC PP, dT1;
    XQ.zero();
    XW.zero();
    XK.zero();
    PP.zero();
    dT1.zero();
    float sdot = 0.f;
    const OT* S0v = (const OT*)p.sv_S + ch * D * D;
    const OT* dSv = (const OT*)p.ws_dS + ch * D * D;
    const OT* Dlt = (const OT*)p.sv_Dl + ch * D * C;
    const OT* dDt = (const OT*)p.ws_dDt + ch * D * C;
    const TI* dO = (const TI*)p.dO + (int64_t)ci.t0 * p.dO_rs + h * D;
    const TI* V = (const TI*)p.v + (int64_t)ci.t0 * p.v_rs + h * D;
    TI* dV = (TI*)p.dv + (int64_t)ci.t0 * p.dv_rs + h * D;
    for (int v0 = 0; v0 < D; v0 += BV) {
      {
        Stage<BV, D, NT, OT> gs, gd;
        Stage<BV, C, NT, OT> gdl, gdd;
        Stage<C, BV, NT, TI> go, gv;
        gs.issue(S0v + (size_t)v0 * D, D, BV);
        gd.issue(dSv + (size_t)v0 * D, D, BV);
        gdl.issue(Dlt + (size_t)v0 * C, C, BV);
        gdd.issue(dDt + (size_t)v0 * C, C, BV);
        go.issue(dO + v0, p.dO_rs, n);
        gv.issue(V + v0, p.v_rs, n);
        __syncthreads();  // the previous block's readers are done
        gs.template to_cols<LBO>(sS0k);
        gd.template to_cols<LBO>(sdSk);
        gd.template to_rows<LDO>(sdSv);
        gdl.template to_cols<LBO>(sDl);
        gdd.template to_cols<LBO>(sdD);
        gdd.template to_rows<LCO>(sdDt);
        go.template to_rows<LBO>(sO);
        gv.template to_rows<LBO>(sV);
      }
      __syncthreads();
      gemm_nt<OT, C, D, BV, 1, DN, NWV, LBO, LBO>(XQ, sO, sS0k);
      gemm_nt<OT, C, D, BV, 1, DN, NWV, LBO, LBO>(XW, sdD, sS0k);
      gemm_nt<OT, C, D, BV, 1, DN, NWV, LBO, LBO>(XK, sDl, sdSk);
      gemm_nt<OT, C, C, BV, 1, 1, NWV, LBO, LBO>(PP, sO, sDl);
      gemm_nt<OT, C, C, BV, 1, 1, NWV, LBO, LBO>(dT1, sdD, sV);
      {
        TCB kds;
        kds.zero();
        gemm_nt<OT, C, BV, D, 1, BN, NWV, LDO, LDO>(kds, sK, sdSv);
        acc_rowsum(kds, [&](int i, int j, float x) { return se[i] * x * (float)sDl[i * LBO + j]; },
                   red + R_EBAR * NWV * C);
      }
      {
        TCB dvb;
        dvb.zero();
        gemm_nt<OT, C, BV, C, 1, BN, NWV, LCO, LCO>(dvb, sTt, sdDt);
        dvb.each([&](int i, int j, float& x) {
          if (i < n) dV[(int64_t)i * p.dv_rs + v0 + j] = (TI)(sbeta[i] * x);
        });
        acc_rowsum(dvb, [&](int i, int j, float x) { return x * (float)sV[i * LBO + j]; },
                   red + R_DB1 * NWV * C);
      }
      for (int idx = threadIdx.x; idx < D * BV; idx += NT) {
        const int d = idx / BV, v = idx % BV;
        sdot += (float)sS0k[d * LBO + v] * (float)sdSk[d * LBO + v];
      }
    }
    // dO~ = scale dO: XQ and P were formed with dO
    const float sc = p.scale;
    XQ.each([&](int, int, float& x) { x *= sc; });
    PP.each([&](int i, int j, float& x) { x = i >= j ? x * sc : 0.f; });
    XK.each([&](int i, int, float& x) { x *= se[i]; });
    dT1.each([&](int, int j, float& x) { x *= sbeta[j]; });
    __syncthreads();  // phase-1 buffers free
    // ---- phase 2
    OT* sXWt = sR;               // [D][LCO]  XW^T; later Z^T
    OT* sXW = sXWt + D * LCO;    // [C][LDO]  XW;   later G
    OT* sPG = sXW + C * LDO;     // [C][LCO]  P o Gamma
    OT* sPGt = sPG + C * LCO;    // [C][LCO]  (P o Gamma)^T
    OT* sdT = sPGt + C * LCO;    // [C][LCO]  dT;   later G^T
    OT* sZt = sXWt;
    OT* sG = sXW;
    OT* sGt = sdT;
    XW.each4([&](int i0, int d, f32x4& x) {
      *reinterpret_cast<o4*>(sXWt + d * LCO + i0) = o4{(OT)x[0], (OT)x[1], (OT)x[2], (OT)x[3]};
    });
    XW.each([&](int i, int d, float& x) { sXW[i * LDO + d] = (OT)x; });
    PP.each([&](int i, int j, float& x) {
      const float pg = i >= j ? x * expf(sg[i] - sg[j]) : 0.f;
      sPG[i * LCO + j] = (OT)pg;
      sPGt[j * LCO + i] = (OT)pg;
    });
    {
      const TI* Q = (const TI*)p.q + (int64_t)ci.t0 * p.q_rs + kh * D;
      acc_rowsum(XQ, [&](int i, int d, float x) { return i < n ? x * (float)Q[(int64_t)i * p.q_rs + d] : 0.f; },
                 red + R_RQ * NWV * C);
    }
    XQ.each([&](int i, int, float& x) { x *= sb[i]; });
    __syncthreads();
    gemm_nt<OT, C, D, C, 1, DN, NWV, LCO, LCO>(XQ, sPG, sKt);  // dQ of this head
    dqf.each_with(XQ, [&](int, int, float& a, float& b) { a += b; });
    TCD kb;  // dK_beta_b
    kb.zero();
    gemm_nt<OT, C, D, C, 1, DN, NWV, LCO, LCO>(kb, sTt, sXWt);  // T^T XW
    kb.each([&](int, int, float& x) { x = -x; });
    acc_rowsum(kb, [&](int i, int d, float x) { return x * (float)sK[i * LDO + d]; }, red + R_RHO * NWV * C);
    {
      TCC dT;
      dT.zero();
      gemm_nt<OT, C, C, D, 1, 1, NWV, LDO, LDO>(dT, sXW, sK);  // XW K^T
      dT.each_with(dT1, [&](int, int j, float& x, float& t1) { x = t1 - sbeta[j] * sb[j] * x; });
      dT.each([&](int i, int j, float& x) { sdT[i * LCO + j] = (OT)x; });
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
    dL.each([&](int i, int j, float& x) {
      x = i > j ? -x : 0.f;
      const float gv = i > j ? x * sbeta[i] * expf(sg[i] - sg[j]) : 0.f;
      sG[i * LCO + j] = (OT)gv;
      sGt[j * LCO + i] = (OT)gv;
    });
    __syncthreads();
    // dK of this head: e o XK + beta b o dK_beta_b + (P o Gamma)^T Q + G K + G^T K
    XK.each_with(kb, [&](int i, int, float& x, float& y) { x += sbeta[i] * sb[i] * y; });
    gemm_nt<OT, C, D, C, 1, DN, NWV, LCO, LCO>(XK, sPGt, sQt);
    gemm_nt<OT, C, D, C, 1, DN, NWV, LCO, LCO>(XK, sG, sKt);
    gemm_nt<OT, C, D, C, 1, DN, NWV, LCO, LCO>(XK, sGt, sKt);
    dkf.each_with(XK, [&](int, int, float& a, float& b) { a += b; });
    // Gbar o Gamma = P o M + dL o beta_i K K^T o Gamma; dbeta's K K^T term
    {
      const OT* M = (const OT*)p.sv_M + ch * C * C;
      TCC gb = PP;
      gb.each([&](int i, int j, float& x) { x *= (float)M[i * C + j]; });
      dL.each_with(KK, [&](int i, int j, float& x, float& kk) {
        x = i > j ? x * expf(sg[i] - sg[j]) * kk : 0.f;  // dL o Gamma o KK
      });
      gb.each_with(dL, [&](int i, int, float& x, float& t) { x += sbeta[i] * t; });
      acc_rowsum(dL, [&](int, int, float x) { return x; }, red + R_DB3 * NWV * C);
      acc_rowsum(gb, [&](int, int, float x) { return x; }, red + R_GROW * NWV * C);
      acc_colsum(gb, [&](int, int, float x) { return x; }, red + R_GCOL * NWV * C);
    }
    sred[threadIdx.x] = sdot;
    __syncthreads();
    if (threadIdx.x < C) {
      const int i = threadIdx.x;
      for (int s = 0; s < R_NSLOT; ++s) {
        float a = 0.f;
        for (int ww = 0; ww < NWV; ++ww) a += red[(s * NWV + ww) * C + i];
        rowv[s * C + i] = a;
      }
    }
    __syncthreads();
    if (threadIdx.x < C) {
      const int i = threadIdx.x;
      const float ebar = rowv[R_EBAR * C + i], rho = rowv[R_RHO * C + i];
      float dgam = sb[i] * rowv[R_RQ * C + i] + sbeta[i] * sb[i] * rho - ebar + rowv[R_GROW * C + i] -
                   rowv[R_GCOL * C + i];
      if (i == n - 1) {
        float st = 0.f, eb = 0.f;
        for (int k = 0; k < NT; ++k) st += sred[k];
        for (int k = 0; k < C; ++k) eb += rowv[R_EBAR * C + k];
        dgam += expf(sg[C - 1]) * st + eb;
      }
      sdg[i] = dgam;
      if (i < n)
        p.dbeta[(int64_t)(ci.t0 + i) * p.Hv + h] = rowv[R_DB1 * C + i] + sb[i] * rho + rowv[R_DB3 * C + i];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float s = 0.f;
      for (int i = C - 1; i >= 0; --i) {
        s += sdg[i];
        sdg[i] = s;
      }
    }
    __syncthreads();
    if (threadIdx.x < n) {
      const int64_t row = (int64_t)(ci.t0 + threadIdx.x) * p.Hv + h;
      p.dg[row] = sdg[threadIdx.x] / p.g[row];
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
    traced("k_bwd_grad", s, [&] { k_bwd_grad<TI, C, D><<<dim3(p.nc_max, p.Hk), kThreadsB, 0, s>>>(p); });
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
