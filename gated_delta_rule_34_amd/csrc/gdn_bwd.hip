// gdn_bwd.hip -- chunked reverse-mode backward of the gated delta rule on gfx950.
//
// Per-token form: lattice-inference gdn_backward.rs, gdn_backward steps 4a-4d (output,
// state update, delta, retrieval), with the state adjoint dS carried in reverse time.
// Chunk form (derived here; the pages give none), with dO~ = scale dO and the adjoint
// dS_C flowing into the end of a chunk:
//   dDelta = (Gamma o Q K^T)^T dO~ + diag(e) K dS_C,            e = exp(gamma_n - gamma)
//   dS_0   = b_n dS_C + Q^T diag(b) dO~ - W^T dDelta            (carried to the previous chunk)
//   dQ     = diag(b) dO~ S0^T + (P o Gamma) K,                  P = tril(dO~ Delta^T)
//   dW     = -dDelta S0^T,  dT = dDelta (diag(beta) V)^T + dW (diag(beta b) K)^T
//   dV     = diag(beta) T^T dDelta,  dK_beta_b = T^T dW,  dL = strictly_lower(-T^T dT T^T)
//   dK     = (P o Gamma)^T Q + diag(e) Delta dS_C^T + diag(beta b) dK_beta_b + G K + G^T K,
//            G = dL o (beta_i Gamma_ij)
//   dbeta  = rowsum(dV/beta o V) + b o rowsum(dK_beta_b o K) + rowsum(dL o Gamma o K K^T)
//   dgamma = b o rowsum(Q o dO~ S0^T) + beta b rho - ebar + rowsum(Gbar o Gamma) - colsum(Gbar o Gamma)
//            with ebar = e o rowsum((K dS_C) o Delta), Gbar = P o Q K^T + dL o beta_i K K^T,
//            and the last valid row also gets b_n <S0, dS_C> + sum(ebar)
//   dlog g = reverse cumulative sum of dgamma within the chunk;  dg = dlog g / g.
// dq and dk of a key head are the sums over its value heads, added in ascending head
// order by one workgroup per (chunk, key head): no atomics, so every run is bit-identical.
//
// Launch sequence: table -> k_wy -> k_bwd_intra -> k_bwd_state (chunk-serial) ->
// k_bwd_grad1 -> k_bwd_grad2a -> k_bwd_grad2b -> k_bwd_fold.
#include "gdn_common.h"

namespace gdn {

template <int D> struct BwdCfg {
  static constexpr int BV = D < 32 ? D : 32;   // column block of the state sweep
  static constexpr int BG = 16;                // column block of k_bwd_grad1
};

// Grid (nc_max, Hv): Delta = U - W S0 (overwrites U) and dDi = (Gamma o Q K^T)^T dO~.
template <typename TI, int C, int D, int BV>
__global__ __launch_bounds__(NTHREADS) void k_bwd_intra(Prob p) {
  constexpr Prec P = PrecOf<TI>::value;
  constexpr int LD = D + 4, LB = BV + 4, LC = C + 4;
  __shared__ __align__(16) float sQ[C * LD];  // Q, then W
  __shared__ __align__(16) float sK[C * LD];
  __shared__ __align__(16) float sM[C * LC];
  __shared__ __align__(16) float sS[D * LB];
  __shared__ __align__(16) float sU[C * LB];
  __shared__ __align__(16) float sO[C * LB];
  __shared__ __align__(16) float sg[C], ssc[C];
  const int c = blockIdx.x, h = blockIdx.y;
  const ChunkInfo ci = p.chunks[c];
  if (ci.seq < 0) return;
  const int kh = h / p.r, n = ci.len;
  const size_t ch = ch_idx(p, c, h);
  load_tile<C, D, LD>(sQ, (const TI*)p.q + (int64_t)ci.t0 * p.q_rs + kh * D, p.q_rs, n);
  load_tile<C, D, LD>(sK, (const TI*)p.k + (int64_t)ci.t0 * p.k_rs + kh * D, p.k_rs, n);
  for (int i = threadIdx.x; i < C; i += NTHREADS) {
    sg[i] = p.gam[ch * C + i];
    ssc[i] = p.scale;
  }
  __syncthreads();
  {
    Acc<C, C> m;
    m.zero();
    mma<P, C, C, D>(m, rows<LD>(sQ), cols<LD>(sK));
    for_each(m, [&](int i, int j, float x) { sM[i * LC + j] = i >= j ? x * expf(sg[i] - sg[j]) : 0.f; });
  }
  __syncthreads();
  load_tile<C, D, LD>(sQ, p.W + ch * C * D, D, C);
  const TI* dO = (const TI*)p.dO + (int64_t)ci.t0 * p.dO_rs + h * D;
  for (int j0 = 0; j0 < D; j0 += BV) {
    load_tile<D, BV, LB>(sS, p.states + ch * D * D + j0, D, D);
    load_tile<C, BV, LB>(sU, p.U + ch * C * D + j0, D, C);
    load_tile<C, BV, LB>(sO, dO + j0, p.dO_rs, n, ssc);
    __syncthreads();
    Acc<C, BV> a, b;
    a.zero();
    b.zero();
    mma<P, C, BV, D>(a, rows<LD>(sQ), rows<LB>(sS));
    mma<P, C, BV, C>(b, cols<LC>(sM), rows<LB>(sO));
    for_each2(a, b, [&](int i, int j, float x, float y) {
      p.U[ch * C * D + (size_t)i * D + j0 + j] = sU[i * LB + j] - x;
      p.dDi[ch * C * D + (size_t)i * D + j0 + j] = y;
    });
    __syncthreads();
  }
}

// Grid (N, Hv, D / BV). Reverse chunk sweep of the state adjoint; saves dS_C of
// every chunk and dDelta.
template <typename TI, int C, int D, int BV>
__global__ __launch_bounds__(NTHREADS) void k_bwd_state(Prob p) {
  constexpr Prec P = PrecOf<TI>::value;
  constexpr int LD = D + 4, LB = BV + 4;
  __shared__ __align__(16) float sdS[D * LB];
  __shared__ __align__(16) float sX[C * LD];
  __shared__ __align__(16) float sDb[C * LB];
  __shared__ __align__(16) float sO[C * LB];
  __shared__ __align__(16) float sg[C], se[C], sb[C], ssc[C];
  const int n = blockIdx.x, h = blockIdx.y, j0 = blockIdx.z * BV;
  const int kh = h / p.r;
  const size_t nh = (size_t)n * p.Hv + h;
  if (p.dST)
    load_tile<D, BV, LB>(sdS, p.dST + nh * D * D + j0, D, D);
  else
    for (int idx = threadIdx.x; idx < D * BV; idx += NTHREADS) sdS[(idx / BV) * LB + idx % BV] = 0.f;
  for (int i = threadIdx.x; i < C; i += NTHREADS) ssc[i] = p.scale;
  const int c0 = p.seq_chunk[n], c1 = p.seq_chunk[n + 1];
  __syncthreads();
  for (int c = c1 - 1; c >= c0; --c) {
    const ChunkInfo ci = p.chunks[c];
    const size_t ch = ch_idx(p, c, h);
    store_tile<D, BV, LB>(p.dstates + ch * D * D + j0, D, sdS, D);
    for (int i = threadIdx.x; i < C; i += NTHREADS) sg[i] = p.gam[ch * C + i];
    __syncthreads();
    for (int i = threadIdx.x; i < C; i += NTHREADS) {
      se[i] = expf(sg[C - 1] - sg[i]);
      sb[i] = expf(sg[i]);
    }
    __syncthreads();
    load_tile<C, D, LD>(sX, (const TI*)p.k + (int64_t)ci.t0 * p.k_rs + kh * D, p.k_rs, ci.len, se);
    load_tile<C, BV, LB>(sDb, p.dDi + ch * C * D + j0, D, C);
    __syncthreads();
    {
      Acc<C, BV> a;
      a.zero();
      mma<P, C, BV, D>(a, rows<LD>(sX), rows<LB>(sdS));
      for_each(a, [&](int i, int j, float x) {
        const float d = sDb[i * LB + j] + x;
        sDb[i * LB + j] = d;
        p.dDel[ch * C * D + (size_t)i * D + j0 + j] = d;
      });
    }
    __syncthreads();
    load_tile<C, D, LD>(sX, (const TI*)p.q + (int64_t)ci.t0 * p.q_rs + kh * D, p.q_rs, ci.len, sb);
    load_tile<C, BV, LB>(sO, (const TI*)p.dO + (int64_t)ci.t0 * p.dO_rs + h * D + j0, p.dO_rs, ci.len, ssc);
    __syncthreads();
    Acc<D, BV> s1, s2;
    s1.zero();
    s2.zero();
    mma<P, D, BV, C>(s1, cols<LD>(sX), rows<LB>(sO));
    __syncthreads();
    load_tile<C, D, LD>(sX, p.W + ch * C * D, D, C);
    __syncthreads();
    mma<P, D, BV, C>(s2, cols<LD>(sX), rows<LB>(sDb));
    const float bn = expf(sg[C - 1]);
    for_each2(s1, s2, [&](int i, int j, float x, float y) { sdS[i * LB + j] = bn * sdS[i * LB + j] + x - y; });
    __syncthreads();
  }
  if (p.dS0) store_tile<D, BV, LB>(p.dS0 + nh * D * D + j0, D, sdS, D);
}

// Grid (nc_max, Hv). Everything that needs the chunk's S0 or dS_C, streamed over
// column blocks of BG: XQ, XW, XK, P, dT's dU part, ebar, <S0, dS_C>, dV and its dbeta part.
template <typename TI, int C, int D, int BG>
__global__ __launch_bounds__(NTHREADS) void k_bwd_grad1(Prob p) {
  constexpr Prec P = PrecOf<TI>::value;
  constexpr int LB = BG + 4, LC = C + 4;
  __shared__ __align__(16) float sS0[D * LB];
  __shared__ __align__(16) float sdS[D * LB];
  __shared__ __align__(16) float sDl[C * LB];   // Delta
  __shared__ __align__(16) float sDe[C * LB];   // diag(e) Delta
  __shared__ __align__(16) float sdD[C * LB];   // dDelta
  __shared__ __align__(16) float sDi[C * LB];   // intra part of dDelta
  __shared__ __align__(16) float sO[C * LB];    // dO~
  __shared__ __align__(16) float sVb[C * LB];   // diag(beta) V
  __shared__ __align__(16) float sV[C * LB];    // V
  __shared__ __align__(16) float sR[C * LB];    // dVbeta o V
  __shared__ __align__(16) float sT[C * LC];
  __shared__ __align__(16) float sg[C], se[C], sbeta[C], ssc[C], sred[NTHREADS];
  const int c = blockIdx.x, h = blockIdx.y;
  const ChunkInfo ci = p.chunks[c];
  if (ci.seq < 0) return;
  const int n = ci.len;
  const size_t ch = ch_idx(p, c, h);
  load_tile<C, C, LC>(sT, p.Tm + ch * C * C, C, C);
  for (int i = threadIdx.x; i < C; i += NTHREADS) {
    sg[i] = p.gam[ch * C + i];
    sbeta[i] = i < n ? p.beta[(int64_t)(ci.t0 + i) * p.Hv + h] : 0.f;
    ssc[i] = p.scale;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < C; i += NTHREADS) se[i] = expf(sg[C - 1] - sg[i]);
  Acc<C, D> XQ, XW, XK;
  Acc<C, C> PP, dT1;
  XQ.zero(); XW.zero(); XK.zero(); PP.zero(); dT1.zero();
  float ebar = 0.f, db1 = 0.f, sdot = 0.f;  // thread i < C owns row i of ebar and db1
  const TI* V = (const TI*)p.v + (int64_t)ci.t0 * p.v_rs + h * D;
  const TI* dO = (const TI*)p.dO + (int64_t)ci.t0 * p.dO_rs + h * D;
  TI* dV = (TI*)p.dv + (int64_t)ci.t0 * p.dv_rs + h * D;
  for (int j0 = 0; j0 < D; j0 += BG) {
    __syncthreads();
    load_tile<D, BG, LB>(sS0, p.states + ch * D * D + j0, D, D);
    load_tile<D, BG, LB>(sdS, p.dstates + ch * D * D + j0, D, D);
    load_tile<C, BG, LB>(sDl, p.U + ch * C * D + j0, D, C);
    load_tile<C, BG, LB>(sDe, p.U + ch * C * D + j0, D, C, se);
    load_tile<C, BG, LB>(sdD, p.dDel + ch * C * D + j0, D, C);
    load_tile<C, BG, LB>(sDi, p.dDi + ch * C * D + j0, D, C);
    load_tile<C, BG, LB>(sO, dO + j0, p.dO_rs, n, ssc);
    load_tile<C, BG, LB>(sVb, V + j0, p.v_rs, n, sbeta);
    load_tile<C, BG, LB>(sV, V + j0, p.v_rs, n);
    __syncthreads();
    mma<P, C, D, BG>(XQ, rows<LB>(sO), cols<LB>(sS0));
    mma<P, C, D, BG>(XW, rows<LB>(sdD), cols<LB>(sS0));
    mma<P, C, D, BG>(XK, rows<LB>(sDe), cols<LB>(sdS));
    mma<P, C, C, BG>(PP, rows<LB>(sO), cols<LB>(sDl));
    mma<P, C, C, BG>(dT1, rows<LB>(sdD), cols<LB>(sVb));
    {
      Acc<C, BG> a;
      a.zero();
      mma<P, C, BG, C>(a, cols<LC>(sT), rows<LB>(sdD));
      for_each(a, [&](int i, int j, float x) {
        if (i < n) dV[(int64_t)i * p.dv_rs + j0 + j] = from_f<TI>(sbeta[i] * x);
        sR[i * LB + j] = x * sV[i * LB + j];
      });
    }
    for (int idx = threadIdx.x; idx < D * BG; idx += NTHREADS) {
      const int i = idx / BG, j = idx % BG;
      sdot += sS0[i * LB + j] * sdS[i * LB + j];
    }
    if (threadIdx.x < C) {
      const int i = threadIdx.x;
      for (int j = 0; j < BG; ++j) ebar += (sdD[i * LB + j] - sDi[i * LB + j]) * sDl[i * LB + j];
    }
    __syncthreads();
    if (threadIdx.x < C) {
      const int i = threadIdx.x;
      for (int j = 0; j < BG; ++j) db1 += sR[i * LB + j];
    }
  }
  const size_t cd = ch * C * D, cc = ch * C * C;
  for_each(XQ, [&](int i, int j, float x) { p.XQ[cd + i * D + j] = x; });
  for_each(XW, [&](int i, int j, float x) { p.XW[cd + i * D + j] = x; });
  for_each(XK, [&](int i, int j, float x) { p.XK[cd + i * D + j] = x; });
  for_each(PP, [&](int i, int j, float x) { p.Pb[cc + i * C + j] = i >= j ? x : 0.f; });
  for_each(dT1, [&](int i, int j, float x) { p.dT[cc + i * C + j] = x; });
  if (threadIdx.x < C) {
    p.ebar[ch * C + threadIdx.x] = ebar;
    p.db1[ch * C + threadIdx.x] = db1;
  }
  sred[threadIdx.x] = sdot;
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int i = 0; i < NTHREADS; ++i) s += sred[i];
    p.sdot[ch] = s;
  }
}

// Grid (nc_max, Hv): dQ of this value head, dK_beta_b, rho, rowsum(Q o XQ), and dT.
template <typename TI, int C, int D>
__global__ __launch_bounds__(NTHREADS) void k_bwd_grad2a(Prob p) {
  constexpr Prec P = PrecOf<TI>::value;
  constexpr int LD = D + 4, LC = C + 4;
  __shared__ __align__(16) float sK[C * LD];
  __shared__ __align__(16) float sX[C * LD];  // XQ, then XW, then dK_beta_b o K
  __shared__ __align__(16) float sT[C * LC];
  __shared__ __align__(16) float sPG[C * LC];
  __shared__ __align__(16) float sg[C], sb[C], sbeta[C];
  const int c = blockIdx.x, h = blockIdx.y;
  const ChunkInfo ci = p.chunks[c];
  if (ci.seq < 0) return;
  const int kh = h / p.r, n = ci.len;
  const size_t ch = ch_idx(p, c, h);
  const size_t cd = ch * C * D, cc = ch * C * C;
  load_tile<C, D, LD>(sK, (const TI*)p.k + (int64_t)ci.t0 * p.k_rs + kh * D, p.k_rs, n);
  load_tile<C, C, LC>(sT, p.Tm + cc, C, C);
  load_tile<C, D, LD>(sX, p.XQ + cd, D, C);
  for (int i = threadIdx.x; i < C; i += NTHREADS) {
    sg[i] = p.gam[ch * C + i];
    sbeta[i] = i < n ? p.beta[(int64_t)(ci.t0 + i) * p.Hv + h] : 0.f;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < C; i += NTHREADS) sb[i] = expf(sg[i]);
  for (int idx = threadIdx.x; idx < C * C; idx += NTHREADS) {
    const int i = idx / C, j = idx % C;
    sPG[i * LC + j] = i >= j ? p.Pb[cc + idx] * expf(sg[i] - sg[j]) : 0.f;
  }
  __syncthreads();
  {
    Acc<C, D> a;
    a.zero();
    mma<P, C, D, C>(a, rows<LC>(sPG), rows<LD>(sK));
    for_each(a, [&](int i, int j, float x) { p.dqh[cd + i * D + j] = sb[i] * sX[i * LD + j] + x; });
  }
  if (threadIdx.x < C) {
    const int i = threadIdx.x;
    float s = 0.f;
    if (i < n) {
      const TI* Q = (const TI*)p.q + (int64_t)(ci.t0 + i) * p.q_rs + kh * D;
      for (int d = 0; d < D; ++d) s += to_f(Q[d]) * sX[i * LD + d];
    }
    p.rq[ch * C + i] = s;
  }
  __syncthreads();
  load_tile<C, D, LD>(sX, p.XW + cd, D, C);
  __syncthreads();
  Acc<C, D> kb;
  Acc<C, C> dt;
  kb.zero();
  dt.zero();
  mma<P, C, D, C>(kb, cols<LC>(sT), rows<LD>(sX));
  mma<P, C, C, D>(dt, rows<LD>(sX), cols<LD>(sK));
  for_each(dt, [&](int i, int j, float x) { p.dT[cc + i * C + j] -= sbeta[j] * sb[j] * x; });
  __syncthreads();
  for_each(kb, [&](int i, int j, float x) {
    p.dKbb[cd + i * D + j] = -x;
    sX[i * LD + j] = -x * sK[i * LD + j];
  });
  __syncthreads();
  if (threadIdx.x < C) {
    const int i = threadIdx.x;
    float s = 0.f;
    for (int d = 0; d < D; ++d) s += sX[i * LD + d];
    p.rho[ch * C + i] = s;
  }
}

// Grid (nc_max, Hv): dL, G, dK of this value head, dbeta and dg.
template <typename TI, int C, int D>
__global__ __launch_bounds__(NTHREADS) void k_bwd_grad2b(Prob p) {
  constexpr Prec P = PrecOf<TI>::value;
  constexpr int LD = D + 4, LC = C + 4;
  __shared__ __align__(16) float sQ[C * LD];
  __shared__ __align__(16) float sK[C * LD];
  __shared__ __align__(16) float sB1[C * LC];  // T, then dL
  __shared__ __align__(16) float sB2[C * LC];  // dT, then Z = dT T^T, then G, then dL o Gamma o KK
  __shared__ __align__(16) float sB3[C * LC];  // P o Gamma, then Gbar o Gamma
  __shared__ __align__(16) float sg[C], sb[C], sbeta[C], sdg[C];
  const int c = blockIdx.x, h = blockIdx.y;
  const ChunkInfo ci = p.chunks[c];
  if (ci.seq < 0) return;
  const int kh = h / p.r, n = ci.len;
  const size_t ch = ch_idx(p, c, h);
  const size_t cd = ch * C * D, cc = ch * C * C;
  load_tile<C, C, LC>(sB1, p.Tm + cc, C, C);
  load_tile<C, C, LC>(sB2, p.dT + cc, C, C);
  for (int i = threadIdx.x; i < C; i += NTHREADS) {
    sg[i] = p.gam[ch * C + i];
    sbeta[i] = i < n ? p.beta[(int64_t)(ci.t0 + i) * p.Hv + h] : 0.f;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < C; i += NTHREADS) sb[i] = expf(sg[i]);
  {
    Acc<C, C> z;
    z.zero();
    mma<P, C, C, C>(z, rows<LC>(sB2), cols<LC>(sB1));
    __syncthreads();
    for_each(z, [&](int i, int j, float x) { sB2[i * LC + j] = x; });
  }
  __syncthreads();
  {
    Acc<C, C> dl;
    dl.zero();
    mma<P, C, C, C>(dl, cols<LC>(sB1), rows<LC>(sB2));
    __syncthreads();
    for_each(dl, [&](int i, int j, float x) { sB1[i * LC + j] = i > j ? -x : 0.f; });
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < C * C; idx += NTHREADS) {
    const int i = idx / C, j = idx % C;
    const float G = i >= j ? expf(sg[i] - sg[j]) : 0.f;
    sB2[i * LC + j] = sB1[i * LC + j] * sbeta[i] * G;
    sB3[i * LC + j] = p.Pb[cc + idx] * G;
  }
  load_tile<C, D, LD>(sQ, (const TI*)p.q + (int64_t)ci.t0 * p.q_rs + kh * D, p.q_rs, n);
  load_tile<C, D, LD>(sK, (const TI*)p.k + (int64_t)ci.t0 * p.k_rs + kh * D, p.k_rs, n);
  __syncthreads();
  {
    Acc<C, D> a;
    a.zero();
    mma<P, C, D, C>(a, cols<LC>(sB3), rows<LD>(sQ));
    mma<P, C, D, C>(a, rows<LC>(sB2), rows<LD>(sK));
    mma<P, C, D, C>(a, cols<LC>(sB2), rows<LD>(sK));
    for_each(a, [&](int i, int j, float x) {
      p.dkh[cd + i * D + j] = x + p.XK[cd + i * D + j] + sbeta[i] * sb[i] * p.dKbb[cd + i * D + j];
    });
  }
  Acc<C, C> qk, kk;
  qk.zero();
  kk.zero();
  mma<P, C, C, D>(qk, rows<LD>(sQ), cols<LD>(sK));
  mma<P, C, C, D>(kk, rows<LD>(sK), cols<LD>(sK));
  __syncthreads();
  for_each2(qk, kk, [&](int i, int j, float xq, float xk) {
    float gb = 0.f, dbt = 0.f;
    if (i >= j) {
      const float G = expf(sg[i] - sg[j]);
      const float dL = sB1[i * LC + j];
      gb = (p.Pb[cc + i * C + j] * xq + dL * sbeta[i] * xk) * G;
      dbt = dL * G * xk;
    }
    sB3[i * LC + j] = gb;
    sB2[i * LC + j] = dbt;
  });
  __syncthreads();
  if (threadIdx.x < C) {
    const int i = threadIdx.x;
    float rs = 0.f, cs = 0.f, bt = 0.f;
    for (int j = 0; j < C; ++j) {
      rs += sB3[i * LC + j];
      cs += sB3[j * LC + i];
      bt += sB2[i * LC + j];
    }
    const float rho = p.rho[ch * C + i];
    float dgam = sb[i] * p.rq[ch * C + i] + sbeta[i] * sb[i] * rho - p.ebar[ch * C + i] + rs - cs;
    if (i == n - 1) {
      float se = 0.f;
      for (int k = 0; k < C; ++k) se += p.ebar[ch * C + k];
      dgam += expf(sg[C - 1]) * p.sdot[ch] + se;
    }
    sdg[i] = dgam;
    if (i < n) p.dbeta[(int64_t)(ci.t0 + i) * p.Hv + h] = p.db1[ch * C + i] + sb[i] * rho + bt;
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
}

// Grid (nc_max, Hk): dq, dk of a key head = sum over its value heads in ascending order.
template <typename TI, int C, int D>
__global__ __launch_bounds__(NTHREADS) void k_bwd_fold(Prob p) {
  const int c = blockIdx.x, kh = blockIdx.y;
  const ChunkInfo ci = p.chunks[c];
  if (ci.seq < 0) return;
  const int n = ci.len;
  TI* dq = (TI*)p.dq + (int64_t)ci.t0 * p.dq_rs + kh * D;
  TI* dk = (TI*)p.dk + (int64_t)ci.t0 * p.dk_rs + kh * D;
  for (int idx = threadIdx.x; idx < n * D; idx += NTHREADS) {
    const int i = idx / D, d = idx % D;
    float sq = 0.f, sk = 0.f;
    for (int h = kh * p.r; h < kh * p.r + p.r; ++h) {
      const size_t off = ch_idx(p, c, h) * C * D + idx;
      sq += p.dqh[off];
      sk += p.dkh[off];
    }
    dq[(int64_t)i * p.dq_rs + d] = from_f<TI>(sq);
    dk[(int64_t)i * p.dk_rs + d] = from_f<TI>(sk);
  }
}

template <typename TI, int C, int D>
static hipError_t bwd_seq(const Prob& p, hipStream_t s) {
  constexpr int BV = BwdCfg<D>::BV, BG = BwdCfg<D>::BG;
  traced("k_table", s, [&] { k_table<C><<<1, NTHREADS, 0, s>>>(p); });
  if (p.nc_max > 0) {
    traced("k_wy", s, [&] { k_wy<TI, C, D><<<dim3(p.nc_max, p.Hv), NTHREADS, 0, s>>>(p); });
    traced("k_bwd_intra", s, [&] { k_bwd_intra<TI, C, D, BV><<<dim3(p.nc_max, p.Hv), NTHREADS, 0, s>>>(p); });
  }
  if (p.N > 0) traced("k_bwd_state", s, [&] { k_bwd_state<TI, C, D, BV><<<dim3(p.N, p.Hv, D / BV), NTHREADS, 0, s>>>(p); });
  if (p.nc_max > 0) {
    traced("k_bwd_grad1", s, [&] { k_bwd_grad1<TI, C, D, BG><<<dim3(p.nc_max, p.Hv), NTHREADS, 0, s>>>(p); });
    traced("k_bwd_grad2a", s, [&] { k_bwd_grad2a<TI, C, D><<<dim3(p.nc_max, p.Hv), NTHREADS, 0, s>>>(p); });
    traced("k_bwd_grad2b", s, [&] { k_bwd_grad2b<TI, C, D><<<dim3(p.nc_max, p.Hv), NTHREADS, 0, s>>>(p); });
    traced("k_bwd_fold", s, [&] { k_bwd_fold<TI, C, D><<<dim3(p.nc_max, p.Hk), NTHREADS, 0, s>>>(p); });
  }
  return hipGetLastError();
}

template <typename TI, int C>
static hipError_t bwd_d(const Prob& p, hipStream_t s) {
  switch (p.D) {
    case 16: return bwd_seq<TI, C, 16>(p, s);
    case 32: return bwd_seq<TI, C, 32>(p, s);
    case 64: return bwd_seq<TI, C, 64>(p, s);
    case 128: return bwd_seq<TI, C, 128>(p, s);
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
