// gdn_fwd.hip -- chunked forward of the gated delta rule on gfx950.
//
// Chunk form (derived from the per-token recurrence of the lattice-inference
// gdn_backward.rs page, "Forward recap"; the pages print no chunk algebra). Within a
// chunk of n <= C tokens starting from state S:
//   gamma = cumsum(log g),  b = exp(gamma),  Gamma_rs = exp(gamma_r - gamma_s) [r >= s]
//   L = strictly_lower(diag(beta) (Gamma o K K^T)),  T = (I + L)^-1
//   W = T diag(beta b) K,  U = T diag(beta) V,  Delta = U - W S   (Delta_r = delta_r)
//   O = scale (diag(b) Q S + (Gamma o Q K^T) Delta)
//   S_next = b_n S + K^T diag(exp(gamma_n - gamma)) Delta
// Rows past the end of a partial chunk carry k = q = v = beta = 0 and log g = 0.
//
// Two kernels after the chunk table:
//  k_prep  (chunk x key head, 8 waves): K K^T and Q K^T once for the r value heads of the
//          key head; per value head gamma, the blocked inverse T, W, U and
//          M = Gamma o Q K^T. Everything the serial pass and the backward need is written
//          once, in the storage type, in the layout its consumer reads.
//  k_sweep (sequence x value head, 8 waves): the chunk-serial pass. The state lives in
//          float32 MFMA accumulators; per chunk it forms Delta = U - W S, the output
//          O = diag(b) Q S + M Delta, and S <- b_n S + K^T (e o Delta), while the next
//          chunk's operands are loaded into registers.
#include "gdn_common.h"
#include "gdn_mma.h"

namespace gdn {

constexpr int kWaves = 8;              // k_sweep
constexpr int kThreads = kWaves * 64;
constexpr int kPrepWaves = 16;         // k_prep
constexpr int kPrepThreads = kPrepWaves * 64;

__host__ __device__ constexpr int blk2(int x) { return x >= 32 ? 2 : 1; }

// T := (I + L)^-1 for strictly lower triangular L (float32 LDS, row stride LC).
// Diagonal 16 x 16 blocks by forward substitution, one column per lane, then the
// off-diagonal blocks level by level: T_ij = -T_ii sum_{k=j}^{i-1} L_ik T_kj, with
// float32 MFMA. X is scratch for 3 tiles of 16 x 20 floats. Ends with a barrier.
template <int C, int LC, int NWV>
__device__ __forceinline__ void invert_unit_lower(const float* L, float* T, float* X) {
  constexpr int NB = C / 16;
  const int w = threadIdx.x / 64, l = threadIdx.x & 63;
  for (int idx = threadIdx.x; idx < C * C; idx += NWV * 64) {
    const int i = idx / C, j = idx % C;
    if (i / 16 < j / 16) T[i * LC + j] = 0.f;  // upper off-diagonal blocks
  }
  if (w < NB && l < 16) {
    const int o = w * 16, j = l;
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
  for (int d = 1; d < NB; ++d) {
    const int npairs = NB - d;
    const int bi = w + d, bj = w;  // wave w < npairs owns block (w + d, w)
    if (w < npairs) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int kb = bj; kb < bi; ++kb)
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) {
          const float a = L[(bi * 16 + (l & 15)) * LC + kb * 16 + k0 + (l >> 4)];
          const float b = T[(kb * 16 + k0 + (l >> 4)) * LC + bj * 16 + (l & 15)];
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
        }
#pragma unroll
      for (int e = 0; e < 4; ++e) X[w * 320 + ((l >> 4) * 4 + e) * 20 + (l & 15)] = acc[e];
    }
    lds_barrier();
    if (w < npairs) {
      f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < 16; k0 += 4) {
        const float a = T[(bi * 16 + (l & 15)) * LC + bi * 16 + k0 + (l >> 4)];
        const float b = X[w * 320 + (k0 + (l >> 4)) * 20 + (l & 15)];
        r = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, r, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) T[(bi * 16 + (l >> 4) * 4 + e) * LC + bj * 16 + (l & 15)] = -r[e];
    }
    lds_barrier();
  }
}

// Grid (nc_max, Hk).
template <typename TI, int C, int D>
__global__ __launch_bounds__(kPrepThreads) void k_prep(Prob p) {
  using OT = TI;
  constexpr int NT = kPrepThreads, NWV = kPrepWaves, LDO = D + 8, LCO = C + 8, LCF = C + 4;
  __shared__ __align__(16) OT sK[C * LDO];
  __shared__ __align__(16) OT sQ[C * LDO];
  __shared__ __align__(16) OT sKt[D * LCO];
  __shared__ __align__(16) OT sVt[D * LCO];  // V^T of each value head
  __shared__ __align__(16) float sL[C * LCF];
  __shared__ __align__(16) float sT[C * LCF];
  __shared__ __align__(16) OT sTp[C * LCO];   // T diag(beta b)
  __shared__ __align__(16) OT sTpp[C * LCO];  // T diag(beta)
  __shared__ __align__(16) float sX[3 * 320];
  __shared__ float sg[C], sb[C], sbeta[C];
  typedef OT o4 __attribute__((ext_vector_type(4)));
  const int c = blockIdx.x, kh = blockIdx.y;
  const ChunkInfo ci = p.chunks[c];
  if (ci.seq < 0) return;
  const int n = ci.len;
  const size_t ck = (size_t)c * p.Hk + kh;

  Stage<C, D, NT, TI> gq;  // Q stays in registers: (diag(b) Q)^T is written per value head
  {
    Stage<C, D, NT, TI> gk;
    gk.issue((const TI*)p.k + (int64_t)ci.t0 * p.k_rs + kh * D, p.k_rs, n);
    gq.issue((const TI*)p.q + (int64_t)ci.t0 * p.q_rs + kh * D, p.q_rs, n);
    gk.template to_rows<LDO>(sK);
    gk.template to_cols<LCO>(sKt);
    gq.template to_rows<LDO>(sQ);
    gq.template to_cols<LCO>(sVt);  // Q^T, saved for the backward
  }
  lds_barrier();
  lds_to_global<D, C, LCO, NT>((OT*)p.sv_Kt + ck * D * C, sKt);
  lds_to_global<D, C, LCO, NT>((OT*)p.sv_Qt + ck * D * C, sVt);
  Tile<C, C, 1, 1, NWV> KK, QK;
  KK.zero();
  QK.zero();
  gemm_nt<OT, C, C, D, 1, 1, NWV, LDO, LDO>(KK, sK, sK);
  gemm_nt<OT, C, C, D, 1, 1, NWV, LDO, LDO>(QK, sQ, sK);

  Stage<C, D, NT, TI> gv;
  gv.issue((const TI*)p.v + (int64_t)ci.t0 * p.v_rs + (kh * p.r) * D, p.v_rs, n);
  for (int hh = 0; hh < p.r; ++hh) {
    const int h = kh * p.r + hh;
    const size_t ch = ch_idx(p, c, h);
    for (int i = threadIdx.x; i < C; i += NT) {
      const bool ok = i < n;
      sbeta[i] = ok ? p.beta[(int64_t)(ci.t0 + i) * p.Hv + h] : 0.f;
      sg[i] = ok ? logf(p.g[(int64_t)(ci.t0 + i) * p.Hv + h]) : 0.f;
    }
    lds_barrier();
    gv.template to_cols<LCO>(sVt);
    if (hh + 1 < p.r) gv.issue((const TI*)p.v + (int64_t)ci.t0 * p.v_rs + (h + 1) * D, p.v_rs, n);
    if (threadIdx.x < 64) {
      const float x = wave_scan_incl(threadIdx.x < C ? sg[threadIdx.x] : 0.f);
      if (threadIdx.x < C) sg[threadIdx.x] = x;
    }
    lds_barrier();
    for (int i = threadIdx.x; i < C; i += NT) {
      sb[i] = expf(sg[i]);
      p.sv_gam[ch * C + i] = sg[i];
    }
    KK.each([&](int i, int j, float& x) {
      sL[i * LCF + j] = i > j ? sbeta[i] * expf(sg[i] - sg[j]) * x : 0.f;
    });
    OT* M = (OT*)p.sv_M + ch * C * C;
    QK.each([&](int i, int j, float& x) { M[i * C + j] = (OT)(i >= j ? expf(sg[i] - sg[j]) * x : 0.f); });
    lds_barrier();
    invert_unit_lower<C, LCF, NWV>(sL, sT, sX);
    OT* Ttsv = (OT*)p.sv_Tt + ch * C * C;
    for (int idx = threadIdx.x; idx < C * C; idx += NT) {
      const int i = idx / C, j = idx % C;
      const float t = sT[i * LCF + j];
      Ttsv[idx] = (OT)sT[j * LCF + i];
      sTp[i * LCO + j] = (OT)(t * sbeta[j] * sb[j]);
      sTpp[i * LCO + j] = (OT)(t * sbeta[j]);
    }
    lds_barrier();
    {
      Tile<C, D, 1, blk2(D), NWV> w;
      w.zero();
      gemm_nt<OT, C, D, C, 1, blk2(D), NWV, LCO, LCO>(w, sTp, sKt);
      OT* W = (OT*)p.sv_W + ch * C * D;
      w.each([&](int i, int d, float& x) { W[i * D + d] = (OT)x; });
    }
    {
      Tile<C, D, 1, blk2(D), NWV> u;
      u.zero();
      gemm_nt<OT, C, D, C, 1, blk2(D), NWV, LCO, LCO>(u, sTpp, sVt);
      OT* Ut = (OT*)p.ws_Ut + ch * D * C;
      u.each4([&](int i0, int v, f32x4& x) {
        *reinterpret_cast<o4*>(Ut + v * C + i0) = o4{(OT)x[0], (OT)x[1], (OT)x[2], (OT)x[3]};
      });
    }
    lds_barrier();  // sVt free: stage (diag(b) Q)^T for the backward
    gq.template to_cols<LCO>(sVt, sb);
    lds_barrier();
    lds_to_global<D, C, LCO, NT>((OT*)p.sv_Qbt + ch * D * C, sVt);
  }
}

// Grid (N, Hv). Chunk-serial pass over one sequence and one value head.
template <typename TI, int C, int D>
__global__ __launch_bounds__(kThreads) void k_sweep(Prob p) {
  using OT = TI;
  constexpr int NT = kThreads, LDO = D + 8, LCO = C + 8;
  constexpr int SM = blk2(D), DN = blk2(D);
  __shared__ __align__(16) OT sW[C * LDO];
  __shared__ __align__(16) OT sQ[C * LDO];
  __shared__ __align__(16) OT sM[C * LCO];
  __shared__ __align__(16) OT sKt[D * LCO];
  __shared__ __align__(16) OT sSt[D * LDO];   // S^T: [v][d]
  __shared__ __align__(16) OT sDt[D * LCO];   // Delta^T: [v][i]
  __shared__ __align__(16) OT sDet[D * LCO];  // (e o Delta)^T
  __shared__ float sg[C], sb[C], se[C];
  typedef OT o4 __attribute__((ext_vector_type(4)));

  const int n = blockIdx.x, h = blockIdx.y, kh = h / p.r;
  const size_t nh = (size_t)n * p.Hv + h;
  const int c0 = p.seq_chunk[n], c1 = p.seq_chunk[n + 1];

  using TS = Tile<D, D, SM, SM, kWaves>;
  using TD = Tile<C, D, 1, DN, kWaves>;
  TS S;
  if (p.S0) {
    const float* s0 = p.S0 + nh * D * D;
    S.each([&](int d, int v, float& x) { x = s0[d * D + v]; });
  } else {
    S.zero();
  }

  Stage<C, D, NT, OT> nW;
  Stage<C, D, NT, TI> nQ;
  Stage<C, C, NT, OT> nM;
  Stage<D, C, NT, OT> nKt;
  float ng = 0.f;
  auto issue = [&](int c) {
    const ChunkInfo ci = p.chunks[c];
    const size_t ch = ch_idx(p, c, h), ck = (size_t)c * p.Hk + kh;
    nW.issue((const OT*)p.sv_W + ch * C * D, D, C);
    nQ.issue((const TI*)p.q + (int64_t)ci.t0 * p.q_rs + kh * D, p.q_rs, ci.len);
    nM.issue((const OT*)p.sv_M + ch * C * C, C, C);
    nKt.issue((const OT*)p.sv_Kt + ck * D * C, C, D);
    if (threadIdx.x < C) ng = p.sv_gam[ch * C + threadIdx.x];
  };
  auto commit = [&]() {
    nW.template to_rows<LDO>(sW);
    nQ.template to_rows<LDO>(sQ);
    nM.template to_rows<LCO>(sM);
    nKt.template to_rows<LCO>(sKt);
    if (threadIdx.x < C) sg[threadIdx.x] = ng;
  };
  auto state_to_lds = [&]() {
    S.each4([&](int d0, int v, f32x4& x) {
      *reinterpret_cast<o4*>(sSt + v * LDO + d0) = o4{(OT)x[0], (OT)x[1], (OT)x[2], (OT)x[3]};
    });
  };

  if (c0 < c1) {
    issue(c0);
    commit();
  }
  state_to_lds();
  lds_barrier();
  for (int c = c0; c < c1; ++c) {
    const ChunkInfo ci = p.chunks[c];
    const size_t ch = ch_idx(p, c, h);
    if (threadIdx.x < C) {
      sb[threadIdx.x] = expf(sg[threadIdx.x]);
      se[threadIdx.x] = expf(sg[C - 1] - sg[threadIdx.x]);
    }
    if (c + 1 < c1) issue(c + 1);
    TD U;  // U of this chunk, in the accumulator layout of Delta
    {
      const OT* Ut = (const OT*)p.ws_Ut + ch * D * C;
      U.each4([&](int i0, int v, f32x4& x) {
        const o4 u = *reinterpret_cast<const o4*>(Ut + v * C + i0);
        x = f32x4{(float)u[0], (float)u[1], (float)u[2], (float)u[3]};
      });
    }
    // the chunk's start state, saved for the backward (key-major, from its LDS copy)
    lds_to_global_t<D, D, LDO, NT>((OT*)p.sv_S + ch * D * D, sSt);
    TD WS, O;
    WS.zero();
    O.zero();
    gemm_nt<OT, C, D, D, 1, DN, kWaves, LDO, LDO>(WS, sW, sSt);
    gemm_nt<OT, C, D, D, 1, DN, kWaves, LDO, LDO>(O, sQ, sSt);
    lds_barrier();  // sb, se visible
    {
#pragma unroll
      for (int q = 0; q < TD::B::PER; ++q)
#pragma unroll
        for (int y = 0; y < DN; ++y) U.a[q][0][y] -= WS.a[q][0][y];
      U.each4([&](int i0, int v, f32x4& x) {
        *reinterpret_cast<o4*>(sDt + v * LCO + i0) = o4{(OT)x[0], (OT)x[1], (OT)x[2], (OT)x[3]};
        *reinterpret_cast<o4*>(sDet + v * LCO + i0) =
            o4{(OT)(x[0] * se[i0]), (OT)(x[1] * se[i0 + 1]), (OT)(x[2] * se[i0 + 2]), (OT)(x[3] * se[i0 + 3])};
      });
      O.each([&](int i, int v, float& x) { x *= sb[i]; });
    }
    lds_barrier();
    lds_to_global_t<D, C, LCO, NT>((OT*)p.sv_Dl + ch * C * D, sDt);  // Delta, row-major
    gemm_nt<OT, C, D, C, 1, DN, kWaves, LCO, LCO>(O, sM, sDt);
    {
      TI* o = (TI*)p.o + (int64_t)ci.t0 * p.o_rs + h * D;
      const int len = ci.len;
      const float sc = p.scale;
      O.each([&](int i, int v, float& x) {
        if (i < len) o[(int64_t)i * p.o_rs + v] = (TI)(sc * x);
      });
    }
    {
      const float bn = sb[C - 1];
      S.each([&](int, int, float& x) { x *= bn; });
      gemm_nt<OT, D, D, C, SM, SM, kWaves, LCO, LCO>(S, sKt, sDet);
    }
    lds_barrier();
    state_to_lds();
    if (c + 1 < c1) commit();
    lds_barrier();
  }
  if (p.ST) {
    float* st = p.ST + nh * D * D;
    S.each([&](int d, int v, float& x) { st[d * D + v] = x; });
  }
}

template <typename TI, int C, int D>
static hipError_t fwd_seq(const Prob& p, hipStream_t s) {
  traced("k_table", s, [&] { k_table<C><<<1, NTHREADS, 0, s>>>(p); });
  if (p.nc_max > 0) traced("k_prep", s, [&] { k_prep<TI, C, D><<<dim3(p.nc_max, p.Hk), kPrepThreads, 0, s>>>(p); });
  if (p.N > 0) traced("k_sweep", s, [&] { k_sweep<TI, C, D><<<dim3(p.N, p.Hv), kThreads, 0, s>>>(p); });
  return hipGetLastError();
}

template <typename TI, int C>
static hipError_t fwd_d(const Prob& p, hipStream_t s) {
  switch (p.D) {
    case 16: return fwd_seq<TI, C, 16>(p, s);
    case 32: return fwd_seq<TI, C, 32>(p, s);
    case 64: return fwd_seq<TI, C, 64>(p, s);
    case 128:
      if constexpr (sizeof(TI) == 4 && C == 64)
        return hipErrorInvalidValue;  // rejected on the host (LDS)
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
