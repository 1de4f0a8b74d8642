// gdn_fwd.hip -- chunked forward of the gated delta rule on gfx950.
//
// Launch sequence: chunk table -> k_wy (per chunk x value head: gamma, T, W, U)
// -> k_fwd_state (per sequence x value head x column block: the chunk-serial state
// pass; saves every chunk's start state, turns U into Delta) -> k_fwd_out (per chunk
// x value head: O = scale (diag(b) Q S0 + (Gamma o Q K^T) Delta)).
// Columns of the state never mix (delta_j depends only on column j of S), which is
// what lets the state pass split over blocks of BV value columns.
#include "gdn_common.h"

namespace gdn {

template <int D> struct FwdCfg { static constexpr int BV = D < 32 ? D : 32; };

// Grid (N, Hv, D / BV). Chunk-serial over one sequence.
template <typename TI, int C, int D, int BV>
__global__ __launch_bounds__(NTHREADS) void k_fwd_state(Prob p) {
  constexpr Prec P = PrecOf<TI>::value;
  constexpr int LD = D + 4, LB = BV + 4;
  __shared__ __align__(16) float sS[D * LB];
  __shared__ __align__(16) float sX[C * LD];  // W, then diag(exp(gamma_n - gamma)) K
  __shared__ __align__(16) float sDl[C * LB];
  __shared__ __align__(16) float sg[C], se[C];
  const int n = blockIdx.x, h = blockIdx.y, j0 = blockIdx.z * BV;
  const int kh = h / p.r;
  const size_t nh = (size_t)n * p.Hv + h;
  if (p.S0)
    load_tile<D, BV, LB>(sS, p.S0 + nh * D * D + j0, D, D);
  else
    for (int idx = threadIdx.x; idx < D * BV; idx += NTHREADS) sS[(idx / BV) * LB + idx % BV] = 0.f;
  const int c0 = p.seq_chunk[n], c1 = p.seq_chunk[n + 1];
  __syncthreads();
  for (int c = c0; c < c1; ++c) {
    const ChunkInfo ci = p.chunks[c];
    const size_t ch = ch_idx(p, c, h);
    store_tile<D, BV, LB>(p.states + ch * D * D + j0, D, sS, D);
    load_tile<C, D, LD>(sX, p.W + ch * C * D, D, C);
    load_tile<C, BV, LB>(sDl, p.U + ch * C * D + j0, D, C);
    for (int i = threadIdx.x; i < C; i += NTHREADS) sg[i] = p.gam[ch * C + i];
    __syncthreads();
    for (int i = threadIdx.x; i < C; i += NTHREADS) se[i] = expf(sg[C - 1] - sg[i]);
    {
      Acc<C, BV> a;
      a.zero();
      mma<P, C, BV, D>(a, rows<LD>(sX), rows<LB>(sS));
      for_each(a, [&](int i, int j, float x) {
        const float d = sDl[i * LB + j] - x;
        sDl[i * LB + j] = d;
        p.U[ch * C * D + (size_t)i * D + j0 + j] = d;
      });
    }
    __syncthreads();
    load_tile<C, D, LD>(sX, (const TI*)p.k + (int64_t)ci.t0 * p.k_rs + kh * D, p.k_rs, ci.len, se);
    __syncthreads();
    {
      Acc<D, BV> a;
      a.zero();
      mma<P, D, BV, C>(a, cols<LD>(sX), rows<LB>(sDl));
      const float bn = expf(sg[C - 1]);
      for_each(a, [&](int i, int j, float x) { sS[i * LB + j] = bn * sS[i * LB + j] + x; });
    }
    __syncthreads();
  }
  if (p.ST) store_tile<D, BV, LB>(p.ST + nh * D * D + j0, D, sS, D);
}

// Grid (nc_max, Hv).
template <typename TI, int C, int D, int BV>
__global__ __launch_bounds__(NTHREADS) void k_fwd_out(Prob p) {
  constexpr Prec P = PrecOf<TI>::value;
  constexpr int LD = D + 4, LB = BV + 4, LC = C + 4;
  __shared__ __align__(16) float sQ[C * LD];  // Q, then diag(b) Q
  __shared__ __align__(16) float sK[C * LD];
  __shared__ __align__(16) float sM[C * LC];
  __shared__ __align__(16) float sS[D * LB];
  __shared__ __align__(16) float sDl[C * LB];
  __shared__ __align__(16) float sg[C];
  const int c = blockIdx.x, h = blockIdx.y;
  const ChunkInfo ci = p.chunks[c];
  if (ci.seq < 0) return;
  const int kh = h / p.r, n = ci.len;
  const size_t ch = ch_idx(p, c, h);
  load_tile<C, D, LD>(sQ, (const TI*)p.q + (int64_t)ci.t0 * p.q_rs + kh * D, p.q_rs, n);
  load_tile<C, D, LD>(sK, (const TI*)p.k + (int64_t)ci.t0 * p.k_rs + kh * D, p.k_rs, n);
  for (int i = threadIdx.x; i < C; i += NTHREADS) sg[i] = p.gam[ch * C + i];
  __syncthreads();
  {
    Acc<C, C> m;
    m.zero();
    mma<P, C, C, D>(m, rows<LD>(sQ), cols<LD>(sK));
    for_each(m, [&](int i, int j, float x) { sM[i * LC + j] = i >= j ? x * expf(sg[i] - sg[j]) : 0.f; });
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < C * D; idx += NTHREADS) {
    const int i = idx / D, j = idx % D;
    sQ[i * LD + j] *= expf(sg[i]);
  }
  TI* O = (TI*)p.o + (int64_t)ci.t0 * p.o_rs + h * D;
  for (int j0 = 0; j0 < D; j0 += BV) {
    load_tile<D, BV, LB>(sS, p.states + ch * D * D + j0, D, D);
    load_tile<C, BV, LB>(sDl, p.U + ch * C * D + j0, D, C);
    __syncthreads();
    Acc<C, BV> a;
    a.zero();
    mma<P, C, BV, D>(a, rows<LD>(sQ), rows<LB>(sS));
    mma<P, C, BV, C>(a, rows<LC>(sM), rows<LB>(sDl));
    for_each(a, [&](int i, int j, float x) {
      if (i < n) O[(int64_t)i * p.o_rs + j0 + j] = from_f<TI>(p.scale * x);
    });
    __syncthreads();
  }
}

template <typename TI, int C, int D>
static hipError_t fwd_seq(const Prob& p, hipStream_t s) {
  constexpr int BV = FwdCfg<D>::BV;
  traced("k_table", s, [&] { k_table<C><<<1, NTHREADS, 0, s>>>(p); });
  if (p.nc_max > 0) traced("k_wy", s, [&] { k_wy<TI, C, D><<<dim3(p.nc_max, p.Hv), NTHREADS, 0, s>>>(p); });
  if (p.N > 0) traced("k_fwd_state", s, [&] { k_fwd_state<TI, C, D, BV><<<dim3(p.N, p.Hv, D / BV), NTHREADS, 0, s>>>(p); });
  if (p.nc_max > 0) traced("k_fwd_out", s, [&] { k_fwd_out<TI, C, D, BV><<<dim3(p.nc_max, p.Hv), NTHREADS, 0, s>>>(p); });
  return hipGetLastError();
}

template <typename TI, int C>
static hipError_t fwd_d(const Prob& p, hipStream_t s) {
  switch (p.D) {
    case 16: return fwd_seq<TI, C, 16>(p, s);
    case 32: return fwd_seq<TI, C, 32>(p, s);
    case 64: return fwd_seq<TI, C, 64>(p, s);
    case 128: return fwd_seq<TI, C, 128>(p, s);
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
