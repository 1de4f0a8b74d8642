// gdn_common.h -- chunk table and the WY/UT preparation shared by forward and backward.
//
// Chunk form of the gated delta rule (derived from the per-token recurrence of the
// lattice-inference gdn_backward.rs page, "Forward recap"; the pages print no chunk
// algebra). Within a chunk of n <= C tokens starting from state S0:
//   gamma_r = sum_{s<=r} log g_s,  b = exp(gamma),  Gamma_rs = exp(gamma_r - gamma_s) [r >= s]
//   L = strictly_lower(diag(beta) (Gamma o K K^T)),  T = (I + L)^-1
//   W = T diag(beta b) K,  U = T diag(beta) V,  Delta = U - W S0   (Delta_r = delta_r)
//   O = scale (diag(b) Q S0 + (Gamma o Q K^T) Delta)
//   S_end = b_n S0 + K^T diag(exp(gamma_n - gamma)) Delta
// Rows past the end of a partial chunk carry k = q = v = beta = 0 and log g = 0, which
// leaves every valid row unchanged.
#pragma once
#include "gdn_internal.h"
#include "gdn_tile.h"

namespace gdn {

// Operand precision of the MFMA products for each storage type.
template <typename TI> struct PrecOf { static constexpr Prec value = Prec::F32; };
template <> struct PrecOf<__bf16> { static constexpr Prec value = Prec::BF16; };

__device__ __forceinline__ size_t ch_idx(const Prob& p, int c, int h) { return (size_t)c * p.Hv + h; }

// Sequence n occupies rows [a, b). Device-side cu_seqlens are clamped into
// [0, T_total] so that a malformed table can never address outside the buffers.
__device__ __forceinline__ void seq_bounds(const Prob& p, int n, int64_t& a, int64_t& b) {
  if (p.cu) {
    int64_t x = p.cu[n], y = p.cu[n + 1];
    x = x < 0 ? 0 : (x > p.T_total ? p.T_total : x);
    y = y < x ? x : (y > p.T_total ? p.T_total : y);
    a = x;
    b = y;
  } else {
    a = (int64_t)n * p.T;
    b = a + p.T;
  }
}

// One workgroup: chunk table and per-sequence first-chunk offsets.
template <int C>
__global__ __launch_bounds__(NTHREADS) void k_table(Prob p) {
  if (threadIdx.x == 0) {
    int64_t off = 0;
    for (int n = 0; n < p.N; ++n) {
      int64_t a, b;
      seq_bounds(p, n, a, b);
      p.seq_chunk[n] = (int)(off < p.nc_max ? off : p.nc_max);
      off += (b - a + C - 1) / C;
    }
    p.seq_chunk[p.N] = (int)(off < p.nc_max ? off : p.nc_max);
  }
  __syncthreads();
  for (int n = threadIdx.x; n < p.N; n += NTHREADS) {
    int64_t a, b;
    seq_bounds(p, n, a, b);
    const int c0 = p.seq_chunk[n], c1 = p.seq_chunk[n + 1];
    for (int c = c0; c < c1; ++c) {
      const int64_t t = a + (int64_t)(c - c0) * C;
      const int64_t len = b - t < C ? b - t : C;
      p.chunks[c] = ChunkInfo{n, (int)t, (int)len, 0};
    }
  }
  for (int c = p.seq_chunk[p.N] + threadIdx.x; c < p.nc_max; c += NTHREADS) p.chunks[c] = ChunkInfo{-1, 0, 0, 0};
}

// T = (I + L)^-1 for strictly lower triangular L (LDS, row stride LC). T must hold
// the identity on entry. Row i: T[i][j] = -sum_{k=j}^{i-1} L[i][k] T[k][j] (j < i),
// four lanes per column, summed in a fixed order.
template <int C>
__device__ __forceinline__ void solve_unit_lower(const float* L, float* T, int LC) {
  const int j = threadIdx.x >> 2, part = threadIdx.x & 3;
  for (int i = 1; i < C; ++i) {
    float s = 0.f;
    if (j < i)
      for (int k = j + part; k < i; k += 4) s += L[i * LC + k] * T[k * LC + j];
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if (j < i && part == 0) T[i * LC + j] = -s;
    __syncthreads();
  }
}

// Grid (nc_max, Hv). Writes gamma, T, W and U of one (chunk, value head).
template <typename TI, int C, int D>
__global__ __launch_bounds__(NTHREADS) void k_wy(Prob p) {
  constexpr Prec P = PrecOf<TI>::value;
  constexpr int LD = D + 4, LC = C + 4;
  __shared__ __align__(16) float sK[C * LD];  // K, then V
  __shared__ __align__(16) float sA[C * LC];  // L, then T diag(beta b), then T diag(beta)
  __shared__ __align__(16) float sT[C * LC];
  __shared__ __align__(16) float sg[C], sb[C], sbeta[C];
  const int c = blockIdx.x, h = blockIdx.y;
  const ChunkInfo ci = p.chunks[c];
  if (ci.seq < 0) return;
  const int kh = h / p.r, n = ci.len;
  const size_t ch = ch_idx(p, c, h);

  load_tile<C, D, LD>(sK, (const TI*)p.k + (int64_t)ci.t0 * p.k_rs + kh * D, p.k_rs, n);
  for (int i = threadIdx.x; i < C; i += NTHREADS) {
    const bool ok = i < n;
    sbeta[i] = ok ? p.beta[(int64_t)(ci.t0 + i) * p.Hv + h] : 0.f;
    sg[i] = ok ? logf(p.g[(int64_t)(ci.t0 + i) * p.Hv + h]) : 0.f;
  }
  for (int idx = threadIdx.x; idx < C * C; idx += NTHREADS) {
    const int i = idx / C, j = idx % C;
    sT[i * LC + j] = i == j ? 1.f : 0.f;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int i = 0; i < C; ++i) {
      s += sg[i];
      sg[i] = s;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < C; i += NTHREADS) {
    sb[i] = expf(sg[i]);
    p.gam[ch * C + i] = sg[i];
  }
  {
    Acc<C, C> a;
    a.zero();
    mma<P, C, C, D>(a, rows<LD>(sK), cols<LD>(sK));
    for_each(a, [&](int i, int j, float x) {
      sA[i * LC + j] = i > j ? sbeta[i] * expf(sg[i] - sg[j]) * x : 0.f;
    });
  }
  __syncthreads();
  solve_unit_lower<C>(sA, sT, LC);
  for (int idx = threadIdx.x; idx < C * C; idx += NTHREADS) {
    const int i = idx / C, j = idx % C;
    const float t = sT[i * LC + j];
    p.Tm[ch * C * C + idx] = t;
    sA[i * LC + j] = t * sbeta[j] * sb[j];
  }
  __syncthreads();
  {
    Acc<C, D> w;
    w.zero();
    mma<P, C, D, C>(w, rows<LC>(sA), rows<LD>(sK));
    for_each(w, [&](int i, int j, float x) { p.W[ch * C * D + i * D + j] = x; });
  }
  __syncthreads();
  load_tile<C, D, LD>(sK, (const TI*)p.v + (int64_t)ci.t0 * p.v_rs + h * D, p.v_rs, n);
  for (int idx = threadIdx.x; idx < C * C; idx += NTHREADS) {
    const int i = idx / C, j = idx % C;
    sA[i * LC + j] = sT[i * LC + j] * sbeta[j];
  }
  __syncthreads();
  {
    Acc<C, D> u;
    u.zero();
    mma<P, C, D, C>(u, rows<LC>(sA), rows<LD>(sK));
    for_each(u, [&](int i, int j, float x) { p.U[ch * C * D + i * D + j] = x; });
  }
}

}  // namespace gdn
