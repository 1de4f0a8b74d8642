// gdn_decode.hip -- one step of the gated delta rule per sequence (token-by-token decode).
//
// Per row n (one token of one sequence) and value head h, with q and k from key head
// h / r and the state S (Dk x Dv, key-major) of the row's slot updated in place
// (lattice-inference 0.6.0, docs.rs source of src/attention/gdn_backward.rs, module doc
// "Forward recap"; the pages' shipping inference path, gated_delta_net_step_fused, steps
// the same recurrence one token at a time):
//   kv = S^T k,  delta = beta (v - g kv),  S' = g S + k delta^T,  o = scale S'^T q
// (with q and k first L2-normalised per head row when the problem asks for it).
// The kernel reads S once: S'^T q = g S^T q + delta (k . q), so S^T k and S^T q come from
// the same pass over S, and S' is written from the registers that hold S. Per row and
// head it moves 2 D^2 float32 of state and O(D) else: it is bound by HBM, and it is plain
// VALU work (two matrix-vector products and a rank-one update; no MFMA shape).
#include "gdn_common.h"

namespace gdn {

// Thread layout for one (row, head): each thread owns 4 adjacent state columns of RPG
// rows d = rg + RG i (i < RPG), so that the threads of a wave read whole, consecutive rows
// of S (D = 128: 32 threads per 512-byte row, a wave covers two rows).
template <int D> struct DecCfg {
  static constexpr int NT = D * D / 4 >= 256 ? 256 : D * D / 4;  // threads per workgroup
  static constexpr int CPR = D / 4;                             // threads per row
  static constexpr int RG = NT / CPR;                           // row groups
  static constexpr int RPG = D / RG;                            // rows per thread
  static_assert(RG * RPG == D && NT % 64 == 0, "layout covers the state");
};

template <typename TI> __device__ __forceinline__ float to_f(TI x) { return (float)x; }

// Grid N * Hv, value head fastest (the heads of one row read the same q, k, v row).
template <typename TI, int D>
__global__ __launch_bounds__(DecCfg<D>::NT) void k_decode(DecArgs a) {
  using CF = DecCfg<D>;
  constexpr int NT = CF::NT, CPR = CF::CPR, RG = CF::RG, RPG = CF::RPG;
  __shared__ float sk[D], sq[D];
  __shared__ __align__(16) float part[2][RG][D];  // per row group: partial S^T k, S^T q
  __shared__ float skq, srk, srq;  // k . q (of the normalised rows when a.l2), the factors of k and q

  const int n = blockIdx.x / a.Hv, h = blockIdx.x - n * a.Hv;
  const int slot = a.idx ? a.idx[n] : n;
  if (slot < 0 || slot >= a.n_slots) return;  // the row is skipped
  const int kh = h / a.r, t = threadIdx.x;
  const int c4 = (t % CPR) * 4, rg = t / CPR;

  const TI* qr = (const TI*)a.q + (int64_t)n * a.q_rs + kh * D;
  const TI* kr = (const TI*)a.k + (int64_t)n * a.k_rs + kh * D;
  for (int d = t; d < D; d += NT) {
    sk[d] = to_f(kr[d]);
    sq[d] = to_f(qr[d]);
  }
  float* S = a.state + ((int64_t)slot * a.Hv + h) * D * D;
  // The state is read once and written once per call: both through non-temporal accesses
  // (streamed past the caches' normal allocation; 5% more bandwidth than plain ones, and
  // either one alone is slower).
  f32x4 s[RPG];
#pragma unroll
  for (int i = 0; i < RPG; ++i) s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (rg + RG * i) * D + c4));
  float gg = a.g[(int64_t)n * a.Hv + h], be = a.beta[(int64_t)n * a.Hv + h];
  if (a.a_log) {  // the gate chain from alpha and beta_raw
    gg = exp2f(chain_log2g(gg, a.a_log[h], a.dt_bias[h]));
    be = chain_beta(be);
  }
  const TI* vr = (const TI*)a.v + (int64_t)n * a.v_rs + h * D + c4;
  const f32x4 vv = {to_f(vr[0]), to_f(vr[1]), to_f(vr[2]), to_f(vr[3])};
  __syncthreads();  // k and q rows in LDS

  f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPG; ++i) {
    const int d = rg + RG * i;
    pk += s[i] * sk[d];
    pq += s[i] * sq[d];
  }
  *reinterpret_cast<f32x4*>(&part[0][rg][c4]) = pk;
  *reinterpret_cast<f32x4*>(&part[1][rg][c4]) = pq;
  if (t < 64) {  // k . q, and the L2 factors of k and q when the rows are normalised here
    float x = 0.f, xk = 0.f, xq = 0.f;
    for (int d = t; d < D; d += 64) {
      x += sk[d] * sq[d];
      xk += sk[d] * sk[d];
      xq += sq[d] * sq[d];
    }
    x = wave_sum(x);
    const float rk = a.l2 ? 1.f / sqrtf(wave_sum(xk) + 1e-6f) : 1.f;
    const float rq = a.l2 ? 1.f / sqrtf(wave_sum(xq) + 1e-6f) : 1.f;
    if (t == 0) {
      skq = x * rk * rq;
      srk = rk;
      srq = rq;
    }
  }
  __syncthreads();  // partial sums complete

  // column sums over the row groups in a fixed order (every thread, its own 4 columns)
  f32x4 kv = {0.f, 0.f, 0.f, 0.f}, qv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < RG; ++j) {
    kv += *reinterpret_cast<const f32x4*>(&part[0][j][c4]);
    qv += *reinterpret_cast<const f32x4*>(&part[1][j][c4]);
  }
  kv *= srk;  // S^T k_hat, S^T q_hat (the factors are 1 without normalisation)
  qv *= srq;
  const f32x4 delta = be * (vv - gg * kv);
  if (rg == 0) {  // o = scale (g S^T q + delta (k . q)) for this thread's 4 columns
    const f32x4 ov = a.scale * (gg * qv + delta * skq);
    TI* orow = (TI*)a.o + (int64_t)n * a.o_rs + h * D + c4;
#pragma unroll
    for (int e = 0; e < 4; ++e) orow[e] = (TI)ov[e];
  }
  // S' = g S + k_hat delta^T
  const float rk = srk;
#pragma unroll
  for (int i = 0; i < RPG; ++i) {
    const int d = rg + RG * i;
    __builtin_nontemporal_store(gg * s[i] + (sk[d] * rk) * delta, reinterpret_cast<f32x4*>(S + d * D + c4));
  }
}

template <typename TI>
static hipError_t decode_d(const DecArgs& a, hipStream_t s) {
  const int grid = a.N * a.Hv;
  switch (a.D) {
    case 16: traced("k_decode", s, [&] { k_decode<TI, 16><<<grid, DecCfg<16>::NT, 0, s>>>(a); }); break;
    case 32: traced("k_decode", s, [&] { k_decode<TI, 32><<<grid, DecCfg<32>::NT, 0, s>>>(a); }); break;
    case 64: traced("k_decode", s, [&] { k_decode<TI, 64><<<grid, DecCfg<64>::NT, 0, s>>>(a); }); break;
    case 128: traced("k_decode", s, [&] { k_decode<TI, 128><<<grid, DecCfg<128>::NT, 0, s>>>(a); }); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecArgs& a, int dtype, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  return dtype == 0 ? decode_d<float>(a, s) : decode_d<__bf16>(a, s);
}

}  // namespace gdn
