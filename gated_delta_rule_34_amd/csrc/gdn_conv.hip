// gdn_conv.hip -- causal depthwise conv1d + SiLU over the packed q/k/v projection, forward
// and input gradient, on gfx950.
//
// Per channel ch of a row (the packed projection row of a token) and kernel size K, with
// the K - 1 previous rows of the same sequence as the conv buffer (zeros before the
// sequence's first row), as the lattice-inference gdn_backward.rs page computes it
// (gdn_forward_save's conv1d_silu_fwd, and step 5 of gdn_backward, "Backward through
// conv1d + SiLU"):
//   pre[t] = sum_{j < K} w[ch][j] x[t - (K - 1) + j],  y[t] = SiLU(pre[t]) = pre sigma(pre)
//   dpre[t] = dy[t] SiLU'(pre[t]),  SiLU'(z) = sigma(z) (1 + z (1 - sigma(z)))
//   dx[t] = sum_{lag < K} w[ch][K - 1 - lag] dpre[t + lag]   (t + lag in the same sequence)
// The pages keep the conv weights fixed (no weight gradient), and so does this file.
//
// Each thread owns 8 adjacent channels (one 16-byte bf16 piece of the row, two for
// float32) and a run of RUN consecutive rows, streaming along time with the window of
// the last K - 1 inputs (and, backward, the last K values of dpre) in registers: every
// input and output element crosses HBM once, up to the K - 1 halo rows at a run's ends.
// The threads of a wave cover 512 consecutive channels, so each row access is one
// contiguous 1 KB (bf16) piece. Plain VALU streaming work, bound by HBM.
#include "gdn_common.h"

namespace gdn {

constexpr int kConvThreads = 256;
constexpr int kConvRun = 32;  // rows per thread
constexpr int kConvPF = 1;    // rows loaded ahead of their use (kConvRun is a multiple)
static_assert(kConvRun % kConvPF == 0, "runs hold whole prefetch groups");

// Rows [lo, hi) of sequence l from the device table, clamped so that 0 <= lo <= hi <= rows:
// a malformed table (a negative or decreasing entry) then gives wrong sequence boundaries but
// never a row outside the caller's buffers (every row a kernel touches is >= lo or >= its
// run's first row, and < rows).
__device__ __forceinline__ void conv_clamp(const ConvArgs& a, int l, int64_t& lo, int64_t& hi) {
  int64_t x = a.cu[l], y = a.cu[l + 1];
  x = x < 0 ? 0 : (x > a.rows ? a.rows : x);
  y = y < x ? x : (y > a.rows ? a.rows : y);
  lo = x;
  hi = y;
}

// Rows [lo, hi) of the sequence that holds row t.
__device__ __forceinline__ void conv_seq(const ConvArgs& a, int64_t t, int64_t& lo, int64_t& hi) {
  if (!a.cu) {
    lo = t / a.T * a.T;
    hi = lo + a.T;
    return;
  }
  int l = 0, r = a.N;  // largest n with cu[n] <= t (empty sequences skipped by the search)
  while (r - l > 1) {
    const int m = (l + r) >> 1;
    if (a.cu[m] <= t) l = m; else r = m;
  }
  conv_clamp(a, l, lo, hi);
  while (hi <= t && l + 1 < a.N) {  // equal offsets (empty sequences) before t's own
    ++l;
    conv_clamp(a, l, lo, hi);
  }
  // (hi <= t still means cu[N] < T_total, a caller error: the row is then treated as the
  // first of a sequence, and nothing outside cu[0 .. N] is read)
}

struct F8 {
  float v[8];
};

template <typename TI> __device__ __forceinline__ F8 ld8(const TI* p) {
  F8 r;
  if constexpr (sizeof(TI) == 2) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) r.v[i] = (float)x[i];
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.v[i] = a[i];
      r.v[4 + i] = b[i];
    }
  }
  return r;
}

template <typename TI> __device__ __forceinline__ void st8(TI* p, const F8& x) {
  if constexpr (sizeof(TI) == 2) {
    bf16x8 y;
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = (__bf16)x.v[i];
    *reinterpret_cast<bf16x8*>(p) = y;
  } else {
    *reinterpret_cast<f32x4*>(p) = f32x4{x.v[0], x.v[1], x.v[2], x.v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{x.v[4], x.v[5], x.v[6], x.v[7]};
  }
}

// One row piece as loaded (bf16 kept packed until its use, so that a prefetched row holds
// no wait for its data before the row is reached).
template <typename TI> struct Raw8 {
  f32x4 a, b;
};
template <> struct Raw8<__bf16> {
  bf16x8 a;
};

// Non-temporal loads: each row piece is read once (apart from the K - 1 halo rows), and the
// kernels measured 10-14% faster with them than with plain loads.
template <typename TI> __device__ __forceinline__ Raw8<TI> ldraw(const TI* p) {
  Raw8<TI> r;
  if constexpr (sizeof(TI) == 2) {
    typedef int32_t i4 __attribute__((ext_vector_type(4)));
    r.a = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const i4*>(p)));
  } else {
    r.a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    r.b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
  }
  return r;
}

template <typename TI> __device__ __forceinline__ F8 cvt(const Raw8<TI>& x) {
  F8 r;
  if constexpr (sizeof(TI) == 2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) r.v[i] = (float)x.a[i];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.v[i] = x.a[i];
      r.v[4 + i] = x.b[i];
    }
  }
  return r;
}

// The reciprocal is the hardware's v_rcp_f32 (about 1 ulp; 0 for an infinite argument,
// NaN for NaN): an IEEE division here took about ten VALU instructions per element
// (measured: the backward 3% faster, the forward faster in every run).
__device__ __forceinline__ float sigmoid(float z) { return __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

// Grid (rows / kConvRun, channel groups / kConvThreads).
template <typename TI, int K>
__global__ __launch_bounds__(kConvThreads) void k_conv_fwd(ConvArgs a) {
  const int cg = blockIdx.y * kConvThreads + threadIdx.x;
  if (cg * 8 >= a.ch) return;
  const int c0 = cg * 8;
  const int64_t t0 = (int64_t)blockIdx.x * kConvRun;
  const int64_t t1 = t0 + kConvRun < a.rows ? t0 + kConvRun : a.rows;
  float w[K][8];
#pragma unroll
  for (int j = 0; j < K; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) w[j][i] = a.w[(int64_t)(c0 + i) * K + j];
  int64_t lo, hi;
  conv_seq(a, t0, lo, hi);
  const TI* __restrict__ x = (const TI*)a.x + c0;
  TI* __restrict__ y = (TI*)a.y + c0;
  F8 win[K > 1 ? K - 1 : 1];  // x[t - (K - 1) + j], j < K - 1 (zeros before the sequence)
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
    const int64_t s = t0 - (K - 1) + j;
    if (s >= lo) {
      win[j] = ld8(x + s * a.x_rs);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) win[j].v[i] = 0.f;
    }
  }
  // Rows t + 1 .. t + kConvPF are in flight while row t is computed: buf[u] holds the row
  // base + u of the current group, and its slot is refilled with the row kConvPF ahead as
  // soon as it is converted (the loads carry no wait until their row is reached).
  Raw8<TI> buf[kConvPF];
#pragma unroll
  for (int u = 0; u < kConvPF; ++u)
    if (t0 + u < t1) buf[u] = ldraw(x + (t0 + u) * a.x_rs);
  // Unrolled by the window length, so that the window's K - 1 rows rename registers
  // instead of moving down one slot per row (forward 1-5% faster; the same unrolling of the
  // backward was 2% slower)
#pragma unroll (K > 1 ? K - 1 : 1)
  for (int64_t base = t0; base < t1; base += kConvPF) {
#pragma unroll
    for (int u = 0; u < kConvPF; ++u) {
      const int64_t t = base + u;
      if (t >= t1) break;
      const F8 xt = cvt<TI>(buf[u]);
      if (t + kConvPF < t1) buf[u] = ldraw(x + (t + kConvPF) * a.x_rs);
      if (t >= hi) {  // the next sequence starts at t: its buffer is empty
        conv_seq(a, t, lo, hi);
#pragma unroll
        for (int j = 0; j < K - 1; ++j)
#pragma unroll
          for (int i = 0; i < 8; ++i) win[j].v[i] = 0.f;
      }
      F8 out;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float z = w[K - 1][i] * xt.v[i];
#pragma unroll
        for (int j = 0; j < K - 1; ++j) z += w[j][i] * win[j].v[i];
        out.v[i] = z * sigmoid(z);
      }
      st8(y + t * a.y_rs, out);
#pragma unroll
      for (int j = 0; j + 1 < K - 1; ++j) win[j] = win[j + 1];
      if constexpr (K > 1) win[K - 2] = xt;
    }
  }
}

// Grid as the forward. Sweeps rows u = t0 .. t1 + K - 2: at row u it forms dpre[u] (from the
// input window and dy[u]) and adds w[j] dpre[u] into the pending sum of dx[u - (K - 1) + j]
// for every such row of u's own sequence; dx[u - (K - 1)] then has all its terms and is
// stored (rows of the run only). Scattering each dpre row at once keeps K - 1 pending row
// sums in registers instead of the last K rows of dpre with their sequence ends.
template <typename TI, int K>
__global__ __launch_bounds__(kConvThreads) void k_conv_bwd(ConvArgs a) {
  const int cg = blockIdx.y * kConvThreads + threadIdx.x;
  if (cg * 8 >= a.ch) return;
  const int c0 = cg * 8;
  const int64_t t0 = (int64_t)blockIdx.x * kConvRun;
  const int64_t t1 = t0 + kConvRun < a.rows ? t0 + kConvRun : a.rows;
  float w[K][8];
#pragma unroll
  for (int j = 0; j < K; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) w[j][i] = a.w[(int64_t)(c0 + i) * K + j];
  int64_t lo, hi;
  conv_seq(a, t0, lo, hi);
  const TI* __restrict__ x = (const TI*)a.x + c0;
  const TI* __restrict__ dy = (const TI*)a.dy + c0;
  TI* __restrict__ dx = (TI*)a.dx + c0;
  F8 win[K > 1 ? K - 1 : 1];
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
    const int64_t s = t0 - (K - 1) + j;
    if (s >= lo) {
      win[j] = ld8(x + s * a.x_rs);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) win[j].v[i] = 0.f;
    }
  }
  // acc[j]: the sum so far of dx[u - (K - 1) + j], j < K - 1 (rows before t0 are never stored)
  F8 acc[K > 1 ? K - 1 : 1];
#pragma unroll
  for (int j = 0; j < K - 1; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[j].v[i] = 0.f;
  const int64_t uend = t1 + K - 1 < a.rows ? t1 + K - 1 : a.rows;  // rows loaded: [t0, uend)
  // x and dy of rows u + 1 .. u + kConvPF are in flight while row u is computed (slots as in
  // the forward); the K - 1 rows past the run are loaded in the last group.
  Raw8<TI> bx[kConvPF], bg[kConvPF];
#pragma unroll
  for (int s = 0; s < kConvPF; ++s)
    if (t0 + s < uend) {
      bx[s] = ldraw(x + (t0 + s) * a.x_rs);
      bg[s] = ldraw(dy + (t0 + s) * a.dy_rs);
    }
  for (int64_t base = t0; base < t1 + K - 1; base += kConvPF) {
#pragma unroll
    for (int s = 0; s < kConvPF; ++s) {
      const int64_t u = base + s;
      if (u >= t1 + K - 1) break;
      F8 dp;  // dpre[u], zero past the last row
      if (u < uend) {
        const F8 xu = cvt<TI>(bx[s]);
        const F8 gu = cvt<TI>(bg[s]);
        if (u + kConvPF < uend) {
          bx[s] = ldraw(x + (u + kConvPF) * a.x_rs);
          bg[s] = ldraw(dy + (u + kConvPF) * a.dy_rs);
        }
        if (u >= hi) {
          conv_seq(a, u, lo, hi);
#pragma unroll
          for (int j = 0; j < K - 1; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) win[j].v[i] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float z = w[K - 1][i] * xu.v[i];
#pragma unroll
          for (int j = 0; j < K - 1; ++j) z += w[j][i] * win[j].v[i];
          const float sg = sigmoid(z);
          dp.v[i] = gu.v[i] * sg * (1.f + z * (1.f - sg));
        }
#pragma unroll
        for (int j = 0; j + 1 < K - 1; ++j) win[j] = win[j + 1];
        if constexpr (K > 1) win[K - 2] = xu;
        // rows u - (K - 1) + j of u's sequence take w[j] dpre[u]
#pragma unroll
        for (int j = 0; j < K - 1; ++j)
          if (u - (K - 1) + j >= lo)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[j].v[i] += w[j][i] * dp.v[i];
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) dp.v[i] = 0.f;
      }
      F8 done;  // dx[u - (K - 1)]: complete once dpre[u] is in
      if constexpr (K > 1) {
        done = acc[0];
#pragma unroll
        for (int j = 0; j + 1 < K - 1; ++j) acc[j] = acc[j + 1];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[K - 2].v[i] = w[K - 1][i] * dp.v[i];
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) done.v[i] = w[0][i] * dp.v[i];
      }
      const int64_t t = u - (K - 1);
      if (t >= t0) st8(dx + t * a.dx_rs, done);
    }
  }
}

template <typename TI, int K>
static hipError_t conv_k(const ConvArgs& a, bool backward, hipStream_t s) {
  const dim3 grid((unsigned)((a.rows + kConvRun - 1) / kConvRun), (unsigned)((a.ch / 8 + kConvThreads - 1) / kConvThreads));
  if (backward)
    traced("k_conv_bwd", s, [&] { k_conv_bwd<TI, K><<<grid, kConvThreads, 0, s>>>(a); });
  else
    traced("k_conv_fwd", s, [&] { k_conv_fwd<TI, K><<<grid, kConvThreads, 0, s>>>(a); });
  return hipGetLastError();
}

template <typename TI>
static hipError_t conv_t(const ConvArgs& a, bool backward, hipStream_t s) {
  switch (a.K) {
    case 1: return conv_k<TI, 1>(a, backward, s);
    case 2: return conv_k<TI, 2>(a, backward, s);
    case 3: return conv_k<TI, 3>(a, backward, s);
    case 4: return conv_k<TI, 4>(a, backward, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_conv(const ConvArgs& a, int dtype, bool backward, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  return dtype == 0 ? conv_t<float>(a, backward, s) : conv_t<__bf16>(a, backward, s);
}

}  // namespace gdn
