// gdn_tile.h -- workgroup-level matrix tiles on CDNA4 (gfx950) MFMA, operands in LDS.
//
// A workgroup is NW = 4 waves of 64 lanes. An M x N output is cut into 16 x 16
// tiles; wave w owns tiles w, w + NW, w + 2 NW, ... (row-major tile order) and keeps
// one f32x4 accumulator per owned tile across calls, so products can be summed over
// several operand pairs before the epilogue. Operands are float matrices in LDS read
// through views with compile-time strides (Row<LD>: element (a, b) at a * LD + b;
// Col<LD>: the transpose), so fragment reads of contiguous runs become vector reads.
//
// MFMA lane layouts used (16 x 16 output, lane l, element e):
//   A (16 x KS): lane l holds A[l % 16][(l / 16) * KE + e], e < KE
//   B (KS x 16): lane l holds B[(l / 16) * KE + e][l % 16]
//   D (16 x 16): lane l holds D[(l / 16) * 4 + e][l % 16], e < 4
// KS = 4, KE = 1 for v_mfma_f32_16x16x4_f32 (float32 operands) and KS = 16, KE = 4
// for v_mfma_f32_16x16x16_bf16 (bfloat16 operands, float32 accumulation).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int WAVE = 64;
constexpr int NW = 4;
constexpr int NTHREADS = NW * WAVE;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / WAVE; }

// Element (a, b) at p[a * LD + b] (Row) or p[b * LD + a] (Col, the transpose).
template <int LD> struct Row {
  const float* p;
  __device__ __forceinline__ float operator()(int a, int b) const { return p[a * LD + b]; }
  // four consecutive b: one 16-byte read when (a * LD + b) % 4 == 0
  __device__ __forceinline__ f32x4 run4(int a, int b) const {
    return *reinterpret_cast<const f32x4*>(p + a * LD + b);
  }
};
template <int LD> struct Col {
  const float* p;
  __device__ __forceinline__ float operator()(int a, int b) const { return p[b * LD + a]; }
  __device__ __forceinline__ f32x4 run4(int a, int b) const {
    return f32x4{p[b * LD + a], p[(b + 1) * LD + a], p[(b + 2) * LD + a], p[(b + 3) * LD + a]};
  }
};
template <int LD> __device__ __forceinline__ Row<LD> rows(const float* p) { return Row<LD>{p}; }
template <int LD> __device__ __forceinline__ Col<LD> cols(const float* p) { return Col<LD>{p}; }

// Arithmetic precision of the MFMA operands.
enum class Prec { F32, BF16 };

template <Prec P> struct Mma;

template <> struct Mma<Prec::F32> {
  static constexpr int KS = 4;
  template <class VA, class VB>
  __device__ __forceinline__ static f32x4 step(f32x4 acc, const VA& A, const VB& B, int i0, int j0, int k0) {
    const int l = lane_id();
    const float a = A(i0 + (l & 15), k0 + (l >> 4));
    const float b = B(k0 + (l >> 4), j0 + (l & 15));
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
  }
};

// B(k, j) for four consecutive k is A-style run4 of the transposed view.
template <int LD> __device__ __forceinline__ f32x4 krun4(const Row<LD>& B, int k, int j) {
  return f32x4{B(k, j), B(k + 1, j), B(k + 2, j), B(k + 3, j)};
}
template <int LD> __device__ __forceinline__ f32x4 krun4(const Col<LD>& B, int k, int j) {
  return *reinterpret_cast<const f32x4*>(B.p + j * LD + k);
}

template <> struct Mma<Prec::BF16> {
  static constexpr int KS = 16;
  template <class VA, class VB>
  __device__ __forceinline__ static f32x4 step(f32x4 acc, const VA& A, const VB& B, int i0, int j0, int k0) {
    const int l = lane_id();
    const int kb = k0 + (l >> 4) * 4;
    const f32x4 a = A.run4(i0 + (l & 15), kb);
    const f32x4 b = krun4(B, kb, j0 + (l & 15));
    bf16x4_t av, bv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      av[e] = (__bf16)a[e];
      bv[e] = (__bf16)b[e];
    }
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, acc, 0, 0, 0);
  }
};

template <int M, int N> struct Tiles {
  static_assert(M % 16 == 0 && N % 16 == 0, "tile dims");
  static constexpr int MT = M / 16, NT = N / 16, TOT = MT * NT;
  static constexpr int PER = (TOT + NW - 1) / NW;  // accumulators per wave
};

template <int M, int N> struct Acc {
  f32x4 a[Tiles<M, N>::PER];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int q = 0; q < Tiles<M, N>::PER; ++q) a[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

// acc += A(M x K) * B(K x N)
template <Prec P, int M, int N, int K, class VA, class VB>
__device__ __forceinline__ void mma(Acc<M, N>& acc, const VA A, const VB B) {
  using TL = Tiles<M, N>;
  static_assert(K % Mma<P>::KS == 0, "K must be a multiple of the MFMA depth");
#pragma unroll
  for (int q = 0; q < TL::PER; ++q) {
    const int t = wave_id() + q * NW;  // uniform across the wave
    if (t < TL::TOT) {
      const int i0 = (t / TL::NT) * 16, j0 = (t % TL::NT) * 16;
      f32x4 c = acc.a[q];
#pragma unroll
      for (int k0 = 0; k0 < K; k0 += Mma<P>::KS) c = Mma<P>::step(c, A, B, i0, j0, k0);
      acc.a[q] = c;
    }
  }
}

// f(i, j, value) for every element the calling lane owns.
template <int M, int N, class F>
__device__ __forceinline__ void for_each(const Acc<M, N>& acc, F&& f) {
  using TL = Tiles<M, N>;
  const int l = lane_id();
#pragma unroll
  for (int q = 0; q < TL::PER; ++q) {
    const int t = wave_id() + q * NW;
    if (t < TL::TOT) {
      const int i0 = (t / TL::NT) * 16 + (l >> 4) * 4, j = (t % TL::NT) * 16 + (l & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) f(i0 + e, j, acc.a[q][e]);
    }
  }
}

template <int M, int N, class F>
__device__ __forceinline__ void for_each2(const Acc<M, N>& x, const Acc<M, N>& y, F&& f) {
  using TL = Tiles<M, N>;
  const int l = lane_id();
#pragma unroll
  for (int q = 0; q < TL::PER; ++q) {
    const int t = wave_id() + q * NW;
    if (t < TL::TOT) {
      const int i0 = (t / TL::NT) * 16 + (l >> 4) * 4, j = (t % TL::NT) * 16 + (l & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) f(i0 + e, j, x.a[q][e], y.a[q][e]);
    }
  }
}

// ---------------------------------------------------------------- global <-> LDS
// 16-byte vectors of the storage types.
template <typename T> struct Vec;
template <> struct Vec<float> {
  static constexpr int N = 4;
  typedef float type __attribute__((ext_vector_type(4)));
};
template <> struct Vec<__bf16> {
  static constexpr int N = 8;
  typedef __bf16 type __attribute__((ext_vector_type(8)));
};

template <typename T> __device__ __forceinline__ float to_f(T x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x) { return (T)x; }

// LDS[r][c] (row stride LD floats) = src[r * rs + c] * (s ? s[r] : 1) for r < nrows,
// zero for nrows <= r < R. Every thread issues all of its 16-byte loads before the
// first LDS store, so the loads are in flight together. Requires src and rs * sizeof(T)
// 16-byte aligned, Cn a multiple of the vector width and LD a multiple of 4.
template <int R, int Cn, int LD, typename T>
__device__ __forceinline__ void load_tile(float* dst, const T* __restrict__ src, int64_t rs, int nrows,
                                          const float* s = nullptr) {
  using V = Vec<T>;
  constexpr int VPR = Cn / V::N;  // vectors per row
  constexpr int NV = R * VPR;
  constexpr int PER = (NV + NTHREADS - 1) / NTHREADS;
  static_assert(Cn % V::N == 0 && LD % 4 == 0, "tile shape");
  typename V::type buf[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int v = threadIdx.x + u * NTHREADS;
    const int r = v / VPR, c = (v % VPR) * V::N;
    if (v < NV && r < nrows)
      buf[u] = *reinterpret_cast<const typename V::type*>(src + (int64_t)r * rs + c);
    else
      buf[u] = typename V::type{};
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int v = threadIdx.x + u * NTHREADS;
    if (v < NV) {
      const int r = v / VPR, c = (v % VPR) * V::N;
      const float sc = s ? s[r] : 1.f;
#pragma unroll
      for (int e = 0; e < V::N; e += 4) {
        f32x4 x{to_f(buf[u][e]), to_f(buf[u][e + 1]), to_f(buf[u][e + 2]), to_f(buf[u][e + 3])};
        *reinterpret_cast<f32x4*>(dst + r * LD + c + e) = x * sc;
      }
    }
  }
}

// dst[r * rs + c] = LDS[r][c] for r < nrows (16-byte stores).
template <int R, int Cn, int LD, typename T>
__device__ __forceinline__ void store_tile(T* __restrict__ dst, int64_t rs, const float* src, int nrows) {
  using V = Vec<T>;
  constexpr int VPR = Cn / V::N;
  constexpr int NV = R * VPR;
  static_assert(Cn % V::N == 0 && LD % 4 == 0, "tile shape");
  for (int v = threadIdx.x; v < NV; v += NTHREADS) {
    const int r = v / VPR, c = (v % VPR) * V::N;
    if (r < nrows) {
      typename V::type x;
#pragma unroll
      for (int e = 0; e < V::N; ++e) x[e] = from_f<T>(src[r * LD + c + e]);
      *reinterpret_cast<typename V::type*>(dst + (int64_t)r * rs + c) = x;
    }
  }
}

}  // namespace gdn
