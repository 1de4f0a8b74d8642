// gdn_tile.h -- workgroup-level matrix tiles on CDNA4 (gfx950) MFMA, operands in LDS.
//
// A workgroup is NW = 4 waves of 64 lanes. An M x N output is cut into 16 x 16
// tiles; wave w owns tiles w, w + NW, w + 2 NW, ... (row-major tile order) and keeps
// one f32x4 accumulator per owned tile across calls, so products can be summed over
// several operand pairs before the epilogue. Operands are float views over LDS with
// arbitrary (row, column) strides, which gives transposes for free.
//
// MFMA lane layouts used (16 x 16 output, lane l, element e):
//   A (16 x KS): lane l holds A[l % 16][(l / 16) * KE + e], e < KE
//   B (KS x 16): lane l holds B[(l / 16) * KE + e][l % 16]
//   D (16 x 16): lane l holds D[(l / 16) * 4 + e][l % 16], e < 4
// with KS = 4, KE = 1 for v_mfma_f32_16x16x4_f32 and KS = 16, KE = 4 for
// v_mfma_f32_16x16x16_bf16.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr int NW = 4;
constexpr int NTHREADS = NW * WAVE;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / WAVE; }

// Element (a, b) of a strided LDS matrix is p[a * sa + b * sb].
struct View {
  const float* p;
  int sa, sb;
  __device__ __forceinline__ float operator()(int a, int b) const { return p[a * sa + b * sb]; }
};
__device__ __forceinline__ View rows(const float* p, int ld) { return View{p, ld, 1}; }
__device__ __forceinline__ View cols(const float* p, int ld) { return View{p, 1, ld}; }  // transpose

// Arithmetic precision of the MFMA operands.
enum class Prec { F32, BF16 };

template <Prec P> struct Mma;

template <> struct Mma<Prec::F32> {
  static constexpr int KS = 4;
  __device__ __forceinline__ static f32x4 step(f32x4 acc, const View& A, const View& B, int i0, int j0, int k0) {
    const int l = lane_id();
    const float a = A(i0 + (l & 15), k0 + (l >> 4));
    const float b = B(k0 + (l >> 4), j0 + (l & 15));
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
  }
};

template <> struct Mma<Prec::BF16> {
  static constexpr int KS = 16;
  __device__ __forceinline__ static f32x4 step(f32x4 acc, const View& A, const View& B, int i0, int j0, int k0) {
    const int l = lane_id();
    const int kb = k0 + (l >> 4) * 4;
    bf16x4_t a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = (__bf16)A(i0 + (l & 15), kb + e);
      b[e] = (__bf16)B(kb + e, j0 + (l & 15));
    }
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
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
template <Prec P, int M, int N, int K>
__device__ __forceinline__ void mma(Acc<M, N>& acc, const View A, const View B) {
  using TL = Tiles<M, N>;
  static_assert(K % Mma<P>::KS == 0, "K must be a multiple of the MFMA depth");
#pragma unroll
  for (int q = 0; q < TL::PER; ++q) {
    const int t = wave_id() + q * NW;  // uniform across the wave
    if (t < TL::TOT) {
      const int i0 = (t / TL::NT) * 16, j0 = (t % TL::NT) * 16;
      f32x4 c = acc.a[q];
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

// ---------------------------------------------------------------- global <-> LDS
template <typename T> __device__ __forceinline__ float to_f(T x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x) { return (T)x; }

// LDS[r][c] (row stride ld) = src[(r) * rs + c] for r < nrows, zero for nrows <= r < R.
template <int R, int Cn, typename T>
__device__ __forceinline__ void load_tile(float* dst, int ld, const T* __restrict__ src, int64_t rs, int nrows) {
  for (int idx = threadIdx.x; idx < R * Cn; idx += NTHREADS) {
    const int r = idx / Cn, c = idx % Cn;
    dst[r * ld + c] = r < nrows ? to_f(src[(int64_t)r * rs + c]) : 0.f;
  }
}

// Same, with every row r scaled by s[r] (an LDS vector).
template <int R, int Cn, typename T>
__device__ __forceinline__ void load_tile_rs(float* dst, int ld, const T* __restrict__ src, int64_t rs, int nrows,
                                             const float* s) {
  for (int idx = threadIdx.x; idx < R * Cn; idx += NTHREADS) {
    const int r = idx / Cn, c = idx % Cn;
    dst[r * ld + c] = r < nrows ? to_f(src[(int64_t)r * rs + c]) * s[r] : 0.f;
  }
}

template <int R, int Cn, typename T>
__device__ __forceinline__ void store_tile(T* __restrict__ dst, int64_t rs, const float* src, int ld, int nrows) {
  for (int idx = threadIdx.x; idx < R * Cn; idx += NTHREADS) {
    const int r = idx / Cn, c = idx % Cn;
    if (r < nrows) dst[(int64_t)r * rs + c] = from_f<T>(src[r * ld + c]);
  }
}

}  // namespace gdn
