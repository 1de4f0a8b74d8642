// gdn_mma.h -- register-blocked "NT" matrix products on CDNA4 MFMA with operands in LDS.
//
// C[M][N] += sum_k A[M][K] * Bt[N][K]: both operands are stored with the contraction
// index contiguous (A row-major, B given as its transpose), so every lane reads its
// fragment with one vector LDS read. Operand element type OT is __bf16 (MFMA
// v_mfma_f32_16x16x32_bf16, or ..._16x16x16_bf16 when K is not a multiple of 32) or
// float (v_mfma_f32_16x16x4_f32); accumulation is float32.
//
// The M x N output is cut into blocks of TM x TN tiles of 16 x 16; block q of a
// workgroup with NWV waves belongs to wave q % NWV. Per k-step a wave reads TM A
// fragments and TN B fragments and issues TM * TN MFMAs (register reuse).
//
// Lane layout of a 16 x 16 x KS MFMA (lane l, element e):
//   A: A[l % 16][(l / 16) * KE + e]   B: B[(l / 16) * KE + e][l % 16]   (KE = KS / 4)
//   D: D[(l / 16) * 4 + e][l % 16], e < 4
// A and B share the k mapping, so any consistent ordering of k inside a step gives
// the same product.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename OT, int K> struct MmaOp;

template <int K> struct MmaOp<float, K> {
  static constexpr int KS = 4, KE = 1;
  typedef float frag;
  __device__ __forceinline__ static frag ld(const float* p) { return *p; }
  __device__ __forceinline__ static f32x4 run(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

template <int K> struct MmaOp<__bf16, K> {
  static constexpr bool wide = (K % 32) == 0;
  static constexpr int KS = wide ? 32 : 16, KE = KS / 4;
  typedef __bf16 frag __attribute__((ext_vector_type(KE)));
  __device__ __forceinline__ static frag ld(const __bf16* p) { return *reinterpret_cast<const frag*>(p); }
  __device__ __forceinline__ static f32x4 run(frag a, frag b, f32x4 c) {
    if constexpr (wide)
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
};

template <int M, int N, int TM, int TN, int NWV> struct Blk {
  static_assert(M % (16 * TM) == 0 && N % (16 * TN) == 0, "block shape");
  static constexpr int BM = M / (16 * TM), BN = N / (16 * TN), NB = BM * BN;
  static constexpr int PER = (NB + NWV - 1) / NWV;
};

// Accumulators of one wave for an M x N product blocked TM x TN over NWV waves.
template <int M, int N, int TM, int TN, int NWV> struct Tile {
  using B = Blk<M, N, TM, TN, NWV>;
  f32x4 a[B::PER][TM][TN];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int q = 0; q < B::PER; ++q)
#pragma unroll
      for (int x = 0; x < TM; ++x)
#pragma unroll
        for (int y = 0; y < TN; ++y) a[q][x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // f(i, j, value&) for every element this lane owns (value may be modified).
  template <class F> __device__ __forceinline__ void each(F&& f) {
    const int w = threadIdx.x / 64, l = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < B::PER; ++q) {
      const int b = w + q * NWV;
      if (b < B::NB) {
        const int bi = (b / B::BN) * 16 * TM, bj = (b % B::BN) * 16 * TN;
#pragma unroll
        for (int x = 0; x < TM; ++x)
#pragma unroll
          for (int y = 0; y < TN; ++y) {
            const int i0 = bi + x * 16 + (l >> 4) * 4, j = bj + y * 16 + (l & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float t = a[q][x][y][e];
              f(i0 + e, j, t);
              a[q][x][y][e] = t;
            }
          }
      }
    }
  }

  // f(i, j, x&, y&) over this tile and another of the same shape (same element order).
  template <class F> __device__ __forceinline__ void each_with(Tile& o, F&& f) {
    const int w = threadIdx.x / 64, l = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < B::PER; ++q) {
      const int b = w + q * NWV;
      if (b < B::NB) {
        const int bi = (b / B::BN) * 16 * TM, bj = (b % B::BN) * 16 * TN;
#pragma unroll
        for (int x = 0; x < TM; ++x)
#pragma unroll
          for (int y = 0; y < TN; ++y) {
            const int i0 = bi + x * 16 + (l >> 4) * 4, j = bj + y * 16 + (l & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float t = a[q][x][y][e], u = o.a[q][x][y][e];
              f(i0 + e, j, t, u);
              a[q][x][y][e] = t;
              o.a[q][x][y][e] = u;
            }
          }
      }
    }
  }

  // f(i0, j, f32x4&) per 4-row run: rows i0..i0+3 of column j.
  template <class F> __device__ __forceinline__ void each4(F&& f) {
    const int w = threadIdx.x / 64, l = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < B::PER; ++q) {
      const int b = w + q * NWV;
      if (b < B::NB) {
        const int bi = (b / B::BN) * 16 * TM, bj = (b % B::BN) * 16 * TN;
#pragma unroll
        for (int x = 0; x < TM; ++x)
#pragma unroll
          for (int y = 0; y < TN; ++y) f(bi + x * 16 + (l >> 4) * 4, bj + y * 16 + (l & 15), a[q][x][y]);
      }
    }
  }
};

// ------------------------------------------------------------------ LDS layouts
// Padded row-major: element (r, c) at r * LD + c.
template <int LD> struct Pad {
  __device__ __forceinline__ static int at(int r, int c) { return r * LD + c; }
};

// Dense row-major [R][Cn] whose 16-byte chunks are XOR-permuted within each row. An MFMA
// fragment load reads the same chunk of 16 consecutive rows; the permutation puts those
// 16 chunks in distinct banks without padding, and dense rows are what the direct
// global-to-LDS loads (dma_tile) write.
template <typename T, int Cn> struct Swz {
  static constexpr int CE = 16 / (int)sizeof(T), NCH = Cn / CE;
  static_assert(Cn % CE == 0 && (NCH & (NCH - 1)) == 0, "row must be a power-of-two count of 16-byte chunks");
  __device__ __forceinline__ static int s(int r) { return NCH >= 16 ? (r & 15) : ((r * NCH) >> 4) & (NCH - 1); }
  __device__ __forceinline__ static int at(int r, int c) { return r * Cn + (((c / CE) ^ s(r)) * CE) + (c % CE); }
};

// acc += A * Bt^T with A [M][K] in layout LA and Bt [N][K] in layout LB (element type OT).
template <typename OT, int M, int N, int K, int TM, int TN, int NWV, class LA, class LB>
__device__ __forceinline__ void gemm_l(Tile<M, N, TM, TN, NWV>& acc, const OT* A, const OT* Bt) {
  using Op = MmaOp<OT, K>;
  using B = Blk<M, N, TM, TN, NWV>;
  static_assert(K % Op::KS == 0, "K must be a multiple of the MFMA depth");
  const int w = threadIdx.x / 64, l = threadIdx.x & 63;
  const int r = l & 15, kq = (l >> 4) * Op::KE;
#pragma unroll
  for (int q = 0; q < B::PER; ++q) {
    const int b = w + q * NWV;
    if (b < B::NB) {
      const int bi = (b / B::BN) * 16 * TM, bj = (b % B::BN) * 16 * TN;
#pragma unroll
      for (int k0 = 0; k0 < K; k0 += Op::KS) {
        typename Op::frag fa[TM], fb[TN];
#pragma unroll
        for (int x = 0; x < TM; ++x) fa[x] = Op::ld(A + LA::at(bi + x * 16 + r, k0 + kq));
#pragma unroll
        for (int y = 0; y < TN; ++y) fb[y] = Op::ld(Bt + LB::at(bj + y * 16 + r, k0 + kq));
#pragma unroll
        for (int x = 0; x < TM; ++x)
#pragma unroll
          for (int y = 0; y < TN; ++y) acc.a[q][x][y] = Op::run(fa[x], fb[y], acc.a[q][x][y]);
      }
    }
  }
}

// acc += A * Bt^T. A: LDS [M][LDA], Bt: LDS [N][LDB] (padded row-major).
template <typename OT, int M, int N, int K, int TM, int TN, int NWV, int LDA, int LDB>
__device__ __forceinline__ void gemm_nt(Tile<M, N, TM, TN, NWV>& acc, const OT* A, const OT* Bt) {
  gemm_l<OT, M, N, K, TM, TN, NWV, Pad<LDA>, Pad<LDB>>(acc, A, Bt);
}

// ------------------------------------------------------------------ direct global -> LDS
typedef __attribute__((address_space(3))) void lds_void_t;

// Asynchronous copy of the global tile [R][Cn] (row stride rs elements) into LDS in the
// layout Swz<T, Cn>, by 16-byte direct global-to-LDS loads (global_load_lds_dwordx4): no
// registers are involved, and each wave instruction fills 1 KiB of LDS. Rows at or past
// nvalid (>= 1) repeat row nvalid - 1, so nothing outside the caller's rows is read.
// Completion: every wave waits with dma_wait(), then the workgroup synchronises.
template <int R, int Cn, int NT, typename T>
__device__ __forceinline__ void dma_tile(T* lds, const T* __restrict__ src, int64_t rs, int nvalid) {
  using L = Swz<T, Cn>;
  constexpr int TOT = R * L::NCH, NW = NT / 64, U = (TOT + NT - 1) / NT;
  const int l = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int base = (u * NW + w) * 64;  // first chunk this wave instruction writes
    if (base < TOT) {
      const int pch = base + l;
      if (pch < TOT) {
        const int r = pch / L::NCH, c = (pch % L::NCH) ^ L::s(r);
        const int rr = r < nvalid ? r : nvalid - 1;
        __builtin_amdgcn_global_load_lds((const void*)(src + (int64_t)rr * rs + c * L::CE),
                                         (lds_void_t*)(lds + base * L::CE), 16, 0, 0);
      }
    }
  }
}

// Wait until this wave's outstanding vector-memory operations (loads into LDS included)
// have completed: s_waitcnt vmcnt(0), other counters left alone.
__device__ __forceinline__ void dma_wait() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier that orders LDS accesses only. Unlike __syncthreads() it does not wait
// for the wave's outstanding global memory operations, so loads into LDS issued before it
// stay in flight across it (dma_wait() waits for them).
// (A fence, even one limited to LDS, would also wait for loads into LDS still in flight.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ------------------------------------------------------------------ LDS staging
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  typedef float type __attribute__((ext_vector_type(4)));
};
template <> struct Vec16<__bf16> {
  static constexpr int N = 8;
  typedef __bf16 type __attribute__((ext_vector_type(8)));
};

template <typename D, typename S> __device__ __forceinline__ D cvt(S x) { return (D)(float)x; }
template <> __device__ __forceinline__ float cvt<float, float>(float x) { return x; }

// Global [R][Cn] (row stride rs elements, rows >= nrows read as zero) into registers:
// each of NT threads holds PER 16-byte vectors. Issue, then commit to LDS later, so
// the loads overlap other work.
template <int R, int Cn, int NT, typename T> struct Stage {
  using V = Vec16<T>;
  static constexpr int VPR = Cn / V::N, NV = R * VPR, PER = (NV + NT - 1) / NT;
  static_assert(Cn % V::N == 0, "row width must be a multiple of the vector width");
  typename V::type v[PER];

  __device__ __forceinline__ void issue(const T* __restrict__ src, int64_t rs, int nrows) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = threadIdx.x + u * NT;
      const int r = idx / VPR, c = (idx % VPR) * V::N;
      if (idx < NV && r < nrows)
        v[u] = *reinterpret_cast<const typename V::type*>(src + (int64_t)r * rs + c);
      else
        v[u] = typename V::type{};
    }
  }
  // LDS [r][c] (row stride LD) as OT, optionally times s[r] and k.
  template <int LD, typename OT>
  __device__ __forceinline__ void to_rows(OT* dst, const float* s = nullptr, float k = 1.f) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = threadIdx.x + u * NT;
      if (idx < NV) {
        const int r = idx / VPR, c = (idx % VPR) * V::N;
        const float sc = (s ? s[r] : 1.f) * k;
        typedef OT ot_vec __attribute__((ext_vector_type(V::N)));
        ot_vec o;
#pragma unroll
        for (int e = 0; e < V::N; ++e) o[e] = cvt<OT>((float)v[u][e] * sc);
        *reinterpret_cast<ot_vec*>(dst + r * LD + c) = o;
      }
    }
  }
  // LDS [r][c] (row stride LD), bits copied unchanged (storage type already the LDS type).
  template <int LD>
  __device__ __forceinline__ void to_rows_raw(T* dst) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = threadIdx.x + u * NT;
      if (idx < NV) {
        const int r = idx / VPR, c = (idx % VPR) * V::N;
        *reinterpret_cast<typename V::type*>(dst + r * LD + c) = v[u];
      }
    }
  }
  // LDS [c][r] (the transpose, row stride LD) as OT, optionally times s[r], k and sc[c].
  template <int LD, typename OT>
  __device__ __forceinline__ void to_cols(OT* dst, const float* s = nullptr, float k = 1.f,
                                          const float* scol = nullptr) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = threadIdx.x + u * NT;
      if (idx < NV) {
        const int r = idx / VPR, c = (idx % VPR) * V::N;
        const float sc = (s ? s[r] : 1.f) * k;
#pragma unroll
        for (int e = 0; e < V::N; ++e)
          dst[(c + e) * LD + r] = cvt<OT>((float)v[u][e] * sc * (scol ? scol[c + e] : 1.f));
      }
    }
  }
};

// Contiguous global [Cn][R] = transpose of the LDS matrix [R][LD] (its first Cn
// columns): each thread gathers one 16-byte run down a column, lanes walk the columns.
template <int R, int Cn, int LD, int NT, typename OT>
__device__ __forceinline__ void lds_to_global_t(OT* __restrict__ dst, const OT* src) {
  using V = Vec16<OT>;
  constexpr int VR = R / V::N;
  static_assert(R % V::N == 0, "rows must fill whole vectors");
  for (int idx = threadIdx.x; idx < Cn * VR; idx += NT) {
    const int c = idx % Cn, r0 = (idx / Cn) * V::N;
    typename V::type x;
#pragma unroll
    for (int e = 0; e < V::N; ++e) x[e] = src[(r0 + e) * LD + c];
    *reinterpret_cast<typename V::type*>(dst + (size_t)c * R + r0) = x;
  }
}

// Contiguous global [R][Cn] = LDS [R][LD] (its first Cn columns), 16 B at a time.
template <int R, int Cn, int LD, int NT, typename OT>
__device__ __forceinline__ void lds_to_global(OT* __restrict__ dst, const OT* src) {
  using V = Vec16<OT>;
  constexpr int VPR = Cn / V::N;
  for (int idx = threadIdx.x; idx < R * VPR; idx += NT) {
    const int r = idx / VPR, c = (idx % VPR) * V::N;
    *reinterpret_cast<typename V::type*>(dst + (size_t)r * Cn + c) =
        *reinterpret_cast<const typename V::type*>(src + r * LD + c);
  }
}

}  // namespace gdn
