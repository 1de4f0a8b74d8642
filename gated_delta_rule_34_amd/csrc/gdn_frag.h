// gdn_frag.h -- MFMA operand fragments for gfx950, read from LDS in either storage
// order, or taken straight from the float32 accumulators of an earlier product.
//
// MFMA shapes: v_mfma_f32_16x16x32_bf16 (KS = 32) or v_mfma_f32_16x16x16_bf16 (KS = 16,
// when the contraction is not a multiple of 32) for bf16 operands, v_mfma_f32_16x16x4_f32
// (KS = 4) for float32 operands. Lane l, group g = l / 16, r = l % 16:
//   A fragment: A[r][k(s, g, j)], j < KE = KS / 4      B fragment: B[k(s, g, j)][r]
//   accumulator element e: D[4 g + e][r]
// Any assignment k(s, g, j) of the contraction index is valid as long as A and B use the
// same one. Two are used:
//   STD: the natural one (g holds KE consecutive indices).
//   ACC: the order in which an accumulator already holds its rows, so that the output of
//        one product feeds the contraction of the next without leaving registers: for
//        KS = 32, step s takes rows 32 s + {4 g + e, 16 + 4 g + e}; for KS = 4 (float32),
//        step s takes row 16 (s / 4) + 4 g + (s % 4). For KS = 16 it equals STD.
//
// Storage orders of an operand X in LDS (layout policy L maps (row, col) to an offset):
//   ld_n: X[m][k] -- the contraction index runs along a row (one 16- or 8-byte read);
//   ld_t: X[k][m] -- the contraction index runs down a column. bf16 uses the CDNA4 LDS
//         transpose read ds_read_b64_tr_b16: in each group of 16 lanes, lane a + 4 f
//         (a, f < 4) points at row f, columns 4a..4a+3 of a 4 x 16 block, and lane d
//         receives column d of the block (rows 0..3). float32 reads one element per lane.
#pragma once
#include <utility>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void_t;

enum { STD = 0, ACC = 1 };

// MFMA depth used for a contraction of length K.
template <typename OT, int K> constexpr int ks_of() {
  if constexpr (sizeof(OT) == 4) return 4;
  else return (K % 32) == 0 ? 32 : 16;
}

template <typename OT, int KS> struct Mf;
template <> struct Mf<float, 4> {
  static constexpr int KE = 1;
  typedef float frag;
  __device__ __forceinline__ static f32x4 run(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};
template <> struct Mf<__bf16, 32> {
  static constexpr int KE = 8;
  typedef bf16x8 frag;
  __device__ __forceinline__ static f32x4 run(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mf<__bf16, 16> {
  static constexpr int KE = 4;
  typedef bf16x4 frag;
  __device__ __forceinline__ static f32x4 run(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
};

// Contraction index of element j held by lane group g at step s.
template <int KS, int ORD> __device__ __forceinline__ int kidx(int s, int g, int j) {
  if constexpr (KS == 4) return ORD == STD ? 4 * s + g : 16 * (s >> 2) + 4 * g + (s & 3);
  else if constexpr (KS == 16) return 16 * s + 4 * g + j;
  else return ORD == STD ? 32 * s + 8 * g + j : 32 * s + 16 * (j >> 2) + 4 * g + (j & 3);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ------------------------------------------------------------------ LDS layouts
// Padded row-major: element (r, c) at r * LD + c.
template <int LD> struct Pad {
  __device__ __forceinline__ static int at(int r, int c) { return r * LD + c; }
};

// Dense row-major [R][Cn] whose 16-byte chunks are XOR-permuted within each row, so that
// the reads of the MFMA fragment loaders fall in distinct banks of the 64 x 4-byte LDS.
// Dense rows are what the direct global-to-LDS loads write. Two row maps:
//  - plain (TR = false): chunk c of row r sits at c xor (r mod 16) (rows of 16 or more
//    chunks; shorter rows use the row's position in its 256-byte bank line band). 16
//    consecutive rows read at one chunk column (ld_n) hit distinct banks;
//  - transpose-friendly (TR = true, bf16 rows of 8 or 16 chunks; RL = 16 / NCH rows per
//    256-byte bank line, k = (r / RL) mod NCH):  s = (2k mod NCH) xor (NCH/2 + 1 if
//    k >= NCH/2). It keeps ld_n conflict-free and also the transpose reads of ld_t and
//    ld_col4, which take two adjacent chunks of 4 rows per lane group and serve two
//    groups per cycle (rows 8j..8j+7, or 8j..8j+3 with 8j+8..8j+11): over any such 8
//    rows the chunk pairs (s >> 1) are distinct. With the plain map those reads measured
//    twice their conflict-free time on the LDS bank-conflict counters (four times where
//    a row's runs are in fragment order; the map leaves the 2-way minimum there). Its
//    row-dependent offsets cost more registers, so kernels choose it per layout.
//
// PT = true leaves a 128-byte gap after every 16 rows. Two reads of one lane in
// neighbouring 16-row tiles then differ by a constant that is not a multiple of 512
// bytes: the compiler keeps them as two ds_read_b64 (one base, immediate offsets) instead
// of fusing them into a ds_read2st64_b64, which measured four times their cost because
// both rows fall in the same banks; and with the gap they fall in different ones.
template <typename T, int Cn, bool TR = false, bool PT = false> struct Swz {
  static constexpr int CE = 16 / (int)sizeof(T), NCH = Cn / CE;
  static_assert(Cn % CE == 0 && (NCH & (NCH - 1)) == 0, "row must be a power-of-two count of 16-byte chunks");
  static_assert(!PT || NCH >= 4, "a direct load of 64 chunks must stay inside one 16-row tile");
  static constexpr int TSTR = 16 * Cn + (PT ? 128 / (int)sizeof(T) : 0);  // elements per 16 rows
  // Elements spanned by R rows (R a multiple of 16 when PT).
  static constexpr int size(int R) { return PT ? (R / 16) * TSTR : R * Cn; }
  __device__ __forceinline__ static int row_off(int r) { return (r >> 4) * TSTR + (r & 15) * Cn; }
  __device__ __forceinline__ static int s(int r) {
    if constexpr (TR && sizeof(T) == 2 && (NCH == 16 || NCH == 8)) {
      constexpr int RL = 16 / NCH, HB = NCH == 16 ? 3 : 2;  // rows per bank line; log2(NCH / 2)
      const int k = (r / RL) & (NCH - 1);
      return ((2 * k) & (NCH - 1)) ^ (((k >> HB) & 1) * (NCH / 2 + 1));
    } else {
      return NCH >= 16 ? (r & 15) : ((r * NCH) >> 4) & (NCH - 1);
    }
  }
  __device__ __forceinline__ static int at(int r, int c) { return row_off(r) + (((c / CE) ^ s(r)) * CE) + (c % CE); }
};

// ------------------------------------------------------------------ fragment loads
template <typename OT, int KS, int ORD, class L>
__device__ __forceinline__ typename Mf<OT, KS>::frag ld_n(const OT* X, int m0, int s) {
  const int l = lane_id(), g = l >> 4, r = l & 15;
  if constexpr (KS == 4) {
    return X[L::at(m0 + r, kidx<KS, ORD>(s, g, 0))];
  } else if constexpr (KS == 16) {
    return *reinterpret_cast<const bf16x4*>(X + L::at(m0 + r, 16 * s + 4 * g));
  } else if constexpr (ORD == STD) {
    return *reinterpret_cast<const bf16x8*>(X + L::at(m0 + r, 32 * s + 8 * g));
  } else {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(X + L::at(m0 + r, 32 * s + 4 * g));
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(X + L::at(m0 + r, 32 * s + 16 + 4 * g));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

// Storage order of a saved row of LEN elements. Rows written from MFMA fragments keep each
// lane's 16-byte fragment contiguous ("fragment order"): for bf16 and LEN % 32 == 0,
// logical index 32 s + 16 h + 4 g + e sits at position 32 s + 8 g + 4 h + e. Runs of four
// consecutive logical indices stay contiguous. Otherwise the order is natural.
template <typename OT, int LEN> struct RowOrd {
  static constexpr bool frag = sizeof(OT) == 2 && LEN % 32 == 0;
  __device__ __forceinline__ static int pos(int j) {
    if constexpr (frag)
      return (j & ~31) | ((j & 12) << 1) | ((j & 16) >> 2) | (j & 3);
    else
      return j;
  }
};
struct NatOrd {
  __device__ __forceinline__ static int pos(int j) { return j; }
};

// Rows kb..kb+3 (kb per lane group) at logical column m0 + l % 16, by one transpose read;
// CM maps a logical column (start of a run of four) to its storage position.
template <class L, class CM = NatOrd>
__device__ __forceinline__ bf16x4 tr4(const __bf16* X, int kb, int m0) {
  const int r = lane_id() & 15;
  const __bf16* p = X + L::at(kb + (r >> 2), CM::pos(m0 + 4 * (r & 3)));
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

template <typename OT, int KS, int ORD, class L, class CM = NatOrd>
__device__ __forceinline__ typename Mf<OT, KS>::frag ld_t(const OT* X, int m0, int s) {
  const int l = lane_id(), g = l >> 4, r = l & 15;
  if constexpr (KS == 4) {
    return X[L::at(kidx<KS, ORD>(s, g, 0), CM::pos(m0 + r))];
  } else if constexpr (KS == 16) {
    return tr4<L, CM>(X, 16 * s + 4 * g, m0);
  } else {
    const bf16x4 lo = tr4<L, CM>(X, kidx<KS, ORD>(s, g, 0), m0);
    const bf16x4 hi = tr4<L, CM>(X, kidx<KS, ORD>(s, g, 4), m0);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

// Four consecutive rows kb..kb+3 of column m0 + l % 16 as float32: the accumulator
// layout of a 16 x 16 tile whose lane group g starts at row kb (kb passed per group).
template <typename OT, class L>
__device__ __forceinline__ f32x4 ld_col4(const OT* X, int kb, int m0) {
  if constexpr (sizeof(OT) == 2) {
    const bf16x4 v = tr4<L>(X, kb, m0);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  } else {
    const int c = m0 + (lane_id() & 15);
    return f32x4{X[L::at(kb, c)], X[L::at(kb + 1, c)], X[L::at(kb + 2, c)], X[L::at(kb + 3, c)]};
  }
}

// Fragment for step s of a contraction over the rows of accumulator tiles t[] (16-row
// tiles along the contraction index), ACC order. Each value passes through
// f(tile, e, value) first; its contraction index is 16 tile + 4 g + e.
template <typename OT, int KS, class F>
__device__ __forceinline__ typename Mf<OT, KS>::frag from_acc(const f32x4* t, int s, F&& f) {
  if constexpr (KS == 4) {
    return f(s >> 2, s & 3, t[s >> 2][s & 3]);
  } else if constexpr (KS == 16) {
    bf16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (__bf16)f(s, e, t[s][e]);
    return o;
  } else {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[e] = (__bf16)f(2 * s, e, t[2 * s][e]);
      o[4 + e] = (__bf16)f(2 * s + 1, e, t[2 * s + 1][e]);
    }
    return o;
  }
}

// An ACC-order fragment whose element of contraction index 16 tile + 4 g + e is
// multiplied by fac[tile][e] (per-row factors held in registers).
template <typename OT, int KS, int NTILE>
__device__ __forceinline__ typename Mf<OT, KS>::frag scale_acc(typename Mf<OT, KS>::frag x, int s,
                                                                const float (&fac)[NTILE][4]) {
  if constexpr (KS == 4) {
    return x * fac[s >> 2][s & 3];
  } else if constexpr (KS == 16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (__bf16)((float)x[e] * fac[s][e]);
    return x;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = (__bf16)((float)x[e] * fac[2 * s][e]);
      x[4 + e] = (__bf16)((float)x[4 + e] * fac[2 * s + 1][e]);
    }
    return x;
  }
}

struct Ident {
  __device__ __forceinline__ float operator()(int, int, float x) const { return x; }
};

// 16-byte vectors of T.
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  typedef float type __attribute__((ext_vector_type(4)));
};
template <> struct Vec16<__bf16> {
  static constexpr int N = 8;
  typedef __bf16 type __attribute__((ext_vector_type(8)));
};

// A product whose A operand is triangular by 16 x 16 tiles (row tile m = rows 16 m ..
// 16 m + 15): TRI_LOW, zero where k >= 16 (m + 1); TRI_UP, zero where k < 16 m. A
// contraction step whose indices all lie there adds nothing and is skipped, with its
// fragment reads. The indices of step s lie in [lo, lo + w): KS s and KS wide for KS = 32 or
// 16 in either order; one tile of 16 for KS = 4 (STD takes four of them, ACC spreads its
// four over the tile).
enum { TRI_NONE = 0, TRI_LOW = 1, TRI_UP = 2 };
template <int TRI, int KS> __device__ __forceinline__ constexpr bool tri_skip(int s, int m) {
  const int lo = KS == 4 ? 16 * (s >> 2) : KS * s, wd = KS == 4 ? 16 : KS;
  return TRI == TRI_LOW ? lo >= 16 * (m + 1) : (TRI == TRI_UP ? lo + wd <= 16 * m : false);
}

// acc[m][n] += sum_k A(m, k) B(k, n) over a contraction of length K for a wave's
// MT x NT block of 16 x 16 tiles. fa(m, s) and fb(n, s) return the step-s fragments;
// the NT B fragments of a step are loaded once and reused across the MT A fragments.
// With TRI, m must be the absolute row tile of A.
template <typename OT, int K, int MT, int NT, int TRI = TRI_NONE, class FA, class FB>
__device__ __forceinline__ void wave_mm(f32x4 (&acc)[MT][NT], FA&& fa, FB&& fb) {
  constexpr int KS = ks_of<OT, K>();
  using M = Mf<OT, KS>;
  static_assert(K % KS == 0, "contraction must be a multiple of the MFMA depth");
#pragma unroll
  for (int s = 0; s < K / KS; ++s) {
    typename M::frag b[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) b[n] = fb(n, s);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (tri_skip<TRI, KS>(s, m)) continue;
      const typename M::frag a = fa(m, s);
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[m][n] = M::run(a, b[n], acc[m][n]);
    }
  }
}

// acc[n][m] += sum_k A(m, k) B(k, n): wave_mm with the accumulator tiles stored
// column-tile major (the layout from_acc reads when the result feeds a later product).
template <typename OT, int K, int MT, int NT, int TRI = TRI_NONE, class FA, class FB>
__device__ __forceinline__ void wave_mm_cm(f32x4 (&acc)[NT][MT], FA&& fa, FB&& fb) {
  constexpr int KS = ks_of<OT, K>();
  using M = Mf<OT, KS>;
#pragma unroll
  for (int s = 0; s < K / KS; ++s) {
    typename M::frag b[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) b[n] = fb(n, s);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (tri_skip<TRI, KS>(s, m)) continue;
      const typename M::frag a = fa(m, s);
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n][m] = M::run(a, b[n], acc[n][m]);
    }
  }
}

template <int MT, int NT> __device__ __forceinline__ void zero(f32x4 (&acc)[MT][NT]) {
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// ------------------------------------------------------------------ direct global -> LDS
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource over [base, base + bytes) (stride 0, the gfx9 default format word):
// a load at a byte offset at or past `bytes` returns zeros. The caller's base and size are
// wave-uniform; readfirstlane makes that explicit, so the resource always lives in SGPRs.
__device__ __forceinline__ i32x4 buf_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a),
               __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(a >> 32)),
               __builtin_amdgcn_readfirstlane((int32_t)bytes), 0x00020000};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(p);
}

// One 16-byte direct load per lane (buffer_load_dwordx4 ... lds): the 16 bytes at byte
// offset voff of the buffer land at LDS byte address lds + 16 * lane. Issued through
// inline assembly on purpose: the compiler's wait-count pass cannot tell which LDS bytes
// such a load writes, and for the builtin it makes every later LDS read wait for all
// outstanding loads, which would expose the whole latency of a prefetch. Completion is
// the caller's business: dma_wait() in every issuing wave, then a workgroup barrier.
// M0 holds the LDS address; nothing in these kernels keeps M0 live across the statement.
// NT marks the load non-temporal (the `nt` cache policy): for data that one workgroup reads
// once, the kernels measured 5-17% faster with it (and the caches keep what several
// workgroups share, such as the sweeps' K and Q, which stay temporal).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <bool NT = false> __device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t lds) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff),
                 "s"(rsrc), "s"(lds)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc),
                 "s"(lds)
                 : "memory", "m0");
}
// As dma16, with the wave-uniform byte offset soff added to every lane's offset (the
// instruction's scalar offset).
template <bool NT = false> __device__ __forceinline__ void dma16s(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen nt lds" ::"v"(voff),
                 "s"(rsrc), "s"(soff), "s"(lds)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc),
                 "s"(soff), "s"(lds)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Direct loads of a global tile [R][Cn] into LDS in the layout Swz<T, Cn, TR, PT>, issued by NW
// waves (wave index w < NW); each wave instruction fills 1 KiB of LDS. Each lane's row and
// byte offset within the row are fixed per instruction and computed once; issue() then
// costs one multiply-add per instruction. Rows at or past nvalid fall outside the buffer
// range and arrive as zeros, so rows past the end of a chunk read as zero and nothing
// outside the caller's rows is read. Row stride times R times sizeof(T) must fit in 32 bits
// (checked on the host).
template <int R, int Cn, int NW, typename T, bool TR = false, bool PT = false> struct TileDma {
  using L = Swz<T, Cn, TR, PT>;
  static_assert(!PT || R % 16 == 0, "padded tiles hold whole 16-row groups");
  static constexpr int TOT = R * L::NCH, U = (TOT + NW * 64 - 1) / (NW * 64);
  // Instructions per wave when every wave issues the same number, else -1.
  static constexpr int CNT = TOT % (NW * 64) == 0 ? U : -1;
  uint32_t row[U], cof[U];
  __device__ __forceinline__ void init(int w) {
    const int l = lane_id();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pch = (u * NW + w) * 64 + l;
      const int r = pch / L::NCH, c = (pch % L::NCH) ^ L::s(r);
      row[u] = (uint32_t)r;
      cof[u] = (uint32_t)(c * 16);
    }
  }
  // Instructions wave w issues per tile (wave-uniform).
  __device__ __forceinline__ static int count(int w) {
    int n = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) n += (u * NW + w) * 64 < TOT ? 1 : 0;
    return n;
  }
  // As issue(), from a resource built by the caller (row stride rsb bytes), every lane's
  // offset moved by the wave-uniform soff bytes.
  template <bool NT = false>
  __device__ __forceinline__ void issue_rs(T* lds, i32x4 rsrc, uint32_t rsb, uint32_t soff, int w) const {
    const uint32_t la = lds_addr(lds);
    const int l = lane_id();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int base = (u * NW + w) * 64;
      if (base < TOT && (TOT % 64 == 0 || base + l < TOT))
        dma16s<NT>(rsrc, row[u] * rsb + cof[u], soff,
               __builtin_amdgcn_readfirstlane(la + (uint32_t)(L::row_off(base / L::NCH) * (int)sizeof(T))));
    }
  }
  template <bool NT = false>
  __device__ __forceinline__ void issue(T* lds, const T* src, int64_t rs, int nvalid, int w) const {
    const uint32_t rsb = (uint32_t)(rs * (int64_t)sizeof(T));
    const i32x4 rsrc = buf_rsrc(src, (uint32_t)nvalid * rsb);
    const uint32_t la = lds_addr(lds);
    const int l = lane_id();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int base = (u * NW + w) * 64;
      if (base < TOT && base + l < TOT)
        dma16<NT>(rsrc, row[u] * rsb + cof[u],
              __builtin_amdgcn_readfirstlane(la + (uint32_t)(L::row_off(base / L::NCH) * (int)sizeof(T))));
    }
  }
};

// Lower-block form of a C x C matrix that is zero above its 16 x 16 diagonal blocks (T and
// M of a chunk): row r keeps its first low_row_len(r) elements, at element low_row_off(r),
// rows one after the other. At C = 64 that is 10 of the 16 blocks.
__host__ __device__ constexpr int low_row_len(int r) { return 16 * (r / 16 + 1); }
__host__ __device__ constexpr int low_row_off(int r) { return 128 * (r / 16) * (r / 16 + 1) + low_row_len(r) * (r % 16); }

// Direct loads of a C x C tile in lower-block form into LDS in the dense layout
// Swz<T, C, TR, PT> (same slots as TileDma<C, C, NW, T, TR, PT>). Lanes whose 16-byte piece
// lies above the diagonal blocks load nothing: those pieces keep the zeros zero_upper()
// wrote into the buffer once.
template <int C, int NW, typename T, bool TR = false, bool PT = false> struct TileDmaLow {
  using L = Swz<T, C, TR, PT>;
  static constexpr int TOT = C * L::NCH, U = (TOT + NW * 64 - 1) / (NW * 64);
  static constexpr uint32_t NONE = 0xFFFFFFFFu;
  uint32_t off[U];  // byte offset of the lane's piece in the lower-block form, or NONE
  __device__ __forceinline__ void init(int w) {
    const int l = lane_id();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pch = (u * NW + w) * 64 + l;
      const int r = pch / L::NCH, c = (pch % L::NCH) ^ L::s(r);
      off[u] = (pch < TOT && c * L::CE < low_row_len(r)) ? (uint32_t)((low_row_off(r) + c * L::CE) * (int)sizeof(T)) : NONE;
    }
  }
  template <bool NT = false> __device__ __forceinline__ void issue(T* lds, const T* src, int w) const {
    const i32x4 rsrc = buf_rsrc(src, (uint32_t)(low_row_off(C) * (int)sizeof(T)));
    const uint32_t la = lds_addr(lds);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int base = (u * NW + w) * 64;
      if (base < TOT && off[u] != NONE)
        dma16<NT>(rsrc, off[u], __builtin_amdgcn_readfirstlane(la + (uint32_t)(L::row_off(base / L::NCH) * (int)sizeof(T))));
    }
  }
  // Zeros into the pieces above the diagonal blocks (the ones issue() never writes).
  __device__ __forceinline__ void zero_upper(T* lds, int w) const {
    const int l = lane_id();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int base = (u * NW + w) * 64;
      if (base + l < TOT && off[u] == NONE) {
        typedef int32_t z4 __attribute__((ext_vector_type(4)));
        *reinterpret_cast<z4*>(reinterpret_cast<char*>(lds) + L::row_off(base / L::NCH) * (int)sizeof(T) + 16 * l) =
            z4{0, 0, 0, 0};
      }
    }
  }
};

// Wait until this wave's outstanding vector-memory operations (loads into LDS included)
// have completed: s_waitcnt vmcnt(0), other counters left alone.
__device__ __forceinline__ void dma_wait() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most n of this wave's vector-memory operations are outstanding. They
// complete in issue order, so this waits for everything issued before the last n. n must
// be wave-uniform; above 15 it waits as for 15 (an earlier point, never a later one).
__device__ __forceinline__ void dma_wait_keep(int n) {
#define GDN_VMCNT(k) \
  case k: __builtin_amdgcn_s_waitcnt(0x0F70 | k); break;
  switch (n < 15 ? n : 15) {
    GDN_VMCNT(0) GDN_VMCNT(1) GDN_VMCNT(2) GDN_VMCNT(3) GDN_VMCNT(4) GDN_VMCNT(5) GDN_VMCNT(6) GDN_VMCNT(7)
    GDN_VMCNT(8) GDN_VMCNT(9) GDN_VMCNT(10) GDN_VMCNT(11) GDN_VMCNT(12) GDN_VMCNT(13) GDN_VMCNT(14)
    default: __builtin_amdgcn_s_waitcnt(0x0F70 | 15); break;
  }
#undef GDN_VMCNT
}

// A 16-byte store with the non-temporal cache policy (for results no later step of the same
// kernel reads back).
template <typename V> __device__ __forceinline__ void store_nt(V* p, V x) {
  static_assert(sizeof(V) == 16, "16-byte stores");
  typedef int32_t i4 __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(__builtin_bit_cast(i4, x), reinterpret_cast<i4*>(p));
}

// Workgroup barrier that orders LDS accesses only: it does not wait for the wave's
// outstanding global memory operations, so loads into LDS stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// f(std::integral_constant<int, i>{}) for i = 0 .. N - 1, in order (i is a constant in f).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F> __device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Wave index, uniform across the wave (kept in a scalar register).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

}  // namespace gdn
