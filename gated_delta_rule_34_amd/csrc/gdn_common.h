// gdn_common.h -- chunk table shared by the forward and backward launch sequences.
#pragma once
#include "gdn_internal.h"
#include "gdn_frag.h"

namespace gdn {

constexpr int NTHREADS = 256;  // threads of the chunk-table kernel

// DPP move of x (lanes whose source is outside the row, or whose row is masked off, get 0).
template <int CTRL, int ROWS = 0xF> __device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xF, false));
}

// Sum over the 16 lanes of a DPP row (lanes 16k .. 16k + 15), returned in every lane of
// the row: pair and quad swaps, then the half-row and row mirrors (no LDS traffic).
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}

// Wave-level scans and sums over 64 lanes, in DPP steps (fixed combination order, so the
// results are deterministic).
__device__ __forceinline__ float wave_scan_incl(float x) {  // sum of lanes 0..l
  x += dpp<0x111>(x);       // row_shr:1
  x += dpp<0x112>(x);       // row_shr:2
  x += dpp<0x114>(x);       // row_shr:4
  x += dpp<0x118>(x);       // row_shr:8: inclusive sums within each row of 16
  x += dpp<0x142, 0xA>(x);  // row_bcast:15 -> rows 1 and 3 add the total of the row before
  x += dpp<0x143, 0xC>(x);  // row_bcast:31 -> rows 2 and 3 add the total of rows 0 and 1
  return x;
}
// wave_scan_incl on ints
template <int CTRL, int ROWS = 0xF> __device__ __forceinline__ int dppi(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ int wave_scan_incl_int(int x) {
  x += dppi<0x111>(x);
  x += dppi<0x112>(x);
  x += dppi<0x114>(x);
  x += dppi<0x118>(x);
  x += dppi<0x142, 0xA>(x);
  x += dppi<0x143, 0xC>(x);
  return x;
}
__device__ __forceinline__ float lane_value(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}
__device__ __forceinline__ float wave_sum(float x) { return lane_value(wave_scan_incl(x), 63); }
__device__ __forceinline__ float wave_rscan_incl(float x) {  // sum of lanes l..63
  x += dpp<0x101>(x);  // row_shl:1
  x += dpp<0x102>(x);  // row_shl:2
  x += dpp<0x104>(x);  // row_shl:4
  x += dpp<0x108>(x);  // row_shl:8: sums of lanes l.. end of row
  const float t1 = lane_value(x, 16), t2 = lane_value(x, 32), t3 = lane_value(x, 48);
  const float t23 = t2 + t3, t123 = t1 + t23;
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row == 0 ? t123 : row == 1 ? t23 : row == 2 ? t3 : 0.f);
}

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

// Workgroup b of a grid of xcd_grid(G, r) workgroups, as member mem of group grp, where a
// group is r units that share a key head. Workgroups are dispatched to the 8 XCDs
// round-robin, so the members of a group land on one XCD and share its L2. Returns false
// for the padding workgroups of the last round.
__device__ __forceinline__ bool xcd_group(int b, int G, int r, int& grp, int& mem) {
  const int x = b & 7, s = b >> 3;
  grp = (s / r) * 8 + x;
  mem = s % r;
  return grp < G;
}
__host__ __device__ constexpr int xcd_grid(int G, int r) { return (G + 7) / 8 * 8 * r; }

// Sequences ranked for the sweeps' order up to this count; beyond it the order is the identity.
constexpr int kOrderMax = 1024;

// Global chunk c as the chunk table lays it out (sequences one after the other, chunk by
// chunk, empty ones taking none), found without the table: the per-sequence chunk counts
// are scanned 64 sequences at a time by one wave (every lane of the wave calls it and gets
// the same result). A slot past the last chunk gives seq = -1.
template <int C> __device__ __forceinline__ ChunkInfo find_chunk(const Prob& p, int c) {
  if (!p.cu) {
    const int64_t cps = ((int64_t)p.T + C - 1) / C;  // chunks per sequence
    const int64_t n = cps > 0 ? c / cps : p.N;
    if (n >= p.N) return ChunkInfo{-1, 0, 0, 0};
    const int64_t loc = c - n * cps, t = n * p.T + loc * C, rest = p.T - loc * C;
    return ChunkInfo{(int)n, (int)t, (int)(rest < C ? rest : C), 0};
  }
  const int l = lane_id();
  int64_t base = 0;  // chunks of the sequences before this group of 64
  for (int n0 = 0; n0 < p.N; n0 += 64) {
    const int n = n0 + l;
    int64_t a = 0, b = 0;
    if (n < p.N) seq_bounds(p, n, a, b);
    const int cnt = (int)((b - a + C - 1) / C);
    const int incl = wave_scan_incl_int(cnt);
    const int64_t first = base + incl - cnt;  // the sequence's first chunk
    const bool hit = n < p.N && cnt > 0 && c >= first && c < first + cnt;  // at most one lane
    const uint64_t m = __ballot(hit);
    if (m) {
      const int src = __builtin_ctzll(m);
      const int64_t t = a + (c - first) * C;  // valid in lane src
      const int64_t rest = b - t;
      const int t32 = __builtin_amdgcn_readlane((int)t, src);
      const int len = __builtin_amdgcn_readlane((int)(rest < C ? rest : C), src);
      return ChunkInfo{n0 + src, t32, len, 0};
    }
    base += __builtin_amdgcn_readlane(incl, 63);
  }
  return ChunkInfo{-1, 0, 0, 0};
}

// The chunk table's per-sequence first-chunk offsets and the sweep order, by one workgroup of
// NT threads (cnt: scratch for kOrderMax ints). The sweeps give one workgroup to each
// (sequence, value head) and walk its chunks serially; when there are more of them than CUs,
// the longest sequences must start first (the dispatcher takes workgroups in index order), so
// seq_order lists the sequences by decreasing chunk count (ties by index: a permutation).
template <int C, int NT> __device__ __forceinline__ void seq_table(const Prob& p, int* cnt) {
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
  if (p.N > kOrderMax) {
    for (int n = threadIdx.x; n < p.N; n += NT) p.seq_order[n] = n;
    return;
  }
  for (int n = threadIdx.x; n < p.N; n += NT) cnt[n] = p.seq_chunk[n + 1] - p.seq_chunk[n];
  __syncthreads();
  for (int n = threadIdx.x; n < p.N; n += NT) {
    const int cn = cnt[n];
    int rank = 0;
    for (int m = 0; m < p.N; ++m) rank += (cnt[m] > cn) || (cnt[m] == cn && m < n);
    p.seq_order[rank] = n;
  }
  __syncthreads();
}

// One workgroup: the whole chunk table (the forward's prep kernel writes it itself; this
// kernel serves a problem with sequences but no chunk slots, where prep does not run).
template <int C>
__global__ __launch_bounds__(NTHREADS) void k_table(Prob p) {
  __shared__ int cnt[kOrderMax];
  for (int c = wave_id(); c < p.nc_max; c += NTHREADS / 64) {
    const ChunkInfo ci = find_chunk<C>(p, c);
    if (lane_id() == 0) p.chunks[c] = ci;
  }
  seq_table<C, NTHREADS>(p, cnt);
}

}  // namespace gdn
