// gdn_internal.h -- problem descriptor shared by the host entry points and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct ChunkInfo {
  int seq;  // sequence index, -1 for an unused table slot
  int t0;   // first token (row) of the chunk
  int len;  // tokens in the chunk, 1..C
  int pad;
};

// Everything a kernel needs, passed by value. Dk == Dv == D. Per-(chunk, head)
// arrays are indexed [c][h][...] with c < nc_max (the chunk table's numbering).
struct Prob {
  int N, Hk, Hv, r, D, C, nc_max, T;  // T: tokens per sequence when cu == nullptr
  int64_t T_total;
  float scale;
  const int* cu;  // device [N + 1] or nullptr

  const void* q; int64_t q_rs;
  const void* k; int64_t k_rs;
  const void* v; int64_t v_rs;
  const float* g;     // [T_total][Hv]: g, or alpha when a_log is set
  const float* beta;  // [T_total][Hv]: beta, or beta_raw when a_log is set
  const float* a_log;    // [Hv] or nullptr: gate chain fused (g, beta from alpha, beta_raw)
  const float* dt_bias;  // [Hv], set together with a_log
  const float* S0;    // [N][Hv][D][D] or nullptr

  void* o; int64_t o_rs;
  float* ST;  // [N][Hv][D][D] or nullptr

  const void* dO; int64_t dO_rs;
  const float* dST;  // or nullptr
  void* dq; int64_t dq_rs;
  void* dk; int64_t dk_rs;
  void* dv; int64_t dv_rs;
  float* dg;
  float* dbeta;
  float* dS0;  // or nullptr

  // chunk table
  ChunkInfo* chunks;  // [nc_max]
  int* seq_chunk;     // [N + 1] first chunk of each sequence
  int* seq_order;     // [N] sequences by decreasing chunk count: the sweeps' workgroup order

  // Saved activations written by the forward for the backward, per chunk c and value
  // head h (element type = the problem's storage type OT unless noted):
  void* sv_S;    // [c][h][D][D]  state at the start of the chunk, transposed: S^T[v][d]
  void* sv_D;    // [c][h][D / BV][C][BV]  Delta in blocks of BV = grad_block<OT, D>() value
                 // columns, each block row-major (rows past the end of a chunk not written)
  void* sv_T;    // [c][h][C][C]  T = (I + L)^-1, lower-block form (low_row_off) at the slot's start
  void* sv_M;    // [c][h][C][C]  M = Gamma o Q K^T (lower incl. diagonal), lower-block form
  float* sv_gb;  // [c][h][kGateRows][C]  float32 gate record, rows below
  // q/k L2 normalisation (fused when sv_qn is set): prep writes the normalised rows and
  // 1 / sqrt(|row|^2 + 1e-6) of each q and k head row; every later kernel reads qu / ku.
  void* sv_qn;   // [T_total][Hk][D] storage type, or nullptr
  void* sv_kn;   // [T_total][Hk][D]
  float* sv_r;   // [T_total][Hk][2]: the factor of q, then of k
  const void* qu; int64_t qu_rs;  // the q rows the chunk kernels read: q, or sv_qn
  const void* ku; int64_t ku_rs;
  // workspace
  void* ws_dS;   // [c][h][D][D]  state adjoint flowing into the end of the chunk, dS^T[v][d]
  void* ws_A;    // [c][h][D/BV][C][BV]  A = T^T dDelta in blocks of BV value columns
                 // (BV = grad_block; rows past a chunk's end not written)
};

// Rows of the per-(chunk, value head) gate record: gamma = cumulative log2 g (rows past the
// end add 0), beta (0 past the end), b = 2^gamma and e = 2^(gamma_last - gamma), the two
// decay factors the sweeps apply to every row.
constexpr int kGateRows = 5;
// Rows 0-3 are what the sweeps read; row 4 is d log g / d alpha of the fused gate chain,
// -exp(a_log) sigmoid(alpha + dt_bias) (0 without it), read by the gradient kernel.
constexpr int kSweepGateRows = 4;

// The layer's gate chain: log g = -exp(a_log) softplus(alpha + dt_bias) (returned in log2
// units), beta = sigmoid(beta_raw); and the derivative of log g with respect to alpha,
// -exp(a_log) sigmoid(alpha + dt_bias).
__device__ __forceinline__ float chain_log2g(float alpha, float a_log, float dt_bias) {
  const float z = alpha + dt_bias;
  const float sp = z > 20.f ? z : log1pf(expf(z));  // softplus
  return -expf(a_log) * sp * 1.4426950408889634f;
}
__device__ __forceinline__ float chain_beta(float beta_raw) { return 1.f / (1.f + expf(-beta_raw)); }
__device__ __forceinline__ float chain_dlogg_dalpha(float alpha, float a_log, float dt_bias) {
  return -expf(a_log) / (1.f + expf(-(alpha + dt_bias)));
}

// Value columns per block of the gradient kernel's value loop (also the block width of the
// saved Delta, so that each block is one contiguous run of memory).
template <typename T, int D> constexpr int grad_block() { return sizeof(T) == 2 ? (D >= 32 ? 32 : D) : 16; }

// Benchmark tracing (gdn_trace.cpp): runs launch(ctx), bracketed by HIP events on s
// while tracing is enabled.
bool trace_on();
void trace_launch(const char* name, hipStream_t s, void (*launch)(const void*), const void* ctx);

template <class F>
inline void traced(const char* name, hipStream_t s, const F& f) {
  if (!trace_on()) {
    f();
    return;
  }
  trace_launch(name, s, [](const void* c) { (*static_cast<const F*>(c))(); }, &f);
}

// Device address of the current device's fixed scratch array (gdn_scratch.hip), the workspace
// of gdn_fwd_noalloc: GDN_NOALLOC_SCRATCH_BYTES, 256-byte aligned; nullptr if it cannot be
// looked up.
void* noalloc_scratch();

// Kernel launch sequences (defined in gdn_fwd.hip / gdn_bwd.hip). Return a HIP error code.
hipError_t launch_forward(const Prob& p, int dtype, hipStream_t s);
hipError_t launch_backward(const Prob& p, int dtype, hipStream_t s);

// One decode step (gdn_decode.hip): N rows, one token each, state slots updated in place.
struct DecArgs {
  int N, Hv, r, D, n_slots;
  float scale;
  const void *q, *k, *v;  // row views, element row strides below
  int64_t q_rs, k_rs, v_rs, o_rs;
  const float *g, *beta;  // [N][Hv]: g and beta, or alpha and beta_raw when a_log is set
  const float *a_log, *dt_bias;  // [Hv] or nullptr
  int l2;                 // L2-normalise the q and k rows first
  float* state;           // [n_slots][Hv][D][D]
  const int* idx;         // [N] slot of each row, or nullptr (row n -> slot n)
  void* o;
};
hipError_t launch_decode(const DecArgs& a, int dtype, hipStream_t s);

// Causal depthwise conv1d + SiLU over packed rows (gdn_conv.hip): forward, or the input
// gradient when backward is set.
struct ConvArgs {
  int N, T, ch, K;   // sequences, rows per sequence when cu is null, channels, kernel size
  int64_t rows;      // T_total
  const int* cu;     // [N + 1] row offsets, or nullptr
  const float* w;    // [ch][K]
  const void* x;
  void *y, *dx;
  const void* dy;
  int64_t x_rs, y_rs, dy_rs, dx_rs;
};
hipError_t launch_conv(const ConvArgs& a, int dtype, bool backward, hipStream_t s);

}  // namespace gdn
