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

// Everything a kernel needs, passed by value. Dk == Dv == D.
// Per-(chunk, value head) workspace arrays are indexed [c][h][...] with
// c < nc_max; the layout of each is given next to its pointer.
struct Prob {
  int N, Hk, Hv, r, D, C, nc_max, T;  // T: tokens per sequence when cu == nullptr
  int64_t T_total;
  float scale;
  const int* cu;  // device [N + 1] or nullptr

  const void* q; int64_t q_rs;
  const void* k; int64_t k_rs;
  const void* v; int64_t v_rs;
  const float* g;     // [T_total][Hv]
  const float* beta;  // [T_total][Hv]
  const float* S0;    // [N][Hv][D][D] or nullptr

  void* o; int64_t o_rs;
  float* ST;      // [N][Hv][D][D] or nullptr
  float* states;  // [nc_max][Hv][D][D]: state at the start of every chunk

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

  // workspace
  float* gam;   // [c][h][C]    within-chunk cumulative log decay
  float* Tm;    // [c][h][C][C] (I + L)^-1
  float* W;     // [c][h][C][D]
  float* U;     // [c][h][C][D] U, overwritten by Delta = U - W S0
  float* dDi;   // [c][h][C][D] intra-chunk part of dDelta
  float* dDel;  // [c][h][C][D] dDelta
  float* dstates;  // [c][h][D][D] state adjoint at the end of every chunk
  float* XQ;    // [c][h][C][D] dO~ S0^T
  float* XW;    // [c][h][C][D] dDelta S0^T
  float* XK;    // [c][h][C][D] (e * Delta) dS^T
  float* Pb;    // [c][h][C][C] tril(dO~ Delta^T)
  float* dT;    // [c][h][C][C] dT (first its dU part)
  float* ebar;  // [c][h][C]
  float* rq;    // [c][h][C] rowsum(Q * XQ)
  float* rho;   // [c][h][C]
  float* db1;   // [c][h][C]
  float* sdot;  // [c][h]
  float* dKbb;  // [c][h][C][D]
  float* dqh;   // [c][h][C][D] per-value-head dq
  float* dkh;   // [c][h][C][D] per-value-head dk
};

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

// Kernel launch sequences (defined in gdn_fwd.hip / gdn_bwd.hip). Return a HIP error code.
hipError_t launch_forward(const Prob& p, int dtype, hipStream_t s);
hipError_t launch_backward(const Prob& p, int dtype, hipStream_t s);

}  // namespace gdn
