// gdn_abi.cpp -- host side of the C ABI declared in include/gdn.h: argument checks,
// workspace layout and kernel launch sequencing. No allocation, no synchronisation.
#include "gdn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "gdn_internal.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Shape {
  int64_t nc_max;
  int C, D;
};

// Upper bound on the number of chunks: sum_n ceil(len_n / C).
int64_t chunk_bound(const gdn_problem* p) {
  const int64_t C = p->chunk;
  if (p->cu_seqlens) return (p->T_total + (int64_t)p->N * (C - 1)) / C;
  return (int64_t)p->N * (((int64_t)p->T + C - 1) / C);
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

gdn_status check_problem(const gdn_problem* p) {
  if (!p) return GDN_EINVAL;
  if (p->N < 0 || p->T_total < 0 || p->Hk <= 0 || p->Hv <= 0 || p->Hv % p->Hk) return GDN_EINVAL;
  if (p->Dk <= 0 || p->Dv <= 0) return GDN_EINVAL;
  if (p->dtype != GDN_F32 && p->dtype != GDN_BF16) return GDN_EUNSUPPORTED;
  if (p->Dk != p->Dv) return GDN_EUNSUPPORTED;
  if (p->Dk != 16 && p->Dk != 32 && p->Dk != 64 && p->Dk != 128) return GDN_EUNSUPPORTED;
  if (p->chunk != 16 && p->chunk != 64) return GDN_EUNSUPPORTED;
  if (p->dtype == GDN_F32 && p->chunk == 64 && p->Dk > 32) return GDN_EUNSUPPORTED;  // LDS budget
  if (!std::isfinite(p->scale)) return GDN_EINVAL;
  if ((p->a_log == nullptr) != (p->dt_bias == nullptr)) return GDN_EINVAL;
  if (!aligned(p->a_log, 4) || !aligned(p->dt_bias, 4)) return GDN_EALIGN;
  if (!p->cu_seqlens) {
    if (p->T < 0 || (int64_t)p->N * p->T != p->T_total) return GDN_EINVAL;
  } else if (p->N == 0 && p->T_total != 0) {
    return GDN_EINVAL;
  }
  if (p->T_total > INT32_MAX - 64) return GDN_EINVAL;
  const int64_t nc = chunk_bound(p);
  if (nc > INT32_MAX / 64) return GDN_EINVAL;
  if (nc * p->Hk > INT32_MAX) return GDN_EINVAL;  // one workgroup per (chunk, key head)
  return GDN_OK;
}

// Region sizes in bytes (each rounded up to 256 B).
struct Regions {
  size_t chunks, seq_chunk;        // chunk table; first chunk per sequence and the sweep order
  size_t oDD, oCD, oCC, gb;        // per (chunk, value head): [D][D], [D][C], [C][C] elements, [kGateRows][C] f32
  size_t qn, rr;                   // normalised q or k rows, their factors (0 without qk_l2norm)
};

Regions regions(const gdn_problem* p) {
  const size_t nc = (size_t)chunk_bound(p), Hv = (size_t)p->Hv, C = (size_t)p->chunk, D = (size_t)p->Dk;
  const size_t es = p->dtype == GDN_BF16 ? 2 : 4;
  Regions r;
  r.chunks = align_up(nc * sizeof(gdn::ChunkInfo));
  r.seq_chunk = align_up((2 * (size_t)p->N + 1) * sizeof(int));  // first chunks, then the sweep order
  r.oDD = align_up(nc * Hv * D * D * es);
  r.oCD = align_up(nc * Hv * C * D * es);
  r.oCC = align_up(nc * Hv * C * C * es);
  r.gb = align_up(nc * Hv * gdn::kGateRows * C * sizeof(float));
  r.qn = p->qk_l2norm ? align_up((size_t)p->T_total * p->Hk * D * es) : 0;
  r.rr = p->qk_l2norm ? align_up((size_t)p->T_total * p->Hk * 2 * sizeof(float)) : 0;
  return r;
}

// A forward that saves its chunk states (for a backward) needs no workspace: its only
// scratch, the chunk table, is saved with them. A forward-only call (chunk_states NULL)
// keeps in the workspace what prep writes and the sweep reads: the chunk table, T, M, the
// gate record (and the normalised q, k rows with their factors), but no chunk-start states
// and no Delta, which only the backward reads.
size_t fwd_ws(const gdn_problem* p) {
  const Regions r = regions(p);
  return r.chunks + r.seq_chunk + 2 * r.oCC + r.gb + 2 * r.qn + r.rr;
}

size_t bwd_ws(const gdn_problem* p) {
  const Regions r = regions(p);
  return r.oDD + r.oCD;  // dS^T and A per chunk
}

// Saved by the forward: the chunk table, then S^T, Delta, T, M per chunk and value head
// and the gate record.
size_t saved_bytes(const gdn_problem* p) {
  const Regions r = regions(p);
  return r.chunks + r.seq_chunk + r.oDD + r.oCD + 2 * r.oCC + r.gb + 2 * r.qn + r.rr;
}

// The saved-state layout (with_states) or the forward-only workspace layout (without the
// chunk-start states and Delta: sv_S and sv_D stay null, and the forward then saves neither).
void carve_saved(gdn::Prob& P, const Regions& r, void* saved, bool with_states = true) {
  char* b = static_cast<char*>(saved);
  P.chunks = reinterpret_cast<gdn::ChunkInfo*>(b);
  b += r.chunks;
  P.seq_chunk = reinterpret_cast<int*>(b);
  P.seq_order = P.seq_chunk + P.N + 1;
  b += r.seq_chunk;
  if (with_states) {
    P.sv_S = b;
    b += r.oDD;
    P.sv_D = b;
    b += r.oCD;
  }
  P.sv_T = b;
  b += r.oCC;
  P.sv_M = b;
  b += r.oCC;
  P.sv_gb = reinterpret_cast<float*>(b);
  b += r.gb;
  if (r.qn) {
    P.sv_qn = b;
    b += r.qn;
    P.sv_kn = b;
    b += r.qn;
    P.sv_r = reinterpret_cast<float*>(b);
  }
}

// The q and k rows the chunk kernels read: the normalised copies when prep writes them.
void set_qk_use(gdn::Prob& P) {
  const int64_t w = (int64_t)P.Hk * P.D;
  P.qu = P.sv_qn ? P.sv_qn : P.q;
  P.qu_rs = P.sv_qn ? w : P.q_rs;
  P.ku = P.sv_kn ? P.sv_kn : P.k;
  P.ku_rs = P.sv_kn ? w : P.k_rs;
}


// Kernels address one chunk of rows with 32-bit byte offsets: chunk * rs * esize < 2^31.
constexpr int64_t kMaxChunkSpan = (int64_t)1 << 31;

gdn_status check_view(const void* ptr, int64_t rs, int64_t width, int esize, int64_t T_total, int chunk) {
  if (T_total == 0) return GDN_OK;
  if (!ptr) return GDN_EINVAL;
  if (rs < width) return GDN_EINVAL;
  if ((int64_t)chunk * rs * esize >= kMaxChunkSpan) return GDN_EINVAL;
  if (!aligned(ptr, 16) || ((size_t)rs * esize) % 16) return GDN_EALIGN;
  return GDN_OK;
}

gdn_status check_f32(const void* ptr, bool required, size_t align = 4) {
  if (!ptr) return required ? GDN_EINVAL : GDN_OK;
  return aligned(ptr, align) ? GDN_OK : GDN_EALIGN;
}

#define GDN_TRY(x)                   \
  do {                               \
    const gdn_status s_ = (x);       \
    if (s_ != GDN_OK) return s_;     \
  } while (0)

struct Carver {
  char* base;
  size_t off = 0;
  template <typename T> T* take(size_t bytes) {
    T* r = reinterpret_cast<T*>(reinterpret_cast<void*>(base + off));
    off += bytes;
    return r;
  }
};

void fill_common(gdn::Prob& P, const gdn_problem* p) {
  P = gdn::Prob{};
  P.N = p->N;
  P.Hk = p->Hk;
  P.Hv = p->Hv;
  P.r = p->Hv / p->Hk;
  P.D = p->Dk;
  P.C = p->chunk;
  P.nc_max = (int)chunk_bound(p);
  P.T = p->cu_seqlens ? 0 : p->T;
  P.T_total = p->T_total;
  P.scale = p->scale;
  P.cu = p->cu_seqlens;
  P.a_log = p->a_log;
  P.dt_bias = p->dt_bias;
}

gdn_status conv_common(const gdn_conv_problem* p, const void* x, int64_t x_rs, const float* w, gdn::ConvArgs& a) {
  if (!p) return GDN_EINVAL;
  if (p->N < 0 || p->T_total < 0 || p->channels <= 0 || p->channels % 8) return GDN_EINVAL;
  if (p->kernel_size < 1 || p->kernel_size > 4) return GDN_EUNSUPPORTED;
  if (p->dtype != GDN_F32 && p->dtype != GDN_BF16) return GDN_EUNSUPPORTED;
  if (!p->cu_seqlens) {
    if (p->T < 0 || (int64_t)p->N * p->T != p->T_total) return GDN_EINVAL;
  } else if (p->N == 0 && p->T_total != 0) {
    return GDN_EINVAL;
  }
  if (p->channels / 8 > 65535LL * 256 || p->T_total > INT32_MAX) return GDN_EINVAL;  // grid limits
  if (p->cu_seqlens && !aligned(p->cu_seqlens, 4)) return GDN_EALIGN;
  const int es = p->dtype == GDN_BF16 ? 2 : 4;
  GDN_TRY(check_view(x, x_rs, p->channels, es, p->T_total, 1));
  GDN_TRY(check_f32(w, p->T_total > 0));
  a = gdn::ConvArgs{};
  a.N = p->N;
  a.T = p->cu_seqlens ? 0 : p->T;
  a.ch = p->channels;
  a.K = p->kernel_size;
  a.rows = p->T_total;
  a.cu = p->cu_seqlens;
  a.w = w;
  a.x = x;
  a.x_rs = x_rs;
  return GDN_OK;
}

// gdn_fwd's checks of everything but the saved buffer and the workspace.
gdn_status check_fwd_views(const gdn_problem* p, const void* q, int64_t q_rs, const void* k, int64_t k_rs,
                           const void* v, int64_t v_rs, const float* g, const float* beta, const float* S0,
                           const void* o, int64_t o_rs, const float* S_T) {
  GDN_TRY(check_problem(p));
  const int es = p->dtype == GDN_BF16 ? 2 : 4;
  const int64_t qkw = (int64_t)p->Hk * p->Dk, vw = (int64_t)p->Hv * p->Dv;
  GDN_TRY(check_view(q, q_rs, qkw, es, p->T_total, p->chunk));
  GDN_TRY(check_view(k, k_rs, qkw, es, p->T_total, p->chunk));
  GDN_TRY(check_view(v, v_rs, vw, es, p->T_total, p->chunk));
  GDN_TRY(check_view(o, o_rs, vw, es, p->T_total, p->chunk));
  GDN_TRY(check_f32(g, p->T_total > 0));
  GDN_TRY(check_f32(beta, p->T_total > 0));
  GDN_TRY(check_f32(S0, false, 16));
  GDN_TRY(check_f32(S_T, false, 16));
  if (p->cu_seqlens && !aligned(p->cu_seqlens, 4)) return GDN_EALIGN;
  return GDN_OK;
}

gdn_status fwd_launch(const gdn_problem* p, const void* q, int64_t q_rs, const void* k, int64_t k_rs,
                      const void* v, int64_t v_rs, const float* g, const float* beta, const float* S0, void* o,
                      int64_t o_rs, float* S_T, void* chunk_states, void* workspace, void* stream) {
  gdn::Prob P;
  fill_common(P, p);
  P.q = q; P.q_rs = q_rs; P.k = k; P.k_rs = k_rs; P.v = v; P.v_rs = v_rs;
  P.g = g; P.beta = beta; P.S0 = S0;
  P.o = o; P.o_rs = o_rs; P.ST = S_T;
  const Regions r = regions(p);
  if (chunk_states) carve_saved(P, r, chunk_states);
  else carve_saved(P, r, workspace, false);
  set_qk_use(P);
  const hipError_t e = gdn::launch_forward(P, p->dtype, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_OK : GDN_EHIP;
}

}  // namespace

extern "C" {

size_t gdn_fwd_workspace_bytes(const gdn_problem* p) { return check_problem(p) == GDN_OK ? fwd_ws(p) : 0; }

size_t gdn_bwd_workspace_bytes(const gdn_problem* p) { return check_problem(p) == GDN_OK ? bwd_ws(p) : 0; }

size_t gdn_chunk_state_bytes(const gdn_problem* p) { return check_problem(p) == GDN_OK ? saved_bytes(p) : 0; }

gdn_status gdn_fwd(const gdn_problem* p, const void* q, int64_t q_rs, const void* k, int64_t k_rs,
                   const void* v, int64_t v_rs, const float* g, const float* beta, const float* S0, void* o,
                   int64_t o_rs, float* S_T, void* chunk_states, void* workspace, size_t workspace_bytes,
                   void* stream) {
  GDN_TRY(check_fwd_views(p, q, q_rs, k, k_rs, v, v_rs, g, beta, S0, o, o_rs, S_T));
  if (p->N == 0) return GDN_OK;
  if (chunk_states) {
    if (!aligned(chunk_states, 16)) return GDN_EALIGN;  // the workspace is not used
  } else {
    if (!workspace || workspace_bytes < fwd_ws(p)) return GDN_EWORKSPACE;
    if (!aligned(workspace, kAlign)) return GDN_EALIGN;
  }
  return fwd_launch(p, q, q_rs, k, k_rs, v, v_rs, g, beta, S0, o, o_rs, S_T, chunk_states, workspace, stream);
}

gdn_status gdn_fwd_noalloc(const gdn_problem* p, const void* q, int64_t q_rs, const void* k, int64_t k_rs,
                           const void* v, int64_t v_rs, const float* g, const float* beta, const float* S0,
                           void* o, int64_t o_rs, float* S_T, void* stream) {
  GDN_TRY(check_fwd_views(p, q, q_rs, k, k_rs, v, v_rs, g, beta, S0, o, o_rs, S_T));
  if (fwd_ws(p) > GDN_NOALLOC_SCRATCH_BYTES) return GDN_EWORKSPACE;
  if (p->N == 0) return GDN_OK;
  void* ws = gdn::noalloc_scratch();
  if (!ws) return GDN_EHIP;
  return fwd_launch(p, q, q_rs, k, k_rs, v, v_rs, g, beta, S0, o, o_rs, S_T, nullptr, ws, stream);
}

gdn_status gdn_bwd(const gdn_problem* p, const void* q, int64_t q_rs, const void* k, int64_t k_rs,
                   const void* v, int64_t v_rs, const float* g, const float* beta, const float* S0,
                   const void* chunk_states, const void* dO, int64_t dO_rs, const float* dS_T, void* dq,
                   int64_t dq_rs, void* dk, int64_t dk_rs, void* dv, int64_t dv_rs, float* dg, float* dbeta,
                   float* dS0, void* workspace, size_t workspace_bytes, void* stream) {
  GDN_TRY(check_problem(p));
  const int es = p->dtype == GDN_BF16 ? 2 : 4;
  const int64_t qkw = (int64_t)p->Hk * p->Dk, vw = (int64_t)p->Hv * p->Dv;
  GDN_TRY(check_view(q, q_rs, qkw, es, p->T_total, p->chunk));
  GDN_TRY(check_view(k, k_rs, qkw, es, p->T_total, p->chunk));
  GDN_TRY(check_view(v, v_rs, vw, es, p->T_total, p->chunk));
  GDN_TRY(check_view(dO, dO_rs, vw, es, p->T_total, p->chunk));
  GDN_TRY(check_view(dq, dq_rs, qkw, es, p->T_total, p->chunk));
  GDN_TRY(check_view(dk, dk_rs, qkw, es, p->T_total, p->chunk));
  GDN_TRY(check_view(dv, dv_rs, vw, es, p->T_total, p->chunk));
  GDN_TRY(check_f32(g, p->T_total > 0));
  GDN_TRY(check_f32(beta, p->T_total > 0));
  GDN_TRY(check_f32(dg, p->T_total > 0));
  GDN_TRY(check_f32(dbeta, p->T_total > 0));
  GDN_TRY(check_f32(S0, false, 16));
  GDN_TRY(check_f32(dS_T, false, 16));
  GDN_TRY(check_f32(dS0, false, 16));
  if (p->N == 0) return GDN_OK;
  if (p->cu_seqlens && !aligned(p->cu_seqlens, 4)) return GDN_EALIGN;
  if (!chunk_states) return GDN_EINVAL;
  if (!aligned(chunk_states, 16)) return GDN_EALIGN;
  const size_t need = bwd_ws(p);
  if (!workspace || workspace_bytes < need) return GDN_EWORKSPACE;
  if (!aligned(workspace, kAlign)) return GDN_EALIGN;

  gdn::Prob P;
  fill_common(P, p);
  P.q = q; P.q_rs = q_rs; P.k = k; P.k_rs = k_rs; P.v = v; P.v_rs = v_rs;
  P.g = g; P.beta = beta; P.S0 = S0;
  P.dO = dO; P.dO_rs = dO_rs; P.dST = dS_T;
  P.dq = dq; P.dq_rs = dq_rs; P.dk = dk; P.dk_rs = dk_rs; P.dv = dv; P.dv_rs = dv_rs;
  P.dg = dg; P.dbeta = dbeta; P.dS0 = dS0;
  const Regions r = regions(p);
  carve_saved(P, r, const_cast<void*>(chunk_states));  // the chunk table comes with it
  set_qk_use(P);
  Carver cv{static_cast<char*>(workspace)};
  P.ws_dS = cv.take<void>(r.oDD);
  P.ws_A = cv.take<void>(r.oCD);
  const hipError_t e = gdn::launch_backward(P, p->dtype, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_OK : GDN_EHIP;
}

gdn_status gdn_decode(const gdn_problem* p, const void* q, int64_t q_rs, const void* k, int64_t k_rs,
                      const void* v, int64_t v_rs, const float* g, const float* beta, float* state,
                      int32_t n_slots, const int32_t* slot_idx, void* o, int64_t o_rs, void* stream) {
  if (!p) return GDN_EINVAL;
  if (p->N < 0 || p->Hk <= 0 || p->Hv <= 0 || p->Hv % p->Hk) return GDN_EINVAL;
  if (p->Dk <= 0 || p->Dv <= 0) return GDN_EINVAL;
  if (p->dtype != GDN_F32 && p->dtype != GDN_BF16) return GDN_EUNSUPPORTED;
  if (p->Dk != p->Dv) return GDN_EUNSUPPORTED;
  if (p->Dk != 16 && p->Dk != 32 && p->Dk != 64 && p->Dk != 128) return GDN_EUNSUPPORTED;
  if (!std::isfinite(p->scale)) return GDN_EINVAL;
  if ((p->a_log == nullptr) != (p->dt_bias == nullptr)) return GDN_EINVAL;
  if (!aligned(p->a_log, 4) || !aligned(p->dt_bias, 4)) return GDN_EALIGN;
  // one token per row: T = 1, T_total = N, no cu_seqlens (the chunk length is not used)
  if (p->cu_seqlens || p->T != 1 || p->T_total != p->N) return GDN_EINVAL;
  if ((int64_t)p->N * p->Hv > INT32_MAX) return GDN_EINVAL;
  if (n_slots < 0 || (!slot_idx && n_slots < p->N)) return GDN_EINVAL;
  const int es = p->dtype == GDN_BF16 ? 2 : 4;
  const int64_t qkw = (int64_t)p->Hk * p->Dk, vw = (int64_t)p->Hv * p->Dv;
  GDN_TRY(check_view(q, q_rs, qkw, es, p->N, 1));
  GDN_TRY(check_view(k, k_rs, qkw, es, p->N, 1));
  GDN_TRY(check_view(v, v_rs, vw, es, p->N, 1));
  GDN_TRY(check_view(o, o_rs, vw, es, p->N, 1));
  GDN_TRY(check_f32(g, p->N > 0));
  GDN_TRY(check_f32(beta, p->N > 0));
  GDN_TRY(check_f32(state, p->N > 0, 16));
  GDN_TRY(check_f32(reinterpret_cast<const float*>(slot_idx), false));
  if (p->N == 0) return GDN_OK;

  gdn::DecArgs a{};
  a.N = p->N;
  a.Hv = p->Hv;
  a.r = p->Hv / p->Hk;
  a.D = p->Dk;
  a.n_slots = n_slots;
  a.scale = p->scale;
  a.q = q; a.k = k; a.v = v;
  a.q_rs = q_rs; a.k_rs = k_rs; a.v_rs = v_rs; a.o_rs = o_rs;
  a.g = g; a.beta = beta;
  a.a_log = p->a_log; a.dt_bias = p->dt_bias;
  a.l2 = p->qk_l2norm != 0;
  a.state = state;
  a.idx = slot_idx;
  a.o = o;
  const hipError_t e = gdn::launch_decode(a, p->dtype, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_OK : GDN_EHIP;
}

gdn_status gdn_conv1d_silu_fwd(const gdn_conv_problem* p, const void* x, int64_t x_rs, const float* w, void* y,
                               int64_t y_rs, void* stream) {
  gdn::ConvArgs a;
  GDN_TRY(conv_common(p, x, x_rs, w, a));
  const int es = p->dtype == GDN_BF16 ? 2 : 4;
  GDN_TRY(check_view(y, y_rs, p->channels, es, p->T_total, 1));
  a.y = y;
  a.y_rs = y_rs;
  const hipError_t e = gdn::launch_conv(a, p->dtype, false, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_OK : GDN_EHIP;
}

gdn_status gdn_conv1d_silu_bwd(const gdn_conv_problem* p, const void* x, int64_t x_rs, const float* w,
                               const void* dy, int64_t dy_rs, void* dx, int64_t dx_rs, void* stream) {
  gdn::ConvArgs a;
  GDN_TRY(conv_common(p, x, x_rs, w, a));
  const int es = p->dtype == GDN_BF16 ? 2 : 4;
  GDN_TRY(check_view(dy, dy_rs, p->channels, es, p->T_total, 1));
  GDN_TRY(check_view(dx, dx_rs, p->channels, es, p->T_total, 1));
  a.dy = dy;
  a.dy_rs = dy_rs;
  a.dx = dx;
  a.dx_rs = dx_rs;
  const hipError_t e = gdn::launch_conv(a, p->dtype, true, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_OK : GDN_EHIP;
}

const char* gdn_strerror(int status) {
  switch (status) {
    case GDN_OK: return "success";
    case GDN_EINVAL: return "invalid argument (size, count, stride or missing pointer)";
    case GDN_EUNSUPPORTED: return "unsupported head size, chunk length or dtype";
    case GDN_EALIGN: return "misaligned pointer or row stride";
    case GDN_EWORKSPACE: return "workspace missing or too small";
    case GDN_EHIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

}  // extern "C"
