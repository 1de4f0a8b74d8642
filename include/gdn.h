/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated delta-net recurrence: forward and
 * reverse-mode backward.
 *
 * The operation (lattice-inference 0.6.0, docs.rs source page of
 * src/attention/gdn_backward.rs, module doc "Forward recap"), per sequence and per
 * value head h, with q and k read from key head kh = h / (Hv / Hk):
 *
 *   kv_t    = S_{t-1}^T k_t                    (retrieval from the pre-decay state)
 *   delta_t = beta_t * (v_t - g_t * kv_t)
 *   S_t     = g_t * S_{t-1} + k_t (x) delta_t    (S is Dk x Dv, stored key-major)
 *   o_t     = scale * S_t^T q_t
 *
 * starting from S_{-1} = S0 (zero when S0 is NULL). The backward is the same page's
 * gdn_backward steps 4a-4d run in reverse time with the state adjoint dS carried
 * across tokens, starting from dS_T (zero when NULL), and returns dq, dk, dv, dg,
 * dbeta and dS0. dq and dk of a key head sum the contributions of every value head
 * that reads it (the cross-head accumulation of page 1, the llama.cpp fork's
 * "delta-net backward at the shape the 27B emits"); the sum is formed in float32 in
 * ascending head order and rounded once, without atomics, so results are
 * bit-reproducible run to run.
 *
 * Memory. Every pointer is a DEVICE pointer unless noted. The caller owns all memory;
 * the library never allocates, never frees and never synchronises the stream: calls
 * only enqueue kernels on `stream` (a hipStream_t; NULL = the default stream).
 * Buffers written by a call must not be read or written by other work until that
 * work is ordered after the call on the stream.
 *
 * Layout. A "row" is one token. q, k, v, o, dO, dq, dk, dv are row-strided views:
 * element (t, head, d) of q is at q[t * q_rs + head * Dk + d]; row strides are in
 * elements. So q, k and v may be column slices of one packed projection row
 * [q heads | k heads | v heads], and dq, dk, dv may be the same slices of a packed
 * gradient buffer. g, beta, dg, dbeta are contiguous [T_total][Hv] float32;
 * S0, S_T, dS_T, dS0 are contiguous [N][Hv][Dk][Dv] float32.
 *
 * Errors. Arguments are checked on the host before anything is enqueued; a negative
 * status means nothing was enqueued and nothing written. Device-side cu_seqlens are
 * not readable from the host without a synchronisation; their values are clamped
 * into [0, T_total] on the device, so a malformed table yields wrong results but
 * never an out-of-bounds access.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_EINVAL = -1,       /* bad size, count, stride or missing required pointer; also more
                            than 2^31 - 1 (chunk, key head) pairs */
  GDN_EUNSUPPORTED = -2, /* head size / chunk / dtype combination not built */
  GDN_EALIGN = -3,       /* pointer or row stride not aligned as required */
  GDN_EWORKSPACE = -4,   /* workspace missing or smaller than the size query returns */
  GDN_EHIP = -5          /* a kernel launch failed (hipGetLastError) */
} gdn_status;

typedef enum {
  GDN_F32 = 0, /* q, k, v, o, dO, dq, dk, dv are float32 */
  GDN_BF16 = 1 /* ... are bfloat16; arithmetic and the state stay float32 */
} gdn_dtype;

typedef struct {
  int32_t N;        /* number of sequences (>= 0) */
  int32_t T;        /* tokens per sequence when cu_seqlens == NULL; ignored otherwise */
  int64_t T_total;  /* total rows: N * T, or cu_seqlens[N] (host-known) */
  const int32_t* cu_seqlens; /* DEVICE int32 [N + 1]: cu[0] = 0, nondecreasing, cu[N] = T_total;
                                NULL = N sequences of T tokens. Zero-length sequences allowed:
                                their S_T is S0 and their dS0 is dS_T. */
  int32_t Hk, Hv;   /* key heads and value heads; Hv % Hk == 0, v_repeat = Hv / Hk */
  int32_t Dk, Dv;   /* head sizes; Dk == Dv in {16, 32, 64, 128} is required */
  int32_t chunk;    /* chunk length of the chunked algorithm: 16 or 64 (results agree
                       up to rounding) */
  float scale;      /* output scale, normally 1 / sqrt(Dk) */
  int32_t dtype;    /* gdn_dtype */
  /* Gate inputs. Both NULL: the g and beta arguments are the decay gate g (0 < g <= 1) and
   * beta themselves. Both set (DEVICE float32 [Hv] each): the layer's gate chain is fused
   * into the kernels (the lattice-inference gdn_backward.rs page, "sigmoid(beta)" and
   * "decay gate g per value-head"): the g argument holds alpha and the beta argument
   * beta_raw ([T_total][Hv] float32 each), and
   *   g = exp(-exp(a_log[h]) softplus(alpha + dt_bias[h])),  beta = sigmoid(beta_raw);
   * gdn_bwd's dg and dbeta outputs then hold d alpha and d beta_raw (the page's steps 4e
   * and 4h). gdn_decode follows the same rule. One set without the other: GDN_EINVAL. */
  const float* a_log;
  const float* dt_bias;
  /* Nonzero: q and k are the layer's raw projections and the kernels L2-normalise every head
   * row themselves, x_hat = x / sqrt(sum x^2 + 1e-6) (the gdn_backward.rs page, "L2-normalize
   * q, k", with the epsilon inside the square root), before any use; gdn_bwd's dq and dk are
   * then the gradients with respect to the raw q and k (the page's step 4f). The normalised
   * rows are kept with the chunk states (gdn_chunk_state_bytes grows by 2 T_total Hk Dk
   * elements and 8 T_total Hk bytes). Zero: q and k are used as given. */
  int32_t qk_l2norm;
} gdn_problem;

/* Bytes of device workspace gdn_fwd / gdn_bwd need for this problem (0 on invalid
 * problem). The workspace is scratch: its contents on entry are ignored, and it must be
 * 256-byte aligned. gdn_fwd needs it only for a forward-only call (chunk_states NULL):
 * then it holds the per-chunk factors the forward's kernels pass to one another; a
 * forward that saves chunk states keeps them there instead and ignores its workspace
 * arguments (NULL, 0 is fine). */
size_t gdn_fwd_workspace_bytes(const gdn_problem* p);
size_t gdn_bwd_workspace_bytes(const gdn_problem* p);

/* Bytes of the saved-state buffer gdn_fwd writes and gdn_bwd reads: the chunk table of
 * the problem's sequences and, per chunk, the state at its start and the other chunk
 * factors (layout internal to the library). */
size_t gdn_chunk_state_bytes(const gdn_problem* p);

/*
 * Forward: the op that returns (o, S_T) (page 2, the dormouse review log, the fused op's
 * (o, s) result; page 3's "Forward recap"). Reads q, k [rows][Hk*Dk], v [rows][Hv*Dv]
 * (dtype), g, beta [T_total][Hv] (float32; 0 < g <= 1 is required by the chunked form: it
 * works with log g), S0 (float32 or NULL = zeros). Writes o [rows][Hv*Dv] (dtype, row
 * stride o_rs) and S_T (or NULL to skip).
 * chunk_states: gdn_chunk_state_bytes bytes (16-byte aligned) to keep what gdn_bwd needs
 * (keep it unchanged for gdn_bwd), or NULL for a forward-only call, which saves nothing
 * and instead needs a workspace of gdn_fwd_workspace_bytes (GDN_EWORKSPACE otherwise).
 * Alignment: q, k, v, o and the row strides times the element size must be
 * multiples of 16 bytes; S0, S_T, dS_T, dS0 need 16-byte alignment, g, beta, dg,
 * dbeta 4-byte alignment (the same rules hold for gdn_bwd).
 */
gdn_status gdn_fwd(const gdn_problem* p,
                   const void* q, int64_t q_rs, const void* k, int64_t k_rs,
                   const void* v, int64_t v_rs, const float* g, const float* beta,
                   const float* S0, void* o, int64_t o_rs, float* S_T, void* chunk_states,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward-only without allocation, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. It is
 * gdn_fwd with chunk_states NULL whose workspace is a fixed scratch array inside the library,
 * GDN_NOALLOC_SCRATCH_BYTES long, one per GPU, which each GPU the library runs on holds until
 * the process ends; the array of the current device (hipGetDevice) is used, so make the
 * stream's device current. The caller passes the inputs and outputs as for gdn_fwd. A
 * problem whose gdn_fwd_workspace_bytes exceeds the array returns GDN_EWORKSPACE (about
 * 3,600 (chunk, value head) pairs: some 4,800 tokens at 48 value heads and chunk 64). Every
 * call on a GPU shares that GPU's array and leaves its own contents there; nothing in it
 * needs to start at any particular value, and calls that overlap on one GPU (on different
 * streams, or from several threads without ordering) race. The first call on a device looks
 * the array's address up (hipGetSymbolAddress); no call allocates or frees anything.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gdn_status gdn_fwd_noalloc(const gdn_problem* p,
                           const void* q, int64_t q_rs, const void* k, int64_t k_rs,
                           const void* v, int64_t v_rs, const float* g, const float* beta,
                           const float* S0, void* o, int64_t o_rs, float* S_T, void* stream);

/*
 * Backward. q, k, v, g, beta, S0 and chunk_states must be those of the forward call
 * on the same problem (same sequences: the chunk table is read from chunk_states). dO [rows][Hv*Dv] (dtype), dS_T (float32 or NULL = zeros).
 * Writes dq, dk [rows][Hk*Dk] and dv [rows][Hv*Dv] (dtype, overwritten, each with
 * its own row stride; they may be disjoint slices of one packed buffer), dg and
 * dbeta [T_total][Hv] float32, dS0 (float32, or NULL to skip). dg is the derivative
 * with respect to the gate value g itself.
 */
gdn_status gdn_bwd(const gdn_problem* p,
                   const void* q, int64_t q_rs, const void* k, int64_t k_rs,
                   const void* v, int64_t v_rs, const float* g, const float* beta,
                   const float* S0, const void* chunk_states,
                   const void* dO, int64_t dO_rs, const float* dS_T,
                   void* dq, int64_t dq_rs, void* dk, int64_t dk_rs, void* dv, int64_t dv_rs,
                   float* dg, float* dbeta, float* dS0,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode: one step of the recurrence for each of p->N rows (one token per sequence),
 * the per-token form of the lattice-inference gdn_backward.rs page, module doc "Forward
 * recap" (the pages' inference path, gated_delta_net_step_fused, runs it token by token):
 * for row n and value head h, with q, k of key head h / (Hv / Hk) and S the state of the
 * row's slot,
 *   kv = S^T k,  delta = beta (v - g kv),  S <- g S + k delta^T,  o = scale S^T q
 * (o from the updated S). The problem holds one token per row: p->T == 1,
 * p->T_total == p->N, p->cu_seqlens == NULL; p->chunk is not used.
 * q, k [N rows][Hk*Dk], v [N rows][Hv*Dv] (dtype, row strides in elements, same
 * alignment rules as gdn_fwd); g, beta [N][Hv] float32 (the gate value g itself).
 * state: float32 [n_slots][Hv][Dk][Dv] (key-major), 16-byte aligned, read and
 * overwritten in place. slot_idx: device int32 [N], the slot of each row, or NULL for
 * row n -> slot n (then n_slots >= N is required). A row whose slot lies outside
 * [0, n_slots) is skipped: its o row and every state are left untouched. Two rows with
 * the same slot race (the result is undefined). o [N rows][Hv*Dv] (dtype). No
 * workspace, no allocation; the call is enqueued on stream.
 */
gdn_status gdn_decode(const gdn_problem* p,
                      const void* q, int64_t q_rs, const void* k, int64_t k_rs,
                      const void* v, int64_t v_rs, const float* g, const float* beta,
                      float* state, int32_t n_slots, const int32_t* slot_idx,
                      void* o, int64_t o_rs, void* stream);

/*
 * Causal depthwise conv1d + SiLU over rows of `channels` values (the layer's packed q/k/v
 * projection: channels = 2 Hk Dk + Hv Dv), the step before the recurrence, as the
 * lattice-inference gdn_backward.rs page computes it (conv1d_silu_fwd in gdn_forward_save;
 * step 5 of gdn_backward, "Backward through conv1d + SiLU"). For channel c and row t of a
 * sequence, with w [channels][kernel_size] float32 and the rows before the sequence's first
 * taken as zero (each sequence starts with an empty conv buffer):
 *   pre[t] = sum_{j < K} w[c][j] x[t - (K - 1) + j],   y[t] = pre[t] sigmoid(pre[t])
 * Backward (input gradient only; the pages keep the conv weights fixed):
 *   dpre[t] = dy[t] sigmoid(pre[t]) (1 + pre[t] (1 - sigmoid(pre[t])))
 *   dx[t] = sum_{l < K} w[c][K - 1 - l] dpre[t + l]   (rows t + l of the same sequence)
 * Sequences as in gdn_problem (N equal-length sequences of T rows, or cu_seqlens).
 * channels: a positive multiple of 8; kernel_size 1..4 (GDN_EUNSUPPORTED otherwise).
 * x, y, dy, dx: [T_total rows][channels] in dtype, row strides in elements, 16-byte
 * aligned rows (as for gdn_fwd); y must not overlap x, dx must not overlap x or dy.
 * No workspace, no allocation; enqueued on stream.
 */
typedef struct {
  int32_t N;                  /* sequences */
  int32_t T;                  /* rows per sequence when cu_seqlens is NULL */
  int64_t T_total;            /* rows */
  const int32_t* cu_seqlens;  /* device int32 [N + 1], or NULL */
  int32_t channels;           /* values per row */
  int32_t kernel_size;        /* K */
  int32_t dtype;              /* gdn_dtype of x, y, dy, dx */
} gdn_conv_problem;

gdn_status gdn_conv1d_silu_fwd(const gdn_conv_problem* p, const void* x, int64_t x_rs, const float* w,
                               void* y, int64_t y_rs, void* stream);
gdn_status gdn_conv1d_silu_bwd(const gdn_conv_problem* p, const void* x, int64_t x_rs, const float* w,
                               const void* dy, int64_t dy_rs, void* dx, int64_t dx_rs, void* stream);

/*
 * Per-kernel timing for benchmarks. While enabled (process-wide), every kernel that
 * gdn_fwd / gdn_bwd enqueue is bracketed by two HIP events recorded on the call's
 * stream (the events are created by the library on first use and reused; no device
 * memory is allocated). gdn_trace_collect waits for the recorded events, returns up
 * to max per-kernel totals (kernel name, summed elapsed milliseconds, launch count)
 * and resets them. Names are static strings owned by the library. Returns the number
 * of entries written.
 */
typedef struct {
  const char* name;
  double total_ms;
  int64_t launches;
} gdn_trace_entry;
gdn_status gdn_trace_enable(int on);
int gdn_trace_collect(gdn_trace_entry* out, int max);

/* Static string for a status code. */
const char* gdn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
