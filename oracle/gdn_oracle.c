/*
 * gdn_oracle.c -- plain, sequential, float64 CPU oracle of the gated delta-net
 * recurrence and its reverse-mode backward.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it. It shares no code, header, table or helper with the HIP path.
 *
 * What it computes (lattice-inference 0.6.0, docs.rs source page of
 * src/attention/gdn_backward.rs: module doc "Forward recap" and the per
 * value-head recurrence of gdn_forward_save):
 *
 *   kv_t    = S_{t-1}^T k_t                  retrieval from the pre-decay state
 *   delta_t = beta_t * (v_t - g_t * kv_t)
 *   S_t     = g_t * S_{t-1} + k_t (x) delta_t  (outer product, state key-major)
 *   o_t     = scale * S_t^T q_t
 *
 * per sequence and per value head h, with q and k taken from key head
 * h / (Hv/Hk) (same page: "key-head k_head = h / ratio"). The state is stored
 * key-major, S[i*Dv + j], i = key index, j = value index, as on that page.
 *
 * The backward is the reverse-mode adjoint of that recurrence, derived here from
 * its Householder form (see run_backward_head), run in reverse time with the state
 * adjoint carried across tokens. The page's backward starts from S = 0 and dS = 0;
 * here the initial state S0 and the incoming adjoint dS_T may be non-zero (NULL
 * means zero), and dS0 is returned. dq and dk of a key head are
 * the sums of the per-value-head contributions over the value heads that read
 * it, added in ascending head order (step 4g of that page; and page 1, the
 * llama.cpp fork's "delta-net backward at the shape the 27B emits", which
 * calls this the cross-head dq/dk accumulation).
 *
 * The backward needs S_{t-1} at every step. Storing every state would cost
 * T*Dk*Dv doubles per head, so the forward is re-run keeping a copy of S every
 * SEG tokens, and each segment's states are recomputed, in the same plain
 * arithmetic, just before that segment is walked backwards.
 *
 * Layout of every array: canonical contiguous float64.
 *   q, k [T_total][Hk][Dk]    v, o, dO, dv [T_total][Hv][Dv]
 *   g, beta, dg, dbeta [T_total][Hv]    S0, S_T, dS_T, dS0 [N][Hv][Dk][Dv]
 * cu[N+1] (host int64) holds the sequence boundaries; cu[0] = 0.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC -pthread
 * (no contraction: every product and sum is rounded as written).
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SEG 64

typedef struct {
  int N, Hk, Hv, Dk, Dv;
  const int64_t* cu;
  double scale;
  const double *q, *k, *v, *g, *beta, *S0, *dO, *dST;
  double *o, *ST, *dq, *dk, *dv, *dg, *dbeta, *dS0;
  int backward;
  /* work distribution: item = n * Hk + kh */
  int next_item;
  pthread_mutex_t lock;
  int failed;
} job_t;

static int take_item(job_t* J) {
  pthread_mutex_lock(&J->lock);
  int it = J->next_item++;
  pthread_mutex_unlock(&J->lock);
  return it;
}

/* Key head read by value head h: the block map h / ratio. */
static int key_head_of(int h, int Hk, int Hv) {
#if defined(ORACLE_PLANT) && ORACLE_PLANT == 1
  /* planted mistake for the falsification test: modulo map */
  return h % Hk;
#else
  return h / (Hv / Hk);
#endif
}

/* One forward token step on state S (Dk x Dv, key-major). Writes kv and delta. */
static void step_forward(double* S, const double* kt, const double* vt, double gt, double bt,
                         double* kv, double* delta, int Dk, int Dv) {
  for (int j = 0; j < Dv; ++j) kv[j] = 0.0;
  for (int i = 0; i < Dk; ++i)
    for (int j = 0; j < Dv; ++j) kv[j] += S[i * Dv + j] * kt[i];
  for (int j = 0; j < Dv; ++j) delta[j] = bt * (vt[j] - gt * kv[j]);
  for (int i = 0; i < Dk; ++i)
    for (int j = 0; j < Dv; ++j) S[i * Dv + j] = gt * S[i * Dv + j] + kt[i] * delta[j];
}

static void run_forward_head(job_t* J, int n, int h, double* S, double* kv, double* delta) {
  const int Hk = J->Hk, Hv = J->Hv, Dk = J->Dk, Dv = J->Dv;
  const int kh = key_head_of(h, Hk, Hv);
  const size_t SS = (size_t)Dk * Dv;
  if (J->S0) memcpy(S, J->S0 + ((size_t)n * Hv + h) * SS, SS * sizeof(double));
  else memset(S, 0, SS * sizeof(double));
  for (int64_t t = J->cu[n]; t < J->cu[n + 1]; ++t) {
    const double* kt = J->k + ((size_t)t * Hk + kh) * Dk;
    const double* qt = J->q + ((size_t)t * Hk + kh) * Dk;
    const double* vt = J->v + ((size_t)t * Hv + h) * Dv;
    const double gt = J->g[(size_t)t * Hv + h];
    const double bt = J->beta[(size_t)t * Hv + h];
    step_forward(S, kt, vt, gt, bt, kv, delta, Dk, Dv);
    double* ot = J->o + ((size_t)t * Hv + h) * Dv;
    for (int j = 0; j < Dv; ++j) ot[j] = 0.0;
    for (int i = 0; i < Dk; ++i)
      for (int j = 0; j < Dv; ++j) ot[j] += S[i * Dv + j] * qt[i];
    for (int j = 0; j < Dv; ++j) ot[j] *= J->scale;
  }
  if (J->ST) memcpy(J->ST + ((size_t)n * Hv + h) * SS, S, SS * sizeof(double));
}

/*
 * Reverse-time backward of one (sequence, value head), as the adjoint of the recurrence
 * regrouped in its Householder form (the same map as the forward above):
 *
 *   S_t = g_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,    o_t = scale S_t^T q_t.
 *
 * Let A = dL/dS_t, the adjoint of the state after token t (o_t's own term included),
 * u = S_{t-1}^T k_t and w = A^T k_t (both Dv vectors). Differentiating the map term by term:
 *
 *   dq_t   = scale S_t dO_t                          (from o_t)
 *   dv_t   = beta_t w                                (from beta k v^T)
 *   dbeta  = w . (v_t - g_t u)                       (from -g beta k u^T + beta k v^T)
 *   dg     = <S_{t-1}, A> - beta_t (u . w)           (from g (I - beta k k^T) S_{t-1})
 *   dk_t   = beta_t A (v_t - g_t u) - g_t beta_t S_{t-1} w
 *            (k enters twice in -g beta k k^T S_{t-1}, once in beta k v^T)
 *   dL/dS_{t-1} = g_t (I - beta_t k_t k_t^T) A = g_t (A - beta_t k_t w^T)
 *
 * The adjoint starts from dS_T (zero when absent) and ends as dS0. dq and dk of this head
 * are added into those of its key head (the caller walks the heads of a group in
 * ascending order).
 */

/* States of tokens a .. b-1 of one segment, recomputed from the segment's checkpoint:
 * st[r] is the state before token a + r, st[b - a] the state after the last token. */
static void segment_states(job_t* J, int h, int kh, int64_t a, int64_t b, const double* ckpt, double* st,
                           double* kv, double* delta) {
  const int Hk = J->Hk, Hv = J->Hv, Dk = J->Dk, Dv = J->Dv;
  const size_t SS = (size_t)Dk * Dv;
  memcpy(st, ckpt, SS * sizeof(double));
  for (int64_t t = a; t < b; ++t) {
    double* next = st + (size_t)(t - a + 1) * SS;
    memcpy(next, st + (size_t)(t - a) * SS, SS * sizeof(double));
    step_forward(next, J->k + ((size_t)t * Hk + kh) * Dk, J->v + ((size_t)t * Hv + h) * Dv,
                 J->g[(size_t)t * Hv + h], J->beta[(size_t)t * Hv + h], kv, delta, Dk, Dv);
  }
}

/* One token of the adjoint: A holds dL/dS_t without o_t's term on entry and dL/dS_{t-1} on
 * return. Sp = S_{t-1}, Sn = S_t. u, w, r are Dv scratch vectors; dqh, dkh receive this
 * head's dq_t, dk_t. */
static void adjoint_token(job_t* J, int64_t t, int h, int kh, const double* Sp, const double* Sn, double* A,
                          double* u, double* w, double* r, double* dqh, double* dkh) {
  const int Hk = J->Hk, Hv = J->Hv, Dk = J->Dk, Dv = J->Dv;
  const double* k = J->k + ((size_t)t * Hk + kh) * Dk;
  const double* q = J->q + ((size_t)t * Hk + kh) * Dk;
  const double* v = J->v + ((size_t)t * Hv + h) * Dv;
  const double* dO = J->dO + ((size_t)t * Hv + h) * Dv;
  const double gt = J->g[(size_t)t * Hv + h], bt = J->beta[(size_t)t * Hv + h], sc = J->scale;

  /* o_t = scale S_t^T q: its adjoint joins A, and dq_t = scale S_t dO_t */
  for (int i = 0; i < Dk; ++i) {
    double s = 0.0;
    for (int j = 0; j < Dv; ++j) {
      A[i * Dv + j] += sc * q[i] * dO[j];
      s += Sn[i * Dv + j] * dO[j];
    }
#if defined(ORACLE_PLANT) && ORACLE_PLANT == 4
    dqh[i] = s; /* planted mistake: the scale of dq dropped */
#else
    dqh[i] = sc * s;
#endif
  }

  /* u = S_{t-1}^T k, w = A^T k, r = v - g u */
  for (int j = 0; j < Dv; ++j) u[j] = w[j] = 0.0;
  for (int i = 0; i < Dk; ++i)
    for (int j = 0; j < Dv; ++j) {
      u[j] += Sp[i * Dv + j] * k[i];
      w[j] += A[i * Dv + j] * k[i];
    }
  double uw = 0.0, wr = 0.0, SA = 0.0;
  for (int j = 0; j < Dv; ++j) {
    r[j] = v[j] - gt * u[j];
    uw += u[j] * w[j];
    wr += w[j] * r[j];
  }
  for (size_t ij = 0; ij < (size_t)Dk * Dv; ++ij) SA += Sp[ij] * A[ij];

  double* dv = J->dv + ((size_t)t * Hv + h) * Dv;
  for (int j = 0; j < Dv; ++j) dv[j] = bt * w[j];
  J->dbeta[(size_t)t * Hv + h] = wr;
#if defined(ORACLE_PLANT) && ORACLE_PLANT == 3
  J->dg[(size_t)t * Hv + h] = SA + bt * uw; /* planted mistake: sign of the k k^T term */
#else
  J->dg[(size_t)t * Hv + h] = SA - bt * uw;
#endif
  for (int i = 0; i < Dk; ++i) {
    double ar = 0.0, sw = 0.0;
    for (int j = 0; j < Dv; ++j) {
      ar += A[i * Dv + j] * r[j];
      sw += Sp[i * Dv + j] * w[j];
    }
#if defined(ORACLE_PLANT) && ORACLE_PLANT == 2
    dkh[i] = bt * ar; /* planted mistake: the k of k^T S_{t-1} (the retrieval) dropped */
    (void)sw;
#else
    dkh[i] = bt * ar - gt * bt * sw;
#endif
  }

  /* dL/dS_{t-1} = g (A - beta k w^T) */
  for (int i = 0; i < Dk; ++i)
    for (int j = 0; j < Dv; ++j) A[i * Dv + j] = gt * (A[i * Dv + j] - bt * k[i] * w[j]);
}

static void run_backward_head(job_t* J, int n, int h, double* ckpt, double* segS, double* dS,
                              double* kv, double* delta, double* u, double* w, double* dqh, double* dkh) {
  const int Hk = J->Hk, Hv = J->Hv, Dk = J->Dk, Dv = J->Dv;
  const int kh = key_head_of(h, Hk, Hv);
  const size_t SS = (size_t)Dk * Dv;
  const int64_t t0 = J->cu[n], t1 = J->cu[n + 1];
  const int64_t nseg = (t1 - t0 + SEG - 1) / SEG;

  /* a forward run keeping the state at the start of every segment of SEG tokens */
  double* S = segS;
  if (J->S0) memcpy(S, J->S0 + ((size_t)n * Hv + h) * SS, SS * sizeof(double));
  else memset(S, 0, SS * sizeof(double));
  for (int64_t s = 0; s < nseg; ++s) {
    memcpy(ckpt + (size_t)s * SS, S, SS * sizeof(double));
    const int64_t a = t0 + s * SEG, b = a + SEG < t1 ? a + SEG : t1;
    for (int64_t t = a; t < b; ++t)
      step_forward(S, J->k + ((size_t)t * Hk + kh) * Dk, J->v + ((size_t)t * Hv + h) * Dv,
                   J->g[(size_t)t * Hv + h], J->beta[(size_t)t * Hv + h], kv, delta, Dk, Dv);
  }

  if (J->dST) memcpy(dS, J->dST + ((size_t)n * Hv + h) * SS, SS * sizeof(double));
  else memset(dS, 0, SS * sizeof(double));
  for (int64_t s = nseg - 1; s >= 0; --s) {
    const int64_t a = t0 + s * SEG, b = a + SEG < t1 ? a + SEG : t1;
    segment_states(J, h, kh, a, b, ckpt + (size_t)s * SS, segS, kv, delta);
    for (int64_t t = b - 1; t >= a; --t) {
      adjoint_token(J, t, h, kh, segS + (size_t)(t - a) * SS, segS + (size_t)(t - a + 1) * SS, dS, u, w, kv,
                    dqh, dkh);
      double* dq = J->dq + ((size_t)t * Hk + kh) * Dk;
      double* dk = J->dk + ((size_t)t * Hk + kh) * Dk;
      for (int i = 0; i < Dk; ++i) {
        dq[i] += dqh[i];
        dk[i] += dkh[i];
      }
    }
  }
  if (J->dS0) memcpy(J->dS0 + ((size_t)n * Hv + h) * SS, dS, SS * sizeof(double));
}

static void* worker(void* arg) {
  job_t* J = (job_t*)arg;
  const int Dk = J->Dk, Dv = J->Dv, r = J->Hv / J->Hk;
  const size_t SS = (size_t)Dk * Dv;
  int64_t maxlen = 0;
  for (int n = 0; n < J->N; ++n)
    if (J->cu[n + 1] - J->cu[n] > maxlen) maxlen = J->cu[n + 1] - J->cu[n];
  const size_t nseg_max = (size_t)((maxlen + SEG - 1) / SEG) + 1;
  const int Dm = Dk > Dv ? Dk : Dv;
  double* S = (double*)malloc(SS * sizeof(double));
  double* ckpt = J->backward ? (double*)malloc(nseg_max * SS * sizeof(double)) : NULL;
  double* segS = J->backward ? (double*)malloc((SEG + 1) * SS * sizeof(double)) : NULL;
  double* dS = J->backward ? (double*)malloc(SS * sizeof(double)) : NULL;
  double* vec = (double*)malloc(6 * (size_t)Dm * sizeof(double));
  if (!S || !vec || (J->backward && (!ckpt || !segS || !dS))) {
    J->failed = 1;
    free(S); free(ckpt); free(segS); free(dS); free(vec);
    return NULL;
  }
  double *kv = vec, *delta = vec + Dm, *u = vec + 2 * Dm, *w = vec + 3 * Dm;
  double *dqh = vec + 4 * Dm, *dkh = vec + 5 * Dm;
  for (;;) {
    int it = take_item(J);
    if (it >= J->N * J->Hk) break;
    int n = it / J->Hk, kh = it % J->Hk;
    /* the value heads of key head kh, in ascending order */
    for (int h = 0; h < J->Hv; ++h) {
      if (key_head_of(h, J->Hk, J->Hv) != kh) continue;
      if (J->backward) run_backward_head(J, n, h, ckpt, segS, dS, kv, delta, u, w, dqh, dkh);
      else run_forward_head(J, n, h, S, kv, delta);
    }
  }
  (void)r;
  free(S); free(ckpt); free(segS); free(dS); free(vec);
  return NULL;
}

static int run(job_t* J, int nthreads) {
  if (J->N < 0 || J->Hk <= 0 || J->Hv <= 0 || J->Hv % J->Hk || J->Dk <= 0 || J->Dv <= 0) return -1;
  if (J->cu[0] != 0) return -1;
  for (int n = 0; n < J->N; ++n)
    if (J->cu[n + 1] < J->cu[n]) return -1;
  if (nthreads <= 0) nthreads = 1;
  if (nthreads > J->N * J->Hk) nthreads = J->N * J->Hk;
  if (nthreads < 1) nthreads = 1;
  J->next_item = 0;
  J->failed = 0;
  pthread_mutex_init(&J->lock, NULL);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  if (!th) return -2;
  int started = 0;
  for (int i = 0; i < nthreads; ++i)
    if (pthread_create(&th[i], NULL, worker, J) == 0) ++started;
  if (started == 0) worker(J);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J->lock);
  return J->failed ? -2 : 0;
}

/* Forward. o must hold T_total*Hv*Dv doubles; S_T may be NULL. Returns 0 on success. */
int oracle_gdn_fwd(int N, const int64_t* cu, int Hk, int Hv, int Dk, int Dv, double scale,
                   const double* q, const double* k, const double* v, const double* g,
                   const double* beta, const double* S0, double* o, double* S_T, int nthreads) {
  job_t J;
  memset(&J, 0, sizeof J);
  J.N = N; J.Hk = Hk; J.Hv = Hv; J.Dk = Dk; J.Dv = Dv; J.cu = cu; J.scale = scale;
  J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.S0 = S0; J.o = o; J.ST = S_T;
  J.backward = 0;
  return run(&J, nthreads);
}

/* Backward. dq, dk are overwritten (zeroed, then accumulated over each key
 * head's value heads in ascending order). dS_T and dS0 may be NULL. */
int oracle_gdn_bwd(int N, const int64_t* cu, int Hk, int Hv, int Dk, int Dv, double scale,
                   const double* q, const double* k, const double* v, const double* g,
                   const double* beta, const double* S0, const double* dO, const double* dS_T,
                   double* dq, double* dk, double* dv, double* dg, double* dbeta, double* dS0,
                   int nthreads) {
  job_t J;
  memset(&J, 0, sizeof J);
  J.N = N; J.Hk = Hk; J.Hv = Hv; J.Dk = Dk; J.Dv = Dv; J.cu = cu; J.scale = scale;
  J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.S0 = S0; J.dO = dO; J.dST = dS_T;
  J.dq = dq; J.dk = dk; J.dv = dv; J.dg = dg; J.dbeta = dbeta; J.dS0 = dS0;
  J.backward = 1;
  const int64_t T = cu[N];
  memset(dq, 0, (size_t)T * Hk * Dk * sizeof(double));
  memset(dk, 0, (size_t)T * Hk * Dk * sizeof(double));
  return run(&J, nthreads);
}
