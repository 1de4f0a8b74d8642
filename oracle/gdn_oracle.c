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
 * The backward follows the same page's gdn_backward, steps 4a-4d (output,
 * state update, delta, retrieval), run in reverse time with the state adjoint
 * dS carried across tokens. Two generalisations of that page, which starts from
 * S = 0 and dS = 0: the initial state S0 and the incoming adjoint dS_T may be
 * non-zero (NULL means zero), and dS0 is returned. dq and dk of a key head are
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
 * Reverse-time backward of one (sequence, value head). dq/dk of this head are
 * added into dq/dk of its key head (the caller walks the heads of a group in
 * ascending order). Buffers: ckpt holds S at every SEG boundary, segS the
 * states before each token of the current segment plus the state after it.
 */
static void run_backward_head(job_t* J, int n, int h, double* ckpt, double* segS, double* dS,
                              double* kv, double* delta, double* ddelta, double* dkv,
                              double* dqh, double* dkh) {
  const int Hk = J->Hk, Hv = J->Hv, Dk = J->Dk, Dv = J->Dv;
  const int kh = key_head_of(h, Hk, Hv);
  const size_t SS = (size_t)Dk * Dv;
  const int64_t t0 = J->cu[n], t1 = J->cu[n + 1];
  const int64_t len = t1 - t0;
  const int64_t nseg = (len + SEG - 1) / SEG;

  /* forward re-run keeping a copy of S at the start of every segment */
  double* S = segS; /* scratch for the re-run */
  if (J->S0) memcpy(S, J->S0 + ((size_t)n * Hv + h) * SS, SS * sizeof(double));
  else memset(S, 0, SS * sizeof(double));
  for (int64_t s = 0; s < nseg; ++s) {
    memcpy(ckpt + (size_t)s * SS, S, SS * sizeof(double));
    int64_t a = t0 + s * SEG, b = a + SEG < t1 ? a + SEG : t1;
    for (int64_t t = a; t < b; ++t) {
      const double* kt = J->k + ((size_t)t * Hk + kh) * Dk;
      const double* vt = J->v + ((size_t)t * Hv + h) * Dv;
      step_forward(S, kt, vt, J->g[(size_t)t * Hv + h], J->beta[(size_t)t * Hv + h], kv, delta, Dk, Dv);
    }
  }

  if (J->dST) memcpy(dS, J->dST + ((size_t)n * Hv + h) * SS, SS * sizeof(double));
  else memset(dS, 0, SS * sizeof(double));

  for (int64_t s = nseg - 1; s >= 0; --s) {
    int64_t a = t0 + s * SEG, b = a + SEG < t1 ? a + SEG : t1;
    /* segS[r] = state before token a+r; segS[b-a] = state after the last token */
    memcpy(segS, ckpt + (size_t)s * SS, SS * sizeof(double));
    for (int64_t t = a; t < b; ++t) {
      double* Snext = segS + (size_t)(t - a + 1) * SS;
      memcpy(Snext, segS + (size_t)(t - a) * SS, SS * sizeof(double));
      const double* kt = J->k + ((size_t)t * Hk + kh) * Dk;
      const double* vt = J->v + ((size_t)t * Hv + h) * Dv;
      step_forward(Snext, kt, vt, J->g[(size_t)t * Hv + h], J->beta[(size_t)t * Hv + h], kv, delta, Dk, Dv);
    }
    for (int64_t t = b - 1; t >= a; --t) {
      const double* Sprev = segS + (size_t)(t - a) * SS;
      const double* St = segS + (size_t)(t - a + 1) * SS;
      const double* kt = J->k + ((size_t)t * Hk + kh) * Dk;
      const double* qt = J->q + ((size_t)t * Hk + kh) * Dk;
      const double* vt = J->v + ((size_t)t * Hv + h) * Dv;
      const double* dot = J->dO + ((size_t)t * Hv + h) * Dv;
      const double gt = J->g[(size_t)t * Hv + h];
      const double bt = J->beta[(size_t)t * Hv + h];
      const double sc = J->scale;

      /* recompute kv = S_{t-1}^T k and delta */
      for (int j = 0; j < Dv; ++j) kv[j] = 0.0;
      for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j) kv[j] += Sprev[i * Dv + j] * kt[i];
      for (int j = 0; j < Dv; ++j) delta[j] = bt * (vt[j] - gt * kv[j]);

      /* 4a: o = scale * S_t^T q  ->  dS += scale * q (x) dO ; dq = scale * S_t dO */
      for (int i = 0; i < Dk; ++i) {
        double acc = 0.0;
        for (int j = 0; j < Dv; ++j) {
          dS[i * Dv + j] += sc * qt[i] * dot[j];
          acc += St[i * Dv + j] * dot[j];
        }
#if defined(ORACLE_PLANT) && ORACLE_PLANT == 4
        dqh[i] = acc; /* planted mistake: scale dropped from dq */
#else
        dqh[i] = sc * acc;
#endif
      }

      /* 4b: S_t = g S_{t-1} + k (x) delta */
      double dgt = 0.0;
      for (int i = 0; i < Dk; ++i) dkh[i] = 0.0;
      for (int j = 0; j < Dv; ++j) ddelta[j] = 0.0;
      for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j) {
          const double d = dS[i * Dv + j];
          dgt += Sprev[i * Dv + j] * d;
          dkh[i] += d * delta[j];
          ddelta[j] += d * kt[i];
        }
      for (size_t ij = 0; ij < SS; ++ij) dS[ij] *= gt;

      /* 4c: delta = beta (v - g kv) */
      double dbt = 0.0;
      double* dvt = J->dv + ((size_t)t * Hv + h) * Dv;
      for (int j = 0; j < Dv; ++j) {
        dvt[j] = bt * ddelta[j];
        dkv[j] = -gt * bt * ddelta[j];
#if defined(ORACLE_PLANT) && ORACLE_PLANT == 3
        dgt += (kv[j] * bt) * ddelta[j]; /* planted mistake: sign */
#else
        dgt += (-kv[j] * bt) * ddelta[j];
#endif
        dbt += (vt[j] - gt * kv[j]) * ddelta[j];
      }

      /* 4d: kv = S_{t-1}^T k */
      for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j) {
          dS[i * Dv + j] += kt[i] * dkv[j];
#if !(defined(ORACLE_PLANT) && ORACLE_PLANT == 2)
          dkh[i] += Sprev[i * Dv + j] * dkv[j]; /* (plant 2 drops this term) */
#endif
        }

      J->dg[(size_t)t * Hv + h] = dgt;
      J->dbeta[(size_t)t * Hv + h] = dbt;
      double* dqt = J->dq + ((size_t)t * Hk + kh) * Dk;
      double* dkt = J->dk + ((size_t)t * Hk + kh) * Dk;
      for (int i = 0; i < Dk; ++i) {
        dqt[i] += dqh[i];
        dkt[i] += dkh[i];
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
  double *kv = vec, *delta = vec + Dm, *ddelta = vec + 2 * Dm, *dkv = vec + 3 * Dm;
  double *dqh = vec + 4 * Dm, *dkh = vec + 5 * Dm;
  for (;;) {
    int it = take_item(J);
    if (it >= J->N * J->Hk) break;
    int n = it / J->Hk, kh = it % J->Hk;
    /* the value heads of key head kh, in ascending order */
    for (int h = 0; h < J->Hv; ++h) {
      if (key_head_of(h, J->Hk, J->Hv) != kh) continue;
      if (J->backward) run_backward_head(J, n, h, ckpt, segS, dS, kv, delta, ddelta, dkv, dqh, dkh);
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
