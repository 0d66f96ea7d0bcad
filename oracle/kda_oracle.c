/*
 * kda_oracle.c -- FP64 reference oracle for the Kimi Delta Attention (KDA)
 * gated delta rule.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The GPU product path never calls it, links it or
 * shares code with it.
 *
 * What it computes (the plain definition, token by token, in double):
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *   o_t = scale * S_t^T q_t
 *
 * per head, with S a dk x dv matrix (row index = key channel c, column
 * index = value channel j).  This is the recurrence whose chunk-32 form is
 * evaluated by the fused kernel described in "FlashInfer PR #4262: CAKE KDA
 * Prefill Highlights", section 2 ("Fully fused M128 recurrent pipeline"):
 * the decay Diag(exp(g_t)) acts first, then the delta-rule erase/write, and
 * the output is read from the post-update state.  g_t is the per-channel
 * natural-log decay (the kernel works in the log2 domain internally; that is
 * an implementation detail and does not appear here).  beta_t is the
 * post-sigmoid write strength in [0, 1].
 *
 * Expanding the matrix form gives the four steps coded in kda_step():
 *   S'   = Diag(exp(g)) S                 (decay each key row c)
 *   w    = S'^T k                         (what the state predicts for k)
 *   u    = beta (v - w)                   (the delta)
 *   S''  = S' + k u^T                     (= (I - b k k^T) S' + b k v^T)
 *   o    = scale S''^T q
 *
 * Decode ("fused KDA decode", flashinfer PR #5551) is the same single step
 * applied to a state gathered from a slot-indexed pool and written back in
 * place; a negative slot index skips the row and zero-fills its output.
 *
 * Layouts (all row-major, all double):
 *   q, k, g : [T, H, dk]      v : [T, H, dv]      beta : [T, H]
 *   out     : [T, H, dv]
 *   state   : [N, H, dk, dv]  (prefill initial / final, per sequence)
 *   pool    : [num_slots, H, dk, dv]              (decode)
 * Sequences are delimited by cu_seqlens[0..N] (cu_seqlens[0] = 0,
 * non-decreasing, cu_seqlens[N] = T).  Units (sequence, head) or
 * (row, head) are independent and are spread over a small pthread pool.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KDA_ORACLE_OK 0
#define KDA_ORACLE_EINVAL -1
#define KDA_ORACLE_ENOMEM -2

/* One recurrence step on state S[dk][dv] (in place).  w and u are scratch of
 * length dv.  Writes o[dv]. */
static void kda_step(double *S, int dk, int dv, const double *q,
                     const double *k, const double *v, const double *g,
                     double beta, double scale, double *w, double *u,
                     double *o) {
  for (int c = 0; c < dk; ++c) {
    double a = exp(g[c]);
    double *row = S + (int64_t)c * dv;
    for (int j = 0; j < dv; ++j) row[j] *= a;
  }
  for (int j = 0; j < dv; ++j) w[j] = 0.0;
  for (int c = 0; c < dk; ++c) {
    const double *row = S + (int64_t)c * dv;
    for (int j = 0; j < dv; ++j) w[j] += k[c] * row[j];
  }
  for (int j = 0; j < dv; ++j) u[j] = beta * (v[j] - w[j]);
  for (int c = 0; c < dk; ++c) {
    double *row = S + (int64_t)c * dv;
    for (int j = 0; j < dv; ++j) row[j] += k[c] * u[j];
  }
  for (int j = 0; j < dv; ++j) o[j] = 0.0;
  for (int c = 0; c < dk; ++c) {
    const double *row = S + (int64_t)c * dv;
    for (int j = 0; j < dv; ++j) o[j] += q[c] * row[j];
  }
  for (int j = 0; j < dv; ++j) o[j] *= scale;
}

/* ------------------------------------------------------------------ pool */

typedef struct {
  int64_t next;         /* next unit to take (guarded by mu) */
  int64_t count;        /* number of units */
  pthread_mutex_t mu;
  void (*fn)(void *ctx, int64_t unit, double *scratch);
  void *ctx;
  size_t scratch_doubles;
  int failed;
} unit_pool;

static void *pool_worker(void *arg) {
  unit_pool *p = (unit_pool *)arg;
  double *scratch = (double *)malloc(p->scratch_doubles * sizeof(double));
  if (!scratch) {
    pthread_mutex_lock(&p->mu);
    p->failed = 1;
    pthread_mutex_unlock(&p->mu);
    return NULL;
  }
  for (;;) {
    pthread_mutex_lock(&p->mu);
    int64_t u = p->next < p->count ? p->next++ : -1;
    pthread_mutex_unlock(&p->mu);
    if (u < 0) break;
    p->fn(p->ctx, u, scratch);
  }
  free(scratch);
  return NULL;
}

static int run_units(int64_t count, int threads, size_t scratch_doubles,
                     void (*fn)(void *, int64_t, double *), void *ctx) {
  unit_pool p;
  p.next = 0;
  p.count = count;
  p.fn = fn;
  p.ctx = ctx;
  p.scratch_doubles = scratch_doubles;
  p.failed = 0;
  pthread_mutex_init(&p.mu, NULL);
  if (threads < 1) threads = 1;
  if (threads > count) threads = count > 0 ? (int)count : 1;
  pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)threads);
  if (!tid) return KDA_ORACLE_ENOMEM;
  int started = 0;
  for (int i = 0; i < threads; ++i) {
    if (pthread_create(&tid[i], NULL, pool_worker, &p) != 0) break;
    ++started;
  }
  if (started == 0) pool_worker(&p); /* no threads: run inline */
  for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
  free(tid);
  pthread_mutex_destroy(&p.mu);
  return p.failed ? KDA_ORACLE_ENOMEM : KDA_ORACLE_OK;
}

/* --------------------------------------------------------------- prefill */

typedef struct {
  const double *q, *k, *v, *g, *beta;
  const int64_t *cu;
  int N, H, dk, dv;
  double scale;
  const double *s0;
  double *s1, *out;
  int64_t snap_every;      /* 0: no snapshots */
  double *snaps;           /* [sum_n floor(len_n / snap_every)][H][dk][dv] */
  const int64_t *snap_base;/* first snapshot row of each sequence */
} prefill_ctx;

static void prefill_unit(void *vctx, int64_t unit, double *scratch) {
  const prefill_ctx *c = (const prefill_ctx *)vctx;
  const int n = (int)(unit / c->H), h = (int)(unit % c->H);
  const int H = c->H, dk = c->dk, dv = c->dv;
  const int64_t sz = (int64_t)dk * dv;
  double *S = scratch, *w = scratch + sz, *u = w + dv;
  if (c->s0)
    memcpy(S, c->s0 + ((int64_t)n * H + h) * sz, sizeof(double) * (size_t)sz);
  else
    memset(S, 0, sizeof(double) * (size_t)sz);
  for (int64_t t = c->cu[n]; t < c->cu[n + 1]; ++t) {
    const int64_t th = t * H + h;
    kda_step(S, dk, dv, c->q + th * dk, c->k + th * dk, c->v + th * dv,
             c->g + th * dk, c->beta[th], c->scale, w, u, c->out + th * dv);
    const int64_t done = t + 1 - c->cu[n];   /* tokens of this sequence processed */
    if (c->snap_every > 0 && done % c->snap_every == 0) {
      const int64_t row = c->snap_base[n] + done / c->snap_every - 1;
      memcpy(c->snaps + (row * H + h) * sz, S, sizeof(double) * (size_t)sz);
    }
  }
  if (c->s1)
    memcpy(c->s1 + ((int64_t)n * H + h) * sz, S, sizeof(double) * (size_t)sz);
}

int kda_oracle_prefill_snapshots(const double *q, const double *k, const double *v,
                                 const double *g, const double *beta,
                                 const int64_t *cu_seqlens, int num_seqs, int num_heads,
                                 int dk, int dv, double scale,
                                 const double *initial_state, double *final_state,
                                 double *out, int64_t snap_every, double *snapshots,
                                 int num_threads);

/* Packed variable-length prefill.  initial_state may be NULL (zeros);
 * final_state may be NULL (not stored) and may equal initial_state.
 * Returns 0, or a negative code for invalid arguments / allocation failure. */
int kda_oracle_prefill(const double *q, const double *k, const double *v,
                       const double *g, const double *beta,
                       const int64_t *cu_seqlens, int num_seqs, int num_heads,
                       int dk, int dv, double scale,
                       const double *initial_state, double *final_state,
                       double *out, int num_threads) {
  if (num_seqs < 0 || num_heads < 1 || dk < 1 || dv < 1 || !cu_seqlens)
    return KDA_ORACLE_EINVAL;
  if (cu_seqlens[0] != 0) return KDA_ORACLE_EINVAL;
  for (int n = 0; n < num_seqs; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return KDA_ORACLE_EINVAL;
  if (cu_seqlens[num_seqs] > 0 && (!q || !k || !v || !g || !beta || !out))
    return KDA_ORACLE_EINVAL;
  return kda_oracle_prefill_snapshots(q, k, v, g, beta, cu_seqlens, num_seqs, num_heads, dk,
                                      dv, scale, initial_state, final_state, out, 0, NULL,
                                      num_threads);
}

/* As kda_oracle_prefill, and in addition the state after every `snap_every`
 * tokens of each sequence (after tokens snap_every, 2 snap_every, ... up to
 * the sequence length), stored row by row in sequence order:
 * snapshots[sum_{m<n} floor(len_m / snap_every) + j - 1] is the state of
 * sequence n after j * snap_every tokens, [H][dk][dv] each. */
int kda_oracle_prefill_snapshots(const double *q, const double *k, const double *v,
                                 const double *g, const double *beta,
                                 const int64_t *cu_seqlens, int num_seqs, int num_heads,
                                 int dk, int dv, double scale,
                                 const double *initial_state, double *final_state,
                                 double *out, int64_t snap_every, double *snapshots,
                                 int num_threads) {
  if (num_seqs < 0 || num_heads < 1 || dk < 1 || dv < 1 || !cu_seqlens)
    return KDA_ORACLE_EINVAL;
  if (cu_seqlens[0] != 0) return KDA_ORACLE_EINVAL;
  for (int n = 0; n < num_seqs; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return KDA_ORACLE_EINVAL;
  if (cu_seqlens[num_seqs] > 0 && (!q || !k || !v || !g || !beta || !out))
    return KDA_ORACLE_EINVAL;
  if (snap_every < 0 || (snap_every > 0 && !snapshots)) return KDA_ORACLE_EINVAL;
  int64_t *base = NULL;
  if (snap_every > 0) {
    base = (int64_t *)malloc(sizeof(int64_t) * (size_t)(num_seqs + 1));
    if (!base) return KDA_ORACLE_ENOMEM;
    base[0] = 0;
    for (int n = 0; n < num_seqs; ++n)
      base[n + 1] = base[n] + (cu_seqlens[n + 1] - cu_seqlens[n]) / snap_every;
  }
  prefill_ctx c = {q, k, v, g, beta, cu_seqlens, num_seqs, num_heads, dk, dv,
                   scale, initial_state, final_state, out, snap_every, snapshots, base};
  /* final_state == initial_state is allowed: each unit copies its slice in
   * before the loop and out after it, and units touch disjoint slices. */
  const int rc = run_units((int64_t)num_seqs * num_heads, num_threads,
                           (size_t)dk * dv + 2 * (size_t)dv, prefill_unit, &c);
  free(base);
  return rc;
}

/* ---------------------------------------------------------------- decode */

typedef struct {
  const double *q, *k, *v, *g, *beta;
  double *pool;
  const int64_t *slots;
  int64_t num_slots;
  int rows, H, dk, dv;
  double scale;
  double *out;
} decode_ctx;

static void decode_unit(void *vctx, int64_t unit, double *scratch) {
  const decode_ctx *c = (const decode_ctx *)vctx;
  const int r = (int)(unit / c->H), h = (int)(unit % c->H);
  const int H = c->H, dk = c->dk, dv = c->dv;
  const int64_t rh = (int64_t)r * H + h;
  const int64_t slot = c->slots[r];
  if (slot < 0) {
    for (int j = 0; j < dv; ++j) c->out[rh * dv + j] = 0.0;
    return;
  }
  double *S = c->pool + (slot * H + h) * (int64_t)dk * dv;
  double *w = scratch, *u = scratch + dv;
  kda_step(S, dk, dv, c->q + rh * dk, c->k + rh * dk, c->v + rh * dv,
           c->g + rh * dk, c->beta[rh], c->scale, w, u, c->out + rh * dv);
}

/* T=1 decode over a slot-indexed pool, updated in place.  Slots must be
 * unique among the non-negative entries; a negative slot skips its row. */
int kda_oracle_decode(const double *q, const double *k, const double *v,
                      const double *g, const double *beta, double *pool,
                      int64_t num_slots, const int64_t *slot_indices,
                      int rows, int num_heads, int dk, int dv, double scale,
                      double *out, int num_threads) {
  if (rows < 0 || num_heads < 1 || dk < 1 || dv < 1 || num_slots < 0)
    return KDA_ORACLE_EINVAL;
  if (rows == 0) return KDA_ORACLE_OK;
  if (!q || !k || !v || !g || !beta || !pool || !slot_indices || !out)
    return KDA_ORACLE_EINVAL;
  for (int r = 0; r < rows; ++r)
    if (slot_indices[r] >= num_slots) return KDA_ORACLE_EINVAL;
  decode_ctx c = {q, k, v, g, beta, pool, slot_indices, num_slots,
                  rows, num_heads, dk, dv, scale, out};
  return run_units((int64_t)rows * num_heads, num_threads, 2 * (size_t)dv,
                   decode_unit, &c);
}

int kda_oracle_version(void) { return 1; }
