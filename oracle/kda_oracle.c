/*
 * kda_oracle.c -- reference oracle for Kimi Delta Attention (KDA), forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Plain, slow, token-by-token fp64 on the CPU.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it; the HIP library never links, includes or calls it, and it
 * shares no code with the HIP library.
 *
 * What it computes, per (batch, head) sequence: eq. (1) of the page
 * "Kimi K3：从三条信息流到完整系统" (wineandchord.com), section
 * "KDA 是带逐通道遗忘的 delta rule",
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t,
 *
 * evaluated token by token.  Multiplying out the product with
 * X = Diag(alpha_t) S_{t-1} gives
 *
 *   S_t = X - beta_t k_t (k_t^T X) + beta_t k_t v_t^T = X + beta_t k_t (v_t - X^T k_t)^T,
 *
 * so each token costs O(d_k d_v) instead of forming the d_k x d_k matrix:
 *
 *   X     =  Diag(alpha_t) S_{t-1}         (the decay acts on the old state)
 *   r     =  v_t - X^T k_t                 (r^T = v_t^T - k_t^T X)
 *   S_t   =  X + beta_t k_t r^T
 *   o_t   =  S_t^T q_t                     (the output reads the new state)
 *
 * with alpha_t = exp(g_t) per key channel.
 * The gate is eq. (5) of the section "下界 log-decay 是一个 kernel 设计":
 * g = g_min * sigmoid(x) with g_min = -5, where x already includes the
 * learned scale e^A (the caller passes x as the gate logit a).
 *
 * S has d_k rows (key channels) and d_v columns, stored row-major.
 * Layouts: q, k, g|a [n][T][d_k]; v, o [n][T][d_v]; beta [n][T];
 * s0, s_final [n][d_k][d_v] (s0 may be NULL for a zero initial state).
 *
 * Optionally the state is also copied out after every `every` tokens (the
 * sparse KDA state checkpoints of the page's section "hybrid prefix cache"):
 * states [n][T / every][d_k][d_v], checkpoint i holding S after token
 * every * (i + 1).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Eq. (5): g = -5 * sigmoid(a). */
double kda_oracle_gate1(double a) { return -5.0 / (1.0 + exp(-a)); }

void kda_oracle_gate(const double* a, double* g, int64_t n) {
  for (int64_t i = 0; i < n; ++i) g[i] = kda_oracle_gate1(a[i]);
}

/* One sequence, T tokens, eq. (1) applied token by token. */
static void kda_oracle_sequence(int T, int dk, int dv, const double* q, const double* k, const double* v,
                                const double* gate, int gate_is_logit, const double* beta, const double* s0,
                                double* o, double* S, double* alpha, double* r, double* states, int every) {
  if (s0) {
    memcpy(S, s0, sizeof(double) * (size_t)dk * dv);
  } else {
    memset(S, 0, sizeof(double) * (size_t)dk * dv);
  }
  for (int t = 0; t < T; ++t) {
    const double* qt = q + (size_t)t * dk;
    const double* kt = k + (size_t)t * dk;
    const double* vt = v + (size_t)t * dv;
    const double* gt = gate + (size_t)t * dk;
    double bt = beta[t];

    /* alpha_t = exp(g_t), per key channel */
    for (int i = 0; i < dk; ++i) alpha[i] = exp(gate_is_logit ? kda_oracle_gate1(gt[i]) : gt[i]);

    /* X = Diag(alpha_t) S_{t-1}, in place */
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= alpha[i];

    /* r = v_t - X^T k_t */
    for (int j = 0; j < dv; ++j) r[j] = vt[j];
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) r[j] -= kt[i] * S[(size_t)i * dv + j];

    /* S_t = X + beta_t k_t r^T */
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += bt * kt[i] * r[j];

    /* o_t = S_t^T q_t */
    double* ot = o + (size_t)t * dv;
    for (int j = 0; j < dv; ++j) ot[j] = 0.0;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) ot[j] += qt[i] * S[(size_t)i * dv + j];

    /* checkpoint: the state after token t + 1 of the sequence */
    if (states && (t + 1) % every == 0)
      memcpy(states + (size_t)((t + 1) / every - 1) * dk * dv, S, sizeof(double) * (size_t)dk * dv);
  }
}

typedef struct {
  int first, last, T, dk, dv, gate_is_logit, every;
  const double *q, *k, *v, *gate, *beta, *s0;
  double *o, *s_final, *states;
  int failed;
} kda_oracle_job;

static void* kda_oracle_worker(void* arg) {
  kda_oracle_job* j = (kda_oracle_job*)arg;
  double* alpha = (double*)malloc(sizeof(double) * (size_t)j->dk);
  double* r = (double*)malloc(sizeof(double) * (size_t)j->dv);
  if (!alpha || !r) {
    j->failed = 1;
    free(alpha);
    free(r);
    return NULL;
  }
  size_t T = (size_t)j->T, dk = (size_t)j->dk, dv = (size_t)j->dv;
  size_t per_seq = j->states ? (T / (size_t)j->every) * dk * dv : 0;
  for (int n = j->first; n < j->last; ++n) {
    kda_oracle_sequence(j->T, j->dk, j->dv, j->q + n * T * dk, j->k + n * T * dk, j->v + n * T * dv,
                        j->gate + n * T * dk, j->gate_is_logit, j->beta + n * T, j->s0 ? j->s0 + n * dk * dv : NULL,
                        j->o + n * T * dv, j->s_final + n * dk * dv, alpha, r,
                        j->states ? j->states + n * per_seq : NULL, j->every);
  }
  free(alpha);
  free(r);
  return NULL;
}

/*
 * n_units independent sequences, each of T tokens.  gate holds log-decays g
 * (gate_is_logit = 0) or gate logits a (gate_is_logit = 1, g = -5 sigmoid(a)).
 * states, when not NULL, receives the checkpoints every `every` tokens
 * [n_units][T / every][dk][dv].  Returns 0 on success, -1 on bad arguments,
 * -2 if memory ran out.
 */
int kda_oracle_forward_states(int n_units, int T, int dk, int dv, const double* q, const double* k, const double* v,
                              const double* gate, int gate_is_logit, const double* beta, const double* s0, double* o,
                              double* s_final, double* states, int every, int n_threads) {
  if (n_units < 0 || T < 0 || dk <= 0 || dv <= 0 || !s_final) return -1;
  if (states && every <= 0) return -1;
  if (T > 0 && (!q || !k || !v || !gate || !beta || !o)) return -1;
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  if (n_threads > n_units) n_threads = n_units > 0 ? n_units : 1;
  pthread_t tid[256];
  kda_oracle_job jobs[256];
  for (int i = 0; i < n_threads; ++i) {
    kda_oracle_job j = {(int)((int64_t)n_units * i / n_threads), (int)((int64_t)n_units * (i + 1) / n_threads),
                        T, dk, dv, gate_is_logit, every, q, k, v, gate, beta, s0, o, s_final, states, 0};
    jobs[i] = j;
  }
  int started = 0;
  for (int i = 1; i < n_threads; ++i) {
    if (pthread_create(&tid[i], NULL, kda_oracle_worker, &jobs[i]) != 0) break;
    started = i;
  }
  kda_oracle_worker(&jobs[0]);
  for (int i = 1; i <= started; ++i) pthread_join(tid[i], NULL);
  for (int i = started + 1; i < n_threads; ++i) kda_oracle_worker(&jobs[i]);
  for (int i = 0; i < n_threads; ++i)
    if (jobs[i].failed) return -2;
  return 0;
}

/* kda_oracle_forward_states without checkpoints. */
int kda_oracle_forward(int n_units, int T, int dk, int dv, const double* q, const double* k, const double* v,
                       const double* gate, int gate_is_logit, const double* beta, const double* s0, double* o,
                       double* s_final, int n_threads) {
  return kda_oracle_forward_states(n_units, T, dk, dv, q, k, v, gate, gate_is_logit, beta, s0, o, s_final, NULL, 0,
                                   n_threads);
}
