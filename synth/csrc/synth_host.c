/*
 * synth_host.c -- host generator for the seeded synthetic KDA inputs.
 * Threads split the rows; every value comes from synth_core.h, so the
 * result does not depend on the thread count and matches the device
 * generator bit for bit.
 */
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>

#include "synth_core.h"

typedef struct {
  int kind; /* 0 rows, 1 beta, 2 state */
  const synth_row_recipe* recipe;
  uint32_t seed;
  double scale;
  int dtype;
  int b0, nb, t0, nt, h0, nh;
  void* dst;
  int64_t first, last; /* [first, last) over the flattened (b, t, h) or (b, h, i) index */
} synth_job;

static void* synth_worker(void* arg) {
  synth_job* j = (synth_job*)arg;
  for (int64_t n = j->first; n < j->last; ++n) {
    if (j->kind == 0) {
      int64_t hh = n % j->nh, tt = (n / j->nh) % j->nt, bb = n / ((int64_t)j->nh * j->nt);
      uint32_t b = (uint32_t)(j->b0 + bb), t = (uint32_t)(j->t0 + tt), h = (uint32_t)(j->h0 + hh);
      double div = synth_row_divisor(j->recipe, b, t, h);
      for (uint32_t g = 0; g < SYNTH_D / 4; ++g) {
        double z[4];
        synth_row_group(j->recipe, b, t, h, g, z);
        for (int c = 0; c < 4; ++c) synth_store(j->dst, (uint64_t)n * SYNTH_D + 4 * g + c, j->dtype, z[c] / div);
      }
    } else if (j->kind == 1) {
      int64_t hh = n % j->nh, tt = (n / j->nh) % j->nt, bb = n / ((int64_t)j->nh * j->nt);
      double x = synth_beta(j->seed, (uint32_t)(j->b0 + bb), (uint32_t)(j->t0 + tt), (uint32_t)(j->h0 + hh));
      synth_store(j->dst, (uint64_t)n, j->dtype, x);
    } else {
      /* n enumerates (b, h, i) rows of the state */
      int64_t i = n % SYNTH_D, hh = (n / SYNTH_D) % j->nh, bb = n / ((int64_t)SYNTH_D * j->nh);
      for (uint32_t g = 0; g < SYNTH_D / 4; ++g) {
        double z[4];
        synth_state4(j->seed, j->scale, (uint32_t)(j->b0 + bb), (uint32_t)(j->h0 + hh), (uint32_t)i, g, z);
        for (int c = 0; c < 4; ++c) synth_store(j->dst, (uint64_t)n * SYNTH_D + 4 * g + c, j->dtype, z[c]);
      }
    }
  }
  return NULL;
}

static int synth_run(synth_job base, int64_t total, int n_threads) {
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  if (total < n_threads) n_threads = total > 0 ? (int)total : 1;
  pthread_t tid[256];
  synth_job jobs[256];
  for (int i = 0; i < n_threads; ++i) {
    jobs[i] = base;
    jobs[i].first = total * i / n_threads;
    jobs[i].last = total * (i + 1) / n_threads;
  }
  int started = 0;
  for (int i = 1; i < n_threads; ++i) {
    if (pthread_create(&tid[i], NULL, synth_worker, &jobs[i]) != 0) break;
    started = i;
  }
  synth_worker(&jobs[0]);
  for (int i = 1; i <= started; ++i) pthread_join(tid[i], NULL);
  for (int i = started + 1; i < n_threads; ++i) synth_worker(&jobs[i]); /* threads that failed to start */
  return 0;
}

/* Rows [b0, b0+nb) x [t0, t0+nt) x [h0, h0+nh) of a row tensor into dst laid
 * out [nb][nt][nh][128] with element type dtype. Returns 0, or -1 on bad
 * arguments. */
int synth_rows_host(const synth_row_recipe* recipe, int dtype, int b0, int nb, int t0, int nt, int h0, int nh,
                    void* dst, int n_threads) {
  if (!recipe || (!dst && (int64_t)nb * nt * nh > 0) || nb < 0 || nt < 0 || nh < 0 || b0 < 0 || t0 < 0 || h0 < 0 || dtype < 0 || dtype > 2) return -1;
  synth_job j = {0, recipe, 0, 0.0, dtype, b0, nb, t0, nt, h0, nh, dst, 0, 0};
  return synth_run(j, (int64_t)nb * nt * nh, n_threads);
}

/* beta for the same block into dst laid out [nb][nt][nh]. */
int synth_beta_host(uint32_t seed, int dtype, int b0, int nb, int t0, int nt, int h0, int nh, void* dst,
                    int n_threads) {
  if ((!dst && (int64_t)nb * nt * nh > 0) || nb < 0 || nt < 0 || nh < 0 || b0 < 0 || t0 < 0 || h0 < 0 || dtype < 0 ||
      dtype > 2)
    return -1;
  synth_job j = {1, NULL, seed, 0.0, dtype, b0, nb, t0, nt, h0, nh, dst, 0, 0};
  return synth_run(j, (int64_t)nb * nt * nh, n_threads);
}

/* Initial states for batches [b0, b0+nb) and heads [h0, h0+nh) into dst laid
 * out [nb][nh][128][128]. */
int synth_state_host(uint32_t seed, double scale, int dtype, int b0, int nb, int h0, int nh, void* dst,
                     int n_threads) {
  if ((!dst && (int64_t)nb * nh > 0) || nb < 0 || nh < 0 || b0 < 0 || h0 < 0 || dtype < 0 || dtype > 2) return -1;
  synth_job j = {2, NULL, seed, scale, dtype, b0, nb, 0, 1, h0, nh, dst, 0, 0};
  return synth_run(j, (int64_t)nb * nh * SYNTH_D, n_threads);
}

/* Raw Philox4x32-10 block, exposed for the known-answer test. */
void synth_philox_host(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  synth_u32x4 c = {ctr[0], ctr[1], ctr[2], ctr[3]};
  synth_u32x4 r = synth_philox(c, key[0], key[1]);
  out[0] = r.x0;
  out[1] = r.x1;
  out[2] = r.x2;
  out[3] = r.x3;
}

/* The generator's own ln, sin/cos(2 pi u) and exp, exposed for accuracy tests. */
double synth_ln_host(double x) { return synth_ln(x); }
void synth_sincos_2pi_host(double u, double* s, double* c) { synth_sincos_2pi(u, s, c); }
double synth_exp_host(double x) { return synth_exp(x); }
