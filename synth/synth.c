/*
 * synth.c -- seeded, counter-based synthetic inputs shared by the tests, the bench and the
 * oracle's callers.  It holds none of the method's arithmetic: only random numbers.
 *
 * Generator (SplitMix64 output function used counter-style, then Box-Muller):
 *   mix(z)      = SplitMix64 finaliser: z ^= z>>30; z *= 0xBF58476D1CE4E5B9;
 *                 z ^= z>>27; z *= 0x94D049BB133111EB; z ^= z>>31
 *   key         = mix(mix(mix(seed + g) + (tensor + 1) g) + (frame + 1) g),
 *                 g = 0x9E3779B97F4A7C15 (the SplitMix64 increment)
 *   word(i)     = mix(key + (i + 1) g)                       (the i-th SplitMix64 output)
 *   uniform(i)  = ((word(i) >> 11) + 1) * 2^-53               in (0, 1]
 *   normal(e)   = sqrt(-2 ln uniform(2e)) * cos(2 pi uniform(2e + 1))   (double, then * stddev,
 *                 then rounded to float)
 * Every element is a pure function of (seed, tensor, frame, element index), so any frame
 * can be regenerated from its id, in any order, on any number of threads.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_stream_key(uint64_t seed, uint32_t tensor, uint64_t frame) {
  uint64_t k = mix64(seed + SYNTH_GAMMA);
  k = mix64(k + ((uint64_t)tensor + 1ULL) * SYNTH_GAMMA);
  return mix64(k + (frame + 1ULL) * SYNTH_GAMMA);
}

static double uniform01(uint64_t key, uint64_t i) {
  uint64_t w = mix64(key + (i + 1ULL) * SYNTH_GAMMA);
  return (double)((w >> 11) + 1ULL) * (1.0 / 9007199254740992.0);
}

static double normal_at(uint64_t key, uint64_t e) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = uniform01(key, 2 * e), u2 = uniform01(key, 2 * e + 1);
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

typedef struct {
  uint64_t key, first, count;
  double stddev, prob;
  float factor;
  float* out;
  int mode; /* 0 normal, 1 outlier multiply, 2 uniform */
} synth_job;

static void* synth_worker(void* p) {
  synth_job* j = (synth_job*)p;
  for (uint64_t i = 0; i < j->count; ++i) {
    uint64_t e = j->first + i;
    if (j->mode == 0) {
      j->out[i] = (float)(normal_at(j->key, e) * j->stddev);
    } else if (j->mode == 1) {
      if (uniform01(j->key, e) < j->prob) j->out[i] = j->out[i] * j->factor;
    } else {
      j->out[i] = (float)uniform01(j->key, e);
    }
  }
  return NULL;
}

static void run_jobs(uint64_t key, uint64_t first, uint64_t count, double stddev, double prob,
                     float factor, float* out, int mode, int threads) {
  if (threads < 1) threads = 1;
  if (threads > 64) threads = 64;
  if ((uint64_t)threads > count / 4096 + 1) threads = (int)(count / 4096 + 1);
  synth_job jobs[64];
  pthread_t tid[64];
  int created[64] = {0};
  uint64_t per = (count + (uint64_t)threads - 1) / (uint64_t)threads;
  for (int t = 0; t < threads; ++t) {
    uint64_t lo = (uint64_t)t * per, hi = lo + per;
    if (lo > count) lo = count;
    if (hi > count) hi = count;
    jobs[t].key = key;
    jobs[t].first = first + lo;
    jobs[t].count = hi - lo;
    jobs[t].stddev = stddev;
    jobs[t].prob = prob;
    jobs[t].factor = factor;
    jobs[t].out = out + lo;
    jobs[t].mode = mode;
  }
  for (int t = 1; t < threads; ++t)
    created[t] = pthread_create(&tid[t], NULL, synth_worker, &jobs[t]) == 0;
  synth_worker(&jobs[0]);
  for (int t = 1; t < threads; ++t) {
    if (created[t])
      pthread_join(tid[t], NULL);
    else
      synth_worker(&jobs[t]);
  }
}

/* out[i] = stddev * normal(first + i) of stream (seed, tensor, frame), i < count. */
void synth_normal(uint64_t seed, uint32_t tensor, uint64_t frame, uint64_t first, uint64_t count,
                  double stddev, float* out, int threads) {
  run_jobs(synth_stream_key(seed, tensor, frame), first, count, stddev, 0.0, 1.0f, out, 0, threads);
}

/* inout[i] *= factor where uniform(first + i) of stream (seed, tensor, frame) < prob. */
void synth_outliers(uint64_t seed, uint32_t tensor, uint64_t frame, uint64_t first, uint64_t count,
                    double prob, float factor, float* inout, int threads) {
  run_jobs(synth_stream_key(seed, tensor, frame), first, count, 0.0, prob, factor, inout, 1,
           threads);
}

/* out[i] = (float)uniform(first + i); used to pick sampled rows. */
void synth_uniform(uint64_t seed, uint32_t tensor, uint64_t frame, uint64_t first, uint64_t count,
                   float* out, int threads) {
  run_jobs(synth_stream_key(seed, tensor, frame), first, count, 0.0, 0.0, 1.0f, out, 2, threads);
}
