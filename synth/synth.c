/*
 * Seeded synthetic inputs shared by the oracle and the GPU library's tests and
 * benchmark.  This module holds none of the method's arithmetic: it only draws
 * normal variates.  Both sides receive the same float32 arrays from here.
 *
 * Generator: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014) used as a counter-based generator: the
 * i-th draw of a stream with seed s is mix(s + (i+1)*GAMMA), so any slice of
 * a stream can be produced independently (and in parallel).  Two consecutive
 * draws make one Box-Muller pair (Box & Muller 1958): even index -> cosine
 * branch, odd index -> sine branch.
 */
#include "synth.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_splitmix64_at(uint64_t seed, uint64_t i) {
  return sm64_mix(seed + (i + 1) * SM64_GAMMA);
}

uint64_t synth_seed_from_tag(const char* tag) {
  /* FNV-1a 64 over the tag bytes, then one SplitMix64 finalisation. */
  uint64_t h = 0xCBF29CE484222325ULL;
  for (const unsigned char* p = (const unsigned char*)tag; *p; ++p) {
    h ^= (uint64_t)*p;
    h *= 0x100000001B3ULL;
  }
  return sm64_mix(h ^ 0x5EEDULL);
}

static inline double normal_at(uint64_t seed, uint64_t i) {
  const uint64_t p = i >> 1;
  /* u1 in (0,1], u2 in [0,1): 53-bit uniforms. */
  const double u1 = (double)((synth_splitmix64_at(seed, 2 * p) >> 11) + 1) * 0x1p-53;
  const double u2 = (double)(synth_splitmix64_at(seed, 2 * p + 1) >> 11) * 0x1p-53;
  const double r = sqrt(-2.0 * log(u1));
  const double a = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(a) : r * cos(a);
}

typedef struct {
  uint64_t seed, offset, begin, end;
  double mean, std;
  float* out;
} job_t;

static void* run_job(void* arg) {
  job_t* j = (job_t*)arg;
  uint64_t i = j->begin;
  /* a leading odd index: its pair started before this slice */
  if (i < j->end && ((j->offset + i) & 1)) {
    j->out[i] = (float)(j->mean + j->std * normal_at(j->seed, j->offset + i));
    ++i;
  }
  /* whole pairs share one radius and one angle */
  for (; i + 1 < j->end; i += 2) {
    const uint64_t p = (j->offset + i) >> 1;
    const double u1 = (double)((synth_splitmix64_at(j->seed, 2 * p) >> 11) + 1) * 0x1p-53;
    const double u2 = (double)(synth_splitmix64_at(j->seed, 2 * p + 1) >> 11) * 0x1p-53;
    const double r = sqrt(-2.0 * log(u1));
    const double a = 6.283185307179586476925286766559 * u2;
    j->out[i] = (float)(j->mean + j->std * (r * cos(a)));
    j->out[i + 1] = (float)(j->mean + j->std * (r * sin(a)));
  }
  if (i < j->end) j->out[i] = (float)(j->mean + j->std * normal_at(j->seed, j->offset + i));
  return NULL;
}

int synth_normal_f32(uint64_t seed, uint64_t offset, uint64_t count, double mean, double std,
                     float* out, int nthreads) {
  if (!out && count) return -1;
  if (nthreads <= 0) {
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    const char* env = getenv("OMP_NUM_THREADS");
    if (env && atoi(env) > 0 && atoi(env) < n) n = atoi(env);
    nthreads = n > 0 ? (int)n : 1;
  }
  if (nthreads > 256) nthreads = 256;
  if (count < (1u << 16) || nthreads == 1) {
    job_t j = {seed, offset, 0, count, mean, std, out};
    run_job(&j);
    return 0;
  }
  pthread_t th[256];
  job_t jobs[256];
  int ok[256];
  const uint64_t per = (count + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    uint64_t b = (uint64_t)t * per, e = b + per;
    if (b > count) b = count;
    if (e > count) e = count;
    jobs[t] = (job_t){seed, offset, b, e, mean, std, out};
    ok[t] = pthread_create(&th[t], NULL, run_job, &jobs[t]) == 0;
    if (!ok[t]) run_job(&jobs[t]);
  }
  for (int t = 0; t < nthreads; ++t)
    if (ok[t]) pthread_join(th[t], NULL);
  return 0;
}

int synth_uniform_f64(uint64_t seed, uint64_t offset, uint64_t count, double* out) {
  if (!out && count) return -1;
  for (uint64_t i = 0; i < count; ++i)
    out[i] = (double)(synth_splitmix64_at(seed, offset + i) >> 11) * 0x1p-53;
  return 0;
}
