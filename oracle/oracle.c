/*
 * CPU oracle for the dual-path quantized-base + LoRA linear.
 *
 * TEST INFRASTRUCTURE ONLY: only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg may load or call it.  It shares no code with
 * the GPU library.  Every reduction is a plain sequential float64 loop; the
 * only parallelism is a static split of output rows across threads, which
 * does not change any result.
 *
 * Parity pins for every function live in tests/test_oracle_*.py; none is
 * "parity unpinned".
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------------ */
/* Floating-point formats (IEEE 754-2008 binary16; bfloat16 = the top half of */
/* binary32).  Round to nearest, ties to even, as the standard's default.     */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}
static float bits_f32(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

uint16_t or_f16_from_f32(float f) {
  const uint32_t x = f32_bits(f);
  const uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
  const uint32_t ax = x & 0x7FFFFFFFu;
  if (ax > 0x7F800000u) /* NaN: keep it quiet, carry the top payload bits */
    return (uint16_t)(sign | 0x7E00u | ((ax >> 13) & 0x03FFu));
  if (ax >= 0x477FF000u) /* >= 65520 (half-way above 65504) rounds to infinity */
    return (uint16_t)(sign | 0x7C00u);
  if (ax < 0x38800000u) { /* below 2^-14: binary16 subnormal range, step 2^-24 */
    const uint32_t e = ax >> 23;
    if (e == 0) return sign; /* binary32 subnormals are far below 2^-25 */
    const uint32_t m = (ax & 0x7FFFFFu) | 0x800000u; /* value = m * 2^(e-150) */
    const uint32_t shift = 126u - e;                 /* value / 2^-24 = m >> shift */
    if (shift > 24u) return sign;                    /* below 2^-25: rounds to zero */
    uint32_t q = m >> shift;
    const uint32_t rem = m & ((1u << shift) - 1u), half = 1u << (shift - 1u);
    if (rem > half || (rem == half && (q & 1u))) ++q;
    return (uint16_t)(sign | q);
  }
  /* normal: re-bias exponent 127 -> 15, keep 10 of 23 mantissa bits */
  uint32_t q = (((ax >> 23) - 112u) << 10) | ((ax & 0x7FFFFFu) >> 13);
  const uint32_t rem = ax & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (q & 1u))) ++q; /* carry may bump the exponent */
  return (uint16_t)(sign | q);
}

float or_f32_from_f16(uint16_t h) {
  const uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
  if (e == 0) { /* zero or subnormal: m * 2^-24, exact in binary32 */
    const float v = (float)m * 0x1p-24f;
    return bits_f32(f32_bits(v) | sign);
  }
  if (e == 31) return bits_f32(sign | 0x7F800000u | (m << 13));
  return bits_f32(sign | ((e + 112u) << 23) | (m << 13));
}

uint16_t or_bf16_from_f32(float f) {
  const uint32_t x = f32_bits(f);
  if ((x & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((x >> 16) | 0x0040u); /* quiet NaN */
  const uint32_t lower = x & 0xFFFFu, upper = x >> 16;
  uint32_t q = upper;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) ++q; /* may carry to Inf */
  return (uint16_t)q;
}

float or_f32_from_bf16(uint16_t b) { return bits_f32((uint32_t)b << 16); }

uint16_t or_bf16_from_f64(double v) {
  /* Round a double straight to the 8-significant-bit bfloat16 grid (one
   * rounding), then the result is exact in binary32. */
  if (isnan(v)) return 0x7FC0u;
  if (v == 0.0) return signbit(v) ? 0x8000u : 0x0000u;
  if (isinf(v)) return v < 0 ? 0xFF80u : 0x7F80u;
  int e;
  const double fr = frexp(v, &e); /* v = fr * 2^e, 0.5 <= |fr| < 1 */
  double r;
  if (e - 8 >= -133) {
    r = ldexp(nearbyint(ldexp(fr, 8)), e - 8); /* 8 significant bits */
  } else {
    r = ldexp(nearbyint(ldexp(v, 133)), -133); /* subnormal step 2^-133 */
  }
  if (fabs(r) > 0x1.FEp127) return v < 0 ? 0xFF80u : 0x7F80u; /* beyond the largest finite */
  return (uint16_t)(f32_bits((float)r) >> 16);
}

/* ------------------------------------------------------------------------ */
/* Block formats.                                                           */
/* q8_0: 32 weights and one fp16 scale (Deep Technical Design, section 5,   */
/* "Quantized-Base Numerical Analysis": 8.5 bits per weight).  Scale        */
/* d = fp16(max|w|/127), q = round(w/d) with the stored d, rounding half    */
/* away from zero.                                                          */
/* q4_sm: 32 unsigned 4-bit q, fp16 scale d and fp16 min m, w = d*q + m;     */
/* m = fp16(min w), d = fp16((max w - m)/15), q = round((w - m)/d) in [0,15].*/
/* ------------------------------------------------------------------------ */

int32_t or_block_bytes(int32_t qtype) {
  return qtype == OR_Q8_0 ? 34 : qtype == OR_Q4_SM ? 20 : qtype == OR_Q4_K ? 144 : 0;
}

int32_t or_block_weights(int32_t qtype) {
  return qtype == OR_Q8_0 || qtype == OR_Q4_SM ? 32 : qtype == OR_Q4_K ? 256 : 0;
}

static void put16(uint8_t* p, uint16_t v) {
  p[0] = (uint8_t)(v & 0xFF);
  p[1] = (uint8_t)(v >> 8);
}
static uint16_t get16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

static void quantize_q8_0_block(const float* w, uint8_t* blk) {
  float amax = 0.0f;
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(w[j]));
  const uint16_t dh = or_f16_from_f32(amax / 127.0f);
  const float d = or_f32_from_f16(dh);
  put16(blk, dh);
  for (int j = 0; j < 32; ++j) {
    float q = d == 0.0f ? 0.0f : roundf(w[j] / d);
    if (q > 127.0f) q = 127.0f;
    if (q < -127.0f) q = -127.0f;
    blk[2 + j] = (uint8_t)(int8_t)q;
  }
}

static void quantize_q4_sm_block(const float* w, uint8_t* blk) {
  float lo = w[0], hi = w[0];
  for (int j = 1; j < 32; ++j) {
    lo = fminf(lo, w[j]);
    hi = fmaxf(hi, w[j]);
  }
  const uint16_t mh = or_f16_from_f32(lo);
  const float m = or_f32_from_f16(mh);
  const uint16_t dh = or_f16_from_f32((hi - m) / 15.0f);
  const float d = or_f32_from_f16(dh);
  put16(blk, dh);
  put16(blk + 2, mh);
  uint8_t q[32];
  for (int j = 0; j < 32; ++j) {
    float v = d == 0.0f ? 0.0f : roundf((w[j] - m) / d);
    if (v < 0.0f) v = 0.0f;
    if (v > 15.0f) v = 15.0f;
    q[j] = (uint8_t)v;
  }
  for (int i = 0; i < 16; ++i) blk[4 + i] = (uint8_t)(q[2 * i] | (q[2 * i + 1] << 4));
}

/* ------------------------------------------------------------------------ */
/* q4_K: a super-block of 256 weights in 8 sub-blocks of 32, each with a     */
/* 6-bit scale and a 6-bit minimum, under two fp16 super-scales (Deep        */
/* Technical Design, section 5: 4.5 bits per weight).  The page gives no     */
/* more than that; the reading taken here:                                   */
/*   sub-block j has step D_j = d * sc_j and offset M_j = dmin * m_j, with   */
/*   sc_j, m_j in 0..63, and a weight is w = D_j * q - M_j, q in 0..15;       */
/*   bytes (144): [d fp16][dmin fp16][12 B of sixteen 6-bit codes: code i    */
/*   in bits 6i..6i+5 of the 96-bit little-endian field, codes 0..7 are      */
/*   sc_0..sc_7 and 8..15 are m_0..m_7][128 B: sub-block j's 16 bytes at     */
/*   offset 16 + 16j, byte i = q[32j + 2i] | q[32j + 2i + 1] << 4].           */
/* Quantiser, per sub-block: lo = min(0, min w), hi = max w,                  */
/* s = (hi - lo)/15, t = 0 - lo; then d = fp16(max s / 63),                   */
/* dmin = fp16(max t / 63); sc = min(63, ceil(s/d)) (the smallest code whose */
/* step covers the range), m = min(63, round(t/dmin)) (codes 0 when their    */
/* super-scale is 0); q = clamp(round((w + M)/D), 0, 15), or 0 when D = 0.   */
/* ------------------------------------------------------------------------ */

static void put_code6(uint8_t* field, int i, unsigned v) {
  for (int b = 0; b < 6; ++b)
    if ((v >> b) & 1u) {
      const int bit = 6 * i + b;
      field[bit >> 3] |= (uint8_t)(1u << (bit & 7));
    }
}

static unsigned get_code6(const uint8_t* field, int i) {
  unsigned v = 0;
  for (int b = 0; b < 6; ++b) {
    const int bit = 6 * i + b;
    v |= (unsigned)((field[bit >> 3] >> (bit & 7)) & 1u) << b;
  }
  return v;
}

static void quantize_q4_k_block(const float* w, uint8_t* blk) {
  float s[8], t[8], smax = 0.0f, tmax = 0.0f;
  for (int j = 0; j < 8; ++j) {
    float lo = 0.0f, hi = w[32 * j];
    for (int i = 0; i < 32; ++i) {
      lo = fminf(lo, w[32 * j + i]);
      hi = fmaxf(hi, w[32 * j + i]);
    }
    s[j] = (hi - lo) / 15.0f;
    t[j] = 0.0f - lo; /* +0 for lo = 0, so a zero block stores dmin = +0 */
    smax = fmaxf(smax, s[j]);
    tmax = fmaxf(tmax, t[j]);
  }
  const uint16_t dh = or_f16_from_f32(smax / 63.0f);
  const uint16_t mh = or_f16_from_f32(tmax / 63.0f);
  const float d = or_f32_from_f16(dh), dmin = or_f32_from_f16(mh);
  memset(blk, 0, 144);
  put16(blk, dh);
  put16(blk + 2, mh);
  for (int j = 0; j < 8; ++j) {
    float sc = d == 0.0f ? 0.0f : ceilf(s[j] / d);
    float mc = dmin == 0.0f ? 0.0f : roundf(t[j] / dmin);
    if (sc > 63.0f) sc = 63.0f;
    if (mc > 63.0f) mc = 63.0f;
    put_code6(blk + 4, j, (unsigned)sc);
    put_code6(blk + 4, 8 + j, (unsigned)mc);
    const float D = d * sc, M = dmin * mc;
    uint8_t q[32];
    for (int i = 0; i < 32; ++i) {
      float v = D == 0.0f ? 0.0f : roundf((w[32 * j + i] + M) / D);
      if (v < 0.0f) v = 0.0f;
      if (v > 15.0f) v = 15.0f;
      q[i] = (uint8_t)v;
    }
    for (int i = 0; i < 16; ++i) blk[16 + 16 * j + i] = (uint8_t)(q[2 * i] | (q[2 * i + 1] << 4));
  }
}

typedef struct {
  int32_t qtype;
  const float* w;
  int64_t k;
  uint8_t* blocks;
} quant_ctx;

static void quant_row(void* vc, int64_t r, double* unused) {
  const quant_ctx* c = (const quant_ctx*)vc;
  (void)unused;
  const int32_t bw = or_block_weights(c->qtype);
  const int64_t nb = c->k / bw;
  const int32_t bb = or_block_bytes(c->qtype);
  for (int64_t b = 0; b < nb; ++b) {
    const float* src = c->w + r * c->k + b * bw;
    uint8_t* dst = c->blocks + (r * nb + b) * bb;
    if (c->qtype == OR_Q8_0)
      quantize_q8_0_block(src, dst);
    else if (c->qtype == OR_Q4_SM)
      quantize_q4_sm_block(src, dst);
    else
      quantize_q4_k_block(src, dst);
  }
}

static int32_t for_rows(int64_t n_rows, int32_t nthreads, int64_t scratch_len,
                        void (*fn)(void*, int64_t, double*), void* ctx);

int32_t or_quantize(int32_t qtype, const float* w, int64_t n, int64_t k, uint8_t* blocks) {
  const int32_t bb = or_block_bytes(qtype);
  if (!bb || !w || !blocks || n < 0 || k <= 0 || k % or_block_weights(qtype)) return -1;
  quant_ctx c = {qtype, w, k, blocks};
  return for_rows(n, 0, 0, quant_row, &c);
}

/* Dequantise one row into float64: exact, since d*q has at most 15
 * significant bits and d*q + m fits easily in 53 (q4_K: d*sc*q has at most
 * 21 and dmin*m at most 17). */
static void dequant_row(int32_t qtype, const uint8_t* blocks, int64_t row, int64_t k,
                        double* out) {
  const int32_t bw = or_block_weights(qtype);
  const int64_t nb = k / bw;
  const int32_t bb = or_block_bytes(qtype);
  for (int64_t b = 0; b < nb; ++b) {
    const uint8_t* blk = blocks + (row * nb + b) * bb;
    const double d = (double)or_f32_from_f16(get16(blk));
    if (qtype == OR_Q8_0) {
      for (int j = 0; j < 32; ++j) out[b * 32 + j] = d * (double)(int8_t)blk[2 + j];
    } else if (qtype == OR_Q4_K) {
      const double dmin = (double)or_f32_from_f16(get16(blk + 2));
      for (int j = 0; j < 8; ++j) {
        const double D = d * (double)get_code6(blk + 4, j);
        const double M = dmin * (double)get_code6(blk + 4, 8 + j);
        for (int i = 0; i < 16; ++i) {
          const uint8_t byte = blk[16 + 16 * j + i];
          out[b * 256 + 32 * j + 2 * i] = D * (double)(byte & 0x0F) - M;
          out[b * 256 + 32 * j + 2 * i + 1] = D * (double)(byte >> 4) - M;
        }
      }
    } else {
      const double m = (double)or_f32_from_f16(get16(blk + 2));
      for (int i = 0; i < 16; ++i) {
        out[b * 32 + 2 * i] = d * (double)(blk[4 + i] & 0x0F) + m;
        out[b * 32 + 2 * i + 1] = d * (double)(blk[4 + i] >> 4) + m;
      }
    }
  }
}

int32_t or_dequantize(int32_t qtype, const uint8_t* blocks, int64_t n, int64_t k, double* out) {
  if (!or_block_bytes(qtype) || !blocks || !out || n < 0 || k <= 0 || k % or_block_weights(qtype))
    return -1;
  for (int64_t r = 0; r < n; ++r) dequant_row(qtype, blocks, r, k, out + r * k);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Row-parallel driver.                                                      */
/* ------------------------------------------------------------------------ */

int32_t or_default_threads(void) {
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  const char* env = getenv("OMP_NUM_THREADS");
  if (env && atoi(env) > 0 && atoi(env) < n) n = atoi(env);
  if (n < 1) n = 1;
  if (n > 256) n = 256;
  return (int32_t)n;
}

typedef void (*row_fn)(void* ctx, int64_t i, double* scratch);
typedef struct {
  row_fn fn;
  void* ctx;
  int64_t begin, end, scratch_len;
  int failed;
} row_job;

static void* row_worker(void* p) {
  row_job* j = (row_job*)p;
  double* scratch = j->scratch_len ? (double*)malloc(sizeof(double) * j->scratch_len) : NULL;
  if (j->scratch_len && !scratch) {
    j->failed = 1;
    return NULL;
  }
  for (int64_t i = j->begin; i < j->end; ++i) j->fn(j->ctx, i, scratch);
  free(scratch);
  return NULL;
}

static int32_t for_rows(int64_t n_rows, int32_t nthreads, int64_t scratch_len, row_fn fn,
                        void* ctx) {
  if (nthreads <= 0) nthreads = or_default_threads();
  if (nthreads > 256) nthreads = 256;
  if (n_rows < 2 * nthreads) nthreads = n_rows > 0 ? (int32_t)(n_rows < 256 ? n_rows : 256) : 1;
  pthread_t th[256];
  row_job jobs[256];
  int started[256];
  const int64_t per = (n_rows + nthreads - 1) / (nthreads ? nthreads : 1);
  int failed = 0;
  for (int t = 0; t < nthreads; ++t) {
    int64_t b = per * t, e = b + per;
    if (b > n_rows) b = n_rows;
    if (e > n_rows) e = n_rows;
    jobs[t] = (row_job){fn, ctx, b, e, scratch_len, 0};
    started[t] = pthread_create(&th[t], NULL, row_worker, &jobs[t]) == 0;
    if (!started[t]) row_worker(&jobs[t]);
  }
  for (int t = 0; t < nthreads; ++t) {
    if (started[t]) pthread_join(th[t], NULL);
    failed |= jobs[t].failed;
  }
  return failed ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Dual path (Deep Technical Design, section 1: base and overlay evaluated as */
/* parallel streams; section 8: dual path for decode; overlay page, "Native/ */
/* WASM Kernel Implications": y = xW + x(BA) via the shrink x A^T then the    */
/* expand).  Adapters enter in list order after the base sum (section 9:     */
/* weighted mixtures at the final accumulation step).                         */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t qtype;
  const uint8_t* blocks;
  int64_t n, k;
  const double* x;
  int32_t batch;
  const or_lora* ads;
  int32_t n_ads;
  const int64_t* rows;
  int64_t n_rows;
  double* y;
  const double* t; /* shrink results: per adapter, batch x rank, concatenated */
  const uint16_t* X16;
  const uint16_t* W16;
  uint16_t* weff;
} lin_ctx;

static int64_t row_of(const lin_ctx* c, int64_t i) { return c->rows ? c->rows[i] : i; }

static double* shrink_all(const double* x, int32_t batch, int64_t k, const or_lora* ads,
                          int32_t n_ads) {
  int64_t total = 0;
  for (int a = 0; a < n_ads; ++a) total += (int64_t)batch * ads[a].rank;
  double* t = (double*)calloc(total ? total : 1, sizeof(double));
  if (!t) return NULL;
  int64_t off = 0;
  for (int a = 0; a < n_ads; ++a) {
    for (int32_t b = 0; b < batch; ++b)
      for (int32_t j = 0; j < ads[a].rank; ++j) {
        double s = 0.0;
        const float* arow = ads[a].A + (int64_t)j * k;
        for (int64_t kk = 0; kk < k; ++kk) s += (double)arow[kk] * x[(int64_t)b * k + kk];
        t[off + (int64_t)b * ads[a].rank + j] = s;
      }
    off += (int64_t)batch * ads[a].rank;
  }
  return t;
}

static void dual_row(void* vc, int64_t i, double* wrow) {
  const lin_ctx* c = (const lin_ctx*)vc;
  const int64_t r = row_of(c, i);
  dequant_row(c->qtype, c->blocks, r, c->k, wrow);
  for (int32_t b = 0; b < c->batch; ++b) {
    const double* xb = c->x + (int64_t)b * c->k;
    double acc = 0.0;
    for (int64_t kk = 0; kk < c->k; ++kk) acc += wrow[kk] * xb[kk];
    int64_t off = 0;
    for (int32_t a = 0; a < c->n_ads; ++a) {
      const or_lora* ad = &c->ads[a];
      double e = 0.0;
      if (ad->rank == 0) { /* sparse delta: S[r] . x */
        for (uint32_t p = ad->row_ptr[r]; p < ad->row_ptr[r + 1]; ++p)
          e += (double)or_f32_from_f16(ad->val[p]) * xb[ad->col[p]];
      } else {
        const double* tb = c->t + off + (int64_t)b * ad->rank;
        for (int32_t j = 0; j < ad->rank; ++j) e += (double)ad->B[r * ad->rank + j] * tb[j];
      }
      acc += (double)ad->scale * e;
      off += (int64_t)c->batch * ad->rank;
    }
    c->y[(int64_t)b * c->n_rows + i] = acc;
  }
}

static int32_t check_lin(int32_t qtype, const uint8_t* blocks, int64_t n, int64_t k,
                         const or_lora* ads, int32_t n_ads, const int64_t* rows, int64_t n_rows) {
  if (!or_block_bytes(qtype) || !blocks || n <= 0 || k <= 0 || k % or_block_weights(qtype) ||
      n_ads < 0)
    return -1;
  if (n_ads && !ads) return -1;
  for (int32_t a = 0; a < n_ads; ++a) {
    if (ads[a].rank < 0) return -1;
    if (ads[a].rank > 0 && (!ads[a].A || !ads[a].B)) return -1;
    if (ads[a].rank == 0) {
      if (!ads[a].row_ptr || (ads[a].row_ptr[n] && (!ads[a].col || !ads[a].val))) return -1;
      for (int64_t r = 0; r < n; ++r)
        if (ads[a].row_ptr[r] > ads[a].row_ptr[r + 1]) return -1;
      for (uint32_t p = 0; p < ads[a].row_ptr[n]; ++p)
        if ((int64_t)ads[a].col[p] >= k) return -1;
    }
  }
  if (!rows && n_rows != n) return -1;
  if (rows)
    for (int64_t i = 0; i < n_rows; ++i)
      if (rows[i] < 0 || rows[i] >= n) return -1;
  return 0;
}

int32_t or_linear_dual(int32_t qtype, const uint8_t* blocks, int64_t n, int64_t k,
                       const double* x, int32_t batch, const or_lora* ads, int32_t n_ads,
                       const int64_t* rows, int64_t n_rows, double* y, int32_t nthreads) {
  if (check_lin(qtype, blocks, n, k, ads, n_ads, rows, n_rows) || !x || !y || batch <= 0)
    return -1;
  double* t = shrink_all(x, batch, k, ads, n_ads);
  if (!t) return -1;
  lin_ctx c = {qtype, blocks, n, k, x, batch, ads, n_ads, rows, n_rows, y, t, NULL, NULL, NULL};
  const int32_t rc = for_rows(n_rows, nthreads, k, dual_row, &c);
  free(t);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Materialised path: W_eff = dequant(W_q) + sum_a s_a B_a A_a (overlay page, */
/* "Compositional Integrity" invariant and the fresh-base oracle; Deep        */
/* Technical Design section 5: W_q is never recomputed, the sum lives only in */
/* an ephemeral buffer).  Here one float64 row at a time.                     */
/* ------------------------------------------------------------------------ */

static void weff_row_f64(const lin_ctx* c, int64_t r, double* wrow) {
  dequant_row(c->qtype, c->blocks, r, c->k, wrow);
  for (int32_t a = 0; a < c->n_ads; ++a) {
    const or_lora* ad = &c->ads[a];
    if (ad->rank == 0)
      for (uint32_t p = ad->row_ptr[r]; p < ad->row_ptr[r + 1]; ++p)
        wrow[ad->col[p]] += (double)ad->scale * (double)or_f32_from_f16(ad->val[p]);
    for (int32_t j = 0; j < ad->rank; ++j) {
      const double sb = (double)ad->scale * (double)ad->B[r * ad->rank + j];
      const float* arow = ad->A + (int64_t)j * c->k;
      for (int64_t kk = 0; kk < c->k; ++kk) wrow[kk] += sb * (double)arow[kk];
    }
  }
}

static void mat_row(void* vc, int64_t i, double* wrow) {
  const lin_ctx* c = (const lin_ctx*)vc;
  weff_row_f64(c, row_of(c, i), wrow);
  for (int32_t b = 0; b < c->batch; ++b) {
    const double* xb = c->x + (int64_t)b * c->k;
    double acc = 0.0;
    for (int64_t kk = 0; kk < c->k; ++kk) acc += wrow[kk] * xb[kk];
    c->y[(int64_t)b * c->n_rows + i] = acc;
  }
}

int32_t or_linear_materialised(int32_t qtype, const uint8_t* blocks, int64_t n, int64_t k,
                               const double* x, int32_t batch, const or_lora* ads,
                               int32_t n_ads, const int64_t* rows, int64_t n_rows, double* y,
                               int32_t nthreads) {
  if (check_lin(qtype, blocks, n, k, ads, n_ads, rows, n_rows) || !x || !y || batch <= 0)
    return -1;
  lin_ctx c = {qtype, blocks, n, k, x, batch, ads, n_ads, rows, n_rows, y, NULL, NULL, NULL, NULL};
  return for_rows(n_rows, nthreads, k, mat_row, &c);
}

/* ------------------------------------------------------------------------ */
/* Per-layer JIT materialisation for prefill (Deep Technical Design, section */
/* 8: prefill is a GEMM, so materialise the layer; section 1: the layer is   */
/* built in scratch, used, discarded).  The scratch holds bfloat16 operands  */
/* for a bf16 matrix-core GEMM with float accumulation: the adapter factors  */
/* are rounded to bf16 (scale folded into B first, in float32), their        */
/* products summed exactly onto float32(dequant), and the sum rounded once.  */
/* ------------------------------------------------------------------------ */

static void jit_row(void* vc, int64_t i, double* acc) {
  const lin_ctx* c = (const lin_ctx*)vc;
  const int64_t r = row_of(c, i);
  dequant_row(c->qtype, c->blocks, r, c->k, acc);
  for (int64_t kk = 0; kk < c->k; ++kk) acc[kk] = (double)(float)acc[kk]; /* float32(deq) */
  for (int32_t a = 0; a < c->n_ads; ++a) {
    const or_lora* ad = &c->ads[a];
    if (ad->rank == 0)
      for (uint32_t p = ad->row_ptr[r]; p < ad->row_ptr[r + 1]; ++p)
        acc[ad->col[p]] += (double)(ad->scale * or_f32_from_f16(ad->val[p]));
    for (int32_t j = 0; j < ad->rank; ++j) {
      const float sb32 = ad->scale * ad->B[r * ad->rank + j];
      const double sb = (double)or_f32_from_bf16(or_bf16_from_f32(sb32));
      const float* arow = ad->A + (int64_t)j * c->k;
      for (int64_t kk = 0; kk < c->k; ++kk)
        acc[kk] += sb * (double)or_f32_from_bf16(or_bf16_from_f32(arow[kk]));
    }
  }
  for (int64_t kk = 0; kk < c->k; ++kk) c->weff[i * c->k + kk] = or_bf16_from_f64(acc[kk]);
}

int32_t or_jit_weff(int32_t qtype, const uint8_t* blocks, int64_t n, int64_t k,
                    const or_lora* ads, int32_t n_ads, const int64_t* rows, int64_t n_rows,
                    uint16_t* weff, int32_t nthreads) {
  if (check_lin(qtype, blocks, n, k, ads, n_ads, rows, n_rows) || !weff) return -1;
  lin_ctx c = {qtype, blocks, n, k, NULL, 0, ads, n_ads, rows, n_rows, NULL, NULL, NULL, NULL, weff};
  return for_rows(n_rows, nthreads, k, jit_row, &c);
}

/* ------------------------------------------------------------------------ */
/* Dequantize-add-requantize, the destructive merge the overlay avoids       */
/* (overlay page, "Quantized-Base Numerical Analysis"; Deep Technical Design, */
/* "The Pathology of Dequantize-Add-Requantize (DAR) Error"): the merged      */
/* float32 weight of each element, then the base format's quantiser.  The    */
/* merged weight follows one fixed float32 recipe, so that a GPU kernel can  */
/* reach the same codes:                                                     */
/*   w = f32(deq(W)[r][k]);                                                  */
/*   for each adapter in list order:                                        */
/*     LoRA:   u = 0; for j = 0..rank-1: u = fma(B[r][j], A[j][k], u);        */
/*             w = fma(scale, u, w)                                          */
/*     sparse: if (r, k) is an entry with value v: w = fma(scale, f32(v), w)  */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t qtype;
  const uint8_t* blocks;
  int64_t k;
  const or_lora* ads;
  int32_t n_ads;
  uint8_t* out;
} dar_ctx;

static void dar_row(void* vc, int64_t r, double* tmp) {
  const dar_ctx* c = (const dar_ctx*)vc;
  const int64_t k = c->k;
  float* w = (float*)malloc((size_t)k * sizeof(float));
  if (!w) return;
  dequant_row(c->qtype, c->blocks, r, k, tmp);
  for (int64_t kk = 0; kk < k; ++kk) w[kk] = (float)tmp[kk];
  for (int32_t a = 0; a < c->n_ads; ++a) {
    const or_lora* ad = &c->ads[a];
    if (ad->rank == 0) {
      for (uint32_t p = ad->row_ptr[r]; p < ad->row_ptr[r + 1]; ++p)
        w[ad->col[p]] = fmaf(ad->scale, or_f32_from_f16(ad->val[p]), w[ad->col[p]]);
      continue;
    }
    for (int64_t kk = 0; kk < k; ++kk) {
      float u = 0.0f;
      for (int32_t j = 0; j < ad->rank; ++j) u = fmaf(ad->B[r * ad->rank + j], ad->A[(int64_t)j * k + kk], u);
      w[kk] = fmaf(ad->scale, u, w[kk]);
    }
  }
  const int32_t bw = or_block_weights(c->qtype), bb = or_block_bytes(c->qtype);
  const int64_t nb = k / bw;
  for (int64_t b = 0; b < nb; ++b) {
    uint8_t* dst = c->out + (r * nb + b) * bb;
    if (c->qtype == OR_Q8_0)
      quantize_q8_0_block(w + b * bw, dst);
    else if (c->qtype == OR_Q4_SM)
      quantize_q4_sm_block(w + b * bw, dst);
    else
      quantize_q4_k_block(w + b * bw, dst);
  }
  free(w);
}

int32_t or_requantize(int32_t qtype, const uint8_t* blocks, int64_t n, int64_t k, const or_lora* ads,
                      int32_t n_ads, uint8_t* blocks_out, int32_t nthreads) {
  if (check_lin(qtype, blocks, n, k, ads, n_ads, NULL, n) || !blocks_out) return -1;
  dar_ctx c = {qtype, blocks, k, ads, n_ads, blocks_out};
  return for_rows(n, nthreads, k, dar_row, &c);
}

typedef struct {
  const uint16_t* X;
  int64_t m;
  const uint16_t* W;
  int64_t n_rows, k;
  double* y;
} gemm_ctx;

static void gemm_row(void* vc, int64_t i, double* xs) {
  const gemm_ctx* c = (const gemm_ctx*)vc;
  (void)xs;
  const uint16_t* w = c->W + i * c->k;
  for (int64_t mm = 0; mm < c->m; ++mm) {
    const uint16_t* xr = c->X + mm * c->k;
    double acc = 0.0;
    for (int64_t kk = 0; kk < c->k; ++kk)
      acc += (double)or_f32_from_bf16(xr[kk]) * (double)or_f32_from_bf16(w[kk]);
    c->y[mm * c->n_rows + i] = acc;
  }
}

int32_t or_gemm_bf16(const uint16_t* X, int64_t m, const uint16_t* weff, int64_t n_rows,
                     int64_t k, double* y, int32_t nthreads) {
  if (!X || !weff || !y || m <= 0 || n_rows <= 0 || k <= 0) return -1;
  gemm_ctx c = {X, m, weff, n_rows, k, y};
  return for_rows(n_rows, nthreads, 0, gemm_row, &c);
}

/* ------------------------------------------------------------------------ */
/* Block of linears and the decode stack.  The pages give no block topology  */
/* beyond "linears only"; the glue read here is linear: sums of parallel     */
/* projections and RMS scaling between stages (eps 1e-6).                    */
/* ------------------------------------------------------------------------ */

void or_rms(const double* v, int64_t n, double eps, double* out) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) ss += v[i] * v[i];
  const double inv = 1.0 / sqrt(ss / (double)n + eps);
  for (int64_t i = 0; i < n; ++i) out[i] = v[i] * inv;
}

static int32_t run_lin(const or_linear_t* L, const double* x, double* y, int32_t nthreads) {
  return or_linear_dual(L->qtype, L->blocks, L->n, L->k, x, 1, L->ads, L->n_ads, NULL, L->n, y,
                        nthreads);
}

int32_t or_block(const or_linear_t* L, const double* h, double* out, int32_t nthreads) {
  if (!L || !h || !out) return -1;
  const int64_t d = L[0].k, hd = L[4].n;
  /* shape contract: q,k,v,o are d x d, gate/up hd x d, down d x hd */
  for (int i = 0; i < 4; ++i)
    if (L[i].n != d || L[i].k != d) return -1;
  if (L[5].n != hd || L[4].k != d || L[5].k != d || L[6].n != d || L[6].k != hd) return -1;
  double* buf = (double*)malloc(sizeof(double) * (size_t)(6 * d + 3 * hd));
  if (!buf) return -1;
  double *q = buf, *kk = q + d, *v = kk + d, *s = v + d, *a = s + d, *dd = a + d;
  double *g = dd + d, *u = g + hd, *gs = u + hd;
  int32_t rc = 0;
  rc |= run_lin(&L[0], h, q, nthreads);
  rc |= run_lin(&L[1], h, kk, nthreads);
  rc |= run_lin(&L[2], h, v, nthreads);
  for (int64_t i = 0; i < d; ++i) s[i] = q[i] + kk[i] + v[i];
  or_rms(s, d, 1e-6, s);
  rc |= run_lin(&L[3], s, a, nthreads);
  or_rms(a, d, 1e-6, s);
  rc |= run_lin(&L[4], s, g, nthreads);
  rc |= run_lin(&L[5], s, u, nthreads);
  for (int64_t i = 0; i < hd; ++i) gs[i] = g[i] + u[i];
  or_rms(gs, hd, 1e-6, gs);
  rc |= run_lin(&L[6], gs, dd, nthreads);
  or_rms(dd, d, 1e-6, out);
  free(buf);
  return rc ? -1 : 0;
}

int32_t or_stack(const or_linear_t* L, int32_t n_blocks, const double* x0, int32_t n_tokens,
                 double* y, int32_t nthreads) {
  if (!L || n_blocks <= 0 || !x0 || n_tokens <= 0 || !y) return -1;
  const int64_t d = L[0].k;
  double* h = (double*)malloc(sizeof(double) * (size_t)(2 * d));
  if (!h) return -1;
  double* h2 = h + d;
  memcpy(h, x0, sizeof(double) * (size_t)d);
  for (int32_t t = 0; t < n_tokens; ++t) {
    for (int32_t b = 0; b < n_blocks; ++b) {
      if (or_block(L + 7 * b, h, h2, nthreads)) {
        free(h);
        return -1;
      }
      memcpy(h, h2, sizeof(double) * (size_t)d);
    }
    memcpy(y + (int64_t)t * d, h, sizeof(double) * (size_t)d);
  }
  free(h);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Array forms of the conversions (for the tests).                          */
/* ------------------------------------------------------------------------ */

void or_f16_from_f32_n(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = or_f16_from_f32(in[i]);
}
void or_f32_from_f16_n(const uint16_t* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = or_f32_from_f16(in[i]);
}
void or_bf16_from_f32_n(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = or_bf16_from_f32(in[i]);
}
void or_bf16_from_f64_n(const double* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = or_bf16_from_f64(in[i]);
}
