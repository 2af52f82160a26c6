/*
 * CPU oracle for the dual-path quantized-base + LoRA linear.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg may load or call this code.  It shares no code,
 * header, table or helper with the GPU library and includes nothing from it.
 *
 * Plain, slow, obviously correct: float64 arithmetic, sequential reductions,
 * parallel only across output rows.  The functions follow the three pages on
 * quantized-base adapter overlays (mikekappel.com "We propose a
 * content-addressed overlay system", mikekappel.com "Deep Technical Design:
 * Exact, Atomic, Reversible Specialist Overlays", contenox.com "LoRA
 * adapters"); each definition names the passage it follows.
 */
#ifndef QBL_ORACLE_H
#define QBL_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { OR_Q8_0 = 1, OR_Q4_SM = 2, OR_Q4_K = 3 };

/* IEEE 754 binary16 / bfloat16 conversions, round to nearest even. */
uint16_t or_f16_from_f32(float f);
float or_f32_from_f16(uint16_t h);
uint16_t or_bf16_from_f32(float f);
uint16_t or_bf16_from_f64(double v);
float or_f32_from_bf16(uint16_t b);

/* Bytes of one block: q8_0 34, q4_sm 20, q4_K 144; 0 for an unknown type. */
int32_t or_block_bytes(int32_t qtype);
/* Weights of one block: 32 (q8_0, q4_sm) or 256 (q4_K); 0 for an unknown type. */
int32_t or_block_weights(int32_t qtype);

/* Quantise a row-major n x k float32 matrix (k a multiple of the block's
 * weights) into canonical blocks: rows in order, blocks along k within a row.
 *   q8_0 block : [fp16 d little-endian][32 x int8 q]                   34 B
 *   q4_sm block: [fp16 d][fp16 m][16 B, byte i = q[2i] | q[2i+1] << 4]  20 B
 *   q4_K block : [fp16 d][fp16 dmin][12 B of 6-bit codes][128 B nibbles] 144 B
 *                (256 weights; the layout and quantiser are spelled out in oracle.c)
 * Returns 0, or -1 on a bad argument. */
int32_t or_quantize(int32_t qtype, const float* w, int64_t n, int64_t k, uint8_t* blocks);

/* Dequantise to float64 (exact for both formats). */
int32_t or_dequantize(int32_t qtype, const uint8_t* blocks, int64_t n, int64_t k, double* out);

/* One adapter on one linear, applied with the single effective multiplier
 * `scale` (alpha/r folded).
 * rank >= 1: a LoRA pair, A rank x k_in and B n_out x rank, row-major float32.
 * rank == 0: a sparse delta S (n_out x k_in) in CSR form (the design page's
 *   "Sparse Overlay Bytes": 4-byte indices, 2-byte f16 values): row r holds
 *   entries row_ptr[r] .. row_ptr[r+1]-1 with columns col[] and fp16 values
 *   val[] (bit patterns).  A and B are unused. */
typedef struct {
  int32_t rank;
  float scale;
  const float* A;
  const float* B;
  const uint32_t* row_ptr;
  const uint32_t* col;
  const uint16_t* val;
} or_lora;

/* Dual path, float64:
 *   y[b][i] = sum_k deq(W)[row_i][k] x[b][k]
 *           + sum_a scale_a * sum_j B_a[row_i][j] * (sum_k A_a[j][k] x[b][k])   (LoRA)
 *           + sum_a scale_a * sum_p val_a[p] x[b][col_a[p]]  over row_i's entries (sparse)
 * with the base sum completed first and the adapters added in list order.
 * x is batch x k (float64).  rows lists the output rows to compute (NULL with
 * n_rows = n means all rows); y is batch x n_rows.  nthreads <= 0 picks the
 * default.  Returns 0 or -1. */
int32_t or_linear_dual(int32_t qtype, const uint8_t* blocks, int64_t n, int64_t k,
                       const double* x, int32_t batch, const or_lora* ads, int32_t n_ads,
                       const int64_t* rows, int64_t n_rows, double* y, int32_t nthreads);

/* Materialised path, float64: W_eff = deq(W) + sum_a scale_a B_a A_a formed
 * row by row, then y = W_eff x.  Same arguments as or_linear_dual. */
int32_t or_linear_materialised(int32_t qtype, const uint8_t* blocks, int64_t n, int64_t k,
                               const double* x, int32_t batch, const or_lora* ads,
                               int32_t n_ads, const int64_t* rows, int64_t n_rows, double* y,
                               int32_t nthreads);

/* Per-layer just-in-time materialisation in bfloat16:
 *   weff[i][k] = bf16( f32(deq(W)[row_i][k])
 *                      + sum_a sum_j bf16(f32(scale_a*B_a[row_i][j])) * bf16(A_a[j][k])   (LoRA)
 *                      + sum_a f32(scale_a * val_a) at (row_i, col_a)                      (sparse) )
 * with the sum formed exactly (float64) and rounded once. weff is n_rows x k. */
int32_t or_jit_weff(int32_t qtype, const uint8_t* blocks, int64_t n, int64_t k,
                    const or_lora* ads, int32_t n_ads, const int64_t* rows, int64_t n_rows,
                    uint16_t* weff, int32_t nthreads);

/* y[m][i] = sum_k X[m][k] * weff[i][k] in float64; X (m x k) and weff
 * (n_rows x k) are bfloat16 bit patterns. */
int32_t or_gemm_bf16(const uint16_t* X, int64_t m, const uint16_t* weff, int64_t n_rows,
                     int64_t k, double* y, int32_t nthreads);

/* Dequantize-add-requantize (the destructive merge the overlay avoids): the
 * base format's quantiser applied to the float32 merged weight
 *   w = f32(deq(W)[r][k]), then per adapter in list order
 *   LoRA   w = fma(scale, u, w), u = fma chain over j = 0..rank-1 of B[r][j]*A[j][k]
 *   sparse w = fma(scale, f32(val), w) at the delta's entries.
 * blocks_out: n x k/block_weights canonical blocks.  Returns 0 or -1. */
int32_t or_requantize(int32_t qtype, const uint8_t* blocks, int64_t n, int64_t k, const or_lora* ads,
                      int32_t n_ads, uint8_t* blocks_out, int32_t nthreads);

/* RMS scaling: out = v / sqrt(mean(v^2) + eps). */
void or_rms(const double* v, int64_t n, double eps, double* out);

/* One linear of a block. */
typedef struct {
  int32_t qtype;
  int64_t n, k;
  const uint8_t* blocks;
  const or_lora* ads;
  int32_t n_ads;
} or_linear_t;

/* One block of linears (q, k, v, o, gate, up, down) at batch 1:
 *   q,k,v = L(h); a = L_o(rms(q+k+v)); g,u = L_gate/up(rms(a));
 *   d = L_down(rms(g+u)); out = rms(d)          (eps 1e-6) */
int32_t or_block(const or_linear_t* L, const double* h, double* out, int32_t nthreads);

/* A stack of n_blocks blocks (7 linears each) decoding n_tokens tokens:
 * token 0 enters with x0, token t+1 with the output of token t.
 * y is n_tokens x d (the output of each token). */
int32_t or_stack(const or_linear_t* L, int32_t n_blocks, const double* x0, int32_t n_tokens,
                 double* y, int32_t nthreads);

/* Array forms of the conversions. */
void or_f16_from_f32_n(const float* in, uint16_t* out, int64_t n);
void or_f32_from_f16_n(const uint16_t* in, float* out, int64_t n);
void or_bf16_from_f32_n(const float* in, uint16_t* out, int64_t n);
void or_bf16_from_f64_n(const double* in, uint16_t* out, int64_t n);

/* Threads used when nthreads <= 0: online cores, capped by OMP_NUM_THREADS. */
int32_t or_default_threads(void);

#ifdef __cplusplus
}
#endif
#endif
