// Decode at batch 2..8 on the matrix cores (gfx950).
//
// The base product of the dual path for a few inputs ("Deep Technical Design",
// section 8: the decode GEMV), y[b][n] = sum_k deq(W)[n][k] x[b][k], is a skinny
// matrix product: every 32-weight block is one v_mfma_f32_16x16x32_f16 with the
// block's integer codes as the B operand (16 weight rows) and the inputs as the
// A operand (16 rows).  The block's scale and minimum multiply float32 results,
// so no weight is ever rounded:
//   y[b][n] = 2^e_b sum_blk ( d[n][blk] S[b][n][blk] + m[n][blk] X[b][blk] ),
//   S = sum over the block of code * x', X = sum over the block of x',
// with x' = x 2^-e_b, e_b chosen per batch row so that its largest |x'| lies in
// [2^14, 2^15).  Each x' is split into two f16 values, x' = hi + lo + r with
// hi = f16(x'), lo = f16(x' - hi), |r| <= 2^-22 |x'| (plus an absolute 2^-25
// where lo is subnormal), so the products carry float32-level precision: the A
// operand's 16 rows are hi of batch rows 0..7 and lo of batch rows 0..7, and
// the two halves of the result are added at the end.  X is the float32 sum of
// x' itself.  Low-rank and sparse terms follow in float32, in list order.
//
// Codes enter as exact f16 integers.  q8_0 codes are stored offset-binary
// (u = q + 128): a byte permute puts u under the f16 exponent of 1024, and one
// subtraction per pair leaves q.  q4 codes go through the gfx950 fp8 (e4m3)
// conversion: a byte c < 16 is the e4m3 value c 2^-9 (subnormals and the first
// binade share one spacing), so the conversion with scale 2^9 yields c exactly,
// two codes per instruction.  (Codes as f16 subnormals, c 2^-24, would need no
// conversion at all, but measured on the device each instruction's sum then
// loses about 2^-20 relative, against 2^-26 with normal codes.)  Scales and
// minima are converted to float32 once per slab (below), and for the q4
// formats the minimum terms of a slab's blocks, sum_blk m[n][blk] X[b][blk],
// are one v_mfma_f32_16x16x4_f32 per 16-row tile (X in A, m in B, float32).
//
// v_mfma_f32_16x16x32_f16 lanes (checked on the device): A lane l holds row
// l % 16, inputs 8 (l / 16) .. +7; B lane l holds column l % 16, the same
// inputs; D lane l holds rows 4 (l / 16) + j, j = 0..3, of column l % 16.  The
// order of the 32 inputs inside one instruction is free as long as A and B
// agree, which the q4 formats use to unpack nibbles with two masks (below).
// v_mfma_f32_16x16x4_f32: A lane l holds A[l % 16][l / 16], B lane l holds
// B[l / 16][l % 16], D as above (checked on the device).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "qbl_device.h"
#include "qbl_kernels.h"

namespace qbl {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

// Waves of a GEMV workgroup, splitting the blocks of K: 8 for the q4 formats
// (two workgroups of 8 waves per compute unit ran the 70B MLP at batch 8 2.5 %
// (q4_sm) and 3 % (q4_K) faster than 4 waves), 4 for q8_0 (the same either way).
template <int QT>
constexpr int mfma_waves() { return QT == QBL_FMT_Q8 ? 4 : 8; }

// Codes of one lane's 8 weights as exact f16 values, in the lane's input order.
//   q8_0: 8 offset-binary bytes u (= q + 128), in order.  Bits 0x64XX are the
//   f16 value 1024 + XX.  v_perm_b32 picks bytes from {w (bytes 4..7),
//   0x64646464 (bytes 0..3)}: selector 0x00050004 gives (w.b0, 0x64, w.b1,
//   0x64), 0x00070006 the upper two; then u - 128 - 1024.
__device__ __forceinline__ half8 codes_q8(uint32_t w0, uint32_t w1) {
  const uint32_t d0 = __builtin_amdgcn_perm(w0, 0x64646464u, 0x00050004u);
  const uint32_t d1 = __builtin_amdgcn_perm(w0, 0x64646464u, 0x00070006u);
  const uint32_t d2 = __builtin_amdgcn_perm(w1, 0x64646464u, 0x00050004u);
  const uint32_t d3 = __builtin_amdgcn_perm(w1, 0x64646464u, 0x00070006u);
  const half8 h = __builtin_bit_cast(half8, make_uint4(d0, d1, d2, d3));
  return h - (half8)(_Float16)1152.0f;
}
//   q4_sm / q4_K: one 32-bit word of nibbles, weights 0..7 of the lane's share
//   (byte i: weight 2i in the low nibble, 2i+1 in the high one).  Low nibbles
//   (weights 0, 2, 4, 6) and high nibbles (1, 3, 5, 7) each into the bytes of
//   one word, then two e4m3 bytes per conversion.  Input order: w0, w2, w4,
//   w6, w1, w3, w5, w7.
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ half8 codes_q4(uint32_t w) {
  constexpr float kFp8Scale = 512.0f;  // 2^9
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  const half2v c0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, kFp8Scale, false);
  const half2v c1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, kFp8Scale, true);
  const half2v c2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, kFp8Scale, false);
  const half2v c3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, kFp8Scale, true);
  return (half8){c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
}

// ---------------------------------------------------------------------------
// Prep: one launch before the GEMV, two kinds of workgroup.
//   Row workgroups [0, 8 nrw): row b = wg / nrw, blocks [256 (wg % nrw), +256)
//   of it.  Each finds the row's largest |x| itself (the whole row, from L2),
//   sets e_b, and writes the A-operand values of its blocks in instruction order:
//   frag[blk][l] for lane l = 16 g + r: row r < 8: hi of batch row r, r >= 8: lo
//   of batch row r - 8, inputs 8 g .. 8 g + 7 of the block (permuted for the q4
//   formats as codes_q4 expects); xsum[blk][r] = X of batch row r for r < 8
//   (float32, input order), 0 for r >= 8; ex[b] = e_b.  Rows b >= batch are zero.
//   Shrink workgroups (range p, adapter rows [16 q, 16 q + 16)) follow:
//   tpart[p][j][b] = sum over inputs [512 p, 512 p + 512) of A[j][k] x[b][k]
//   (lane l takes inputs 4 l + 256 c, c = 0..1, in order, then a fixed-order
//   wave sum); the GEMV adds the ranges in order.  Wave w takes rows 16 q + 4 w
//   .. + 3, their loads issued together.
// ---------------------------------------------------------------------------
constexpr int kScanK = 512;
constexpr int kScanC = kScanK / 256;  // 16-byte pieces of a range per lane
constexpr int kScanJ = 16;
constexpr int kRowBlocks = 256;  // blocks per row workgroup

struct ScanArgs {
  const float* x;
  int64_t x_stride;
  int batch, k, T, n_ent;
  int nrw;         // row workgroups per batch row
  PrepEntry ent[kMaxPrepEntries];
  float* tpart;    // [P][T][8]
  u32x4* frag;     // [nblk][64]
  float* xsum;     // [nblk][16]
  int* ex;         // [8]
};

// The prep launch's leading scalar arguments (preloaded into SGPRs at wave
// launch), repeating fields of ScanArgs.
struct PrepHot {
  const float* x;
  u32x4* frag;
  float* xsum;
  float* tpart;
  int x_stride, batch, k, nrw, T;
};

template <int QT>
__device__ __forceinline__ void prep_rows(const PrepHot& h, const ScanArgs& a, int wg) {
  __shared__ float mxw[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int b = wg / h.nrw, part = wg % h.nrw, K = h.k, nblk = K / 32;
  const bool live = b < h.batch;
  const float* xr = h.x + (int64_t)b * h.x_stride;
  float mx = 0.0f;
  if (live) {
#pragma unroll 8
    for (int i = tid; i < K / 4; i += 256) {
      const float4 v = gload4(xr + 4 * i);
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
  }
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) mxw[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(mxw[0], mxw[1]), fmaxf(mxw[2], mxw[3]));
  int e = 0;
  if (mx > 0.0f) {
    int me;
    frexpf(mx, &me);  // mx in [2^(me-1), 2^me)
    e = me - 15;
  }
  if (part == 0 && tid == 0) a.ex[b] = e;
  const int blk = part * kRowBlocks + tid;
  if (blk >= nblk) return;
  u32x4* dst = h.frag + (int64_t)blk * 64 + b;
  float s = 0.0f;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (live) {
      const float4 p = gload4(xr + 32 * blk + 8 * g), q = gload4(xr + 32 * blk + 8 * g + 4);
      v[0] = p.x, v[1] = p.y, v[2] = p.z, v[3] = p.w, v[4] = q.x, v[5] = q.y, v[6] = q.z, v[7] = q.w;
    }
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      o[i] = ldexpf(v[i], -e);
      s += o[i];
    }
    if constexpr (QT != QBL_FMT_Q8) {  // input order of codes_q4
      const float tt[8] = {o[0], o[2], o[4], o[6], o[1], o[3], o[5], o[7]};
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = tt[i];
    }
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __half h0 = __float2half_rn(o[2 * i]), h1 = __float2half_rn(o[2 * i + 1]);
      const __half l0 = __float2half_rn(o[2 * i] - __half2float(h0));
      const __half l1 = __float2half_rn(o[2 * i + 1] - __half2float(h1));
      hw[i] = (uint32_t)__half_as_ushort(h0) | ((uint32_t)__half_as_ushort(h1) << 16);
      lw[i] = (uint32_t)__half_as_ushort(l0) | ((uint32_t)__half_as_ushort(l1) << 16);
    }
    const u32x4 hv = {hw[0], hw[1], hw[2], hw[3]}, lv = {lw[0], lw[1], lw[2], lw[3]};
    dst[16 * g] = hv;
    dst[16 * g + 8] = lv;
  }
  float* xs = h.xsum + (int64_t)blk * 16;
  xs[b] = s;
  xs[b + 8] = 0.0f;
}

__device__ __forceinline__ void prep_shrink(const PrepHot& h, const ScanArgs& a, int wg) {
  __shared__ __attribute__((aligned(16))) float xs[8][kScanK];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nq = (h.T + kScanJ - 1) / kScanJ;
  const int p = wg / nq, q = wg % nq, k0 = p * kScanK, kn = min(kScanK, h.k - k0);
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // thread: rows wave and wave + 4, inputs 4 lane + 256 c
    const int b = wave + 4 * i;
#pragma unroll
    for (int c = 0; c < kScanC; ++c) {
      const int k = 4 * lane + 256 * c;
      f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
      if (b < h.batch && k < kn) v = *gp(reinterpret_cast<const f32x4*>(h.x + (int64_t)b * h.x_stride + k0 + k));
      *reinterpret_cast<f32x4*>(&xs[b][k]) = v;
    }
  }
  const int j0 = q * kScanJ + 4 * wave;
  f32x4 w[4][kScanC];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float* Ar = nullptr;
    if (j0 + u < h.T) {
      const int j = j0 + u;
      int e = 0, base = 0;
      while (base + a.ent[e].rank <= j) base += a.ent[e++].rank;
      Ar = a.ent[e].A + (int64_t)(j - base) * h.k + k0;
    }
#pragma unroll
    for (int c = 0; c < kScanC; ++c) {
      const int k = 4 * lane + 256 * c;
      w[u][c] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
      if (Ar && k < kn) w[u][c] = *gp(reinterpret_cast<const f32x4*>(Ar + k));
    }
  }
  __syncthreads();
  if (j0 >= h.T) return;
  float acc[4][8];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[u][b] = 0.0f;
#pragma unroll
  for (int c = 0; c < kScanC; ++c) {
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const f32x4 xv = *reinterpret_cast<const f32x4*>(&xs[b][4 * lane + 256 * c]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        acc[u][b] = fmaf(w[u][c].x, xv.x, fmaf(w[u][c].y, xv.y, fmaf(w[u][c].z, xv.z, fmaf(w[u][c].w, xv.w, acc[u][b]))));
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (j0 + u >= h.T) break;
    float sum[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) sum[b] = wave_sum(acc[u][b]);
    if (lane < 8) {
      float v = sum[0];
#pragma unroll
      for (int b = 1; b < 8; ++b) v = lane == b ? sum[b] : v;
      h.tpart[((int64_t)p * h.T + j0 + u) * 8 + lane] = v;
    }
  }
}

template <int QT>
__global__ __launch_bounds__(256) void prep8_kernel(const float* p_x, u32x4* p_frag, float* p_xsum, float* p_tpart,
                                                    int p_xs, int p_batch, int p_k, int p_nrw, int p_T, ScanArgs a) {
  const PrepHot h{p_x, p_frag, p_xsum, p_tpart, p_xs, p_batch, p_k, p_nrw, p_T};
  const int wg = blockIdx.x, nrow = 8 * h.nrw;
  if (wg < nrow) prep_rows<QT>(h, a, wg);
  else prep_shrink(h, a, wg - nrow);
}

// t[b][j] = the range partial sums tpart[p][j][b] added in range order; the
// loads go out 8 at a time.
__device__ __forceinline__ float t_value(const float* tpart, int P, int T, int j, int b) {
  float s = 0.0f;
  for (int p0 = 0; p0 < P; p0 += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p0 + u < P ? tpart[((int64_t)(p0 + u) * T + j) * 8 + b] : 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (p0 + u < P) s += v[u];
  }
  return s;
}

// ---------------------------------------------------------------------------
// GEMV.  A workgroup owns 64 consecutive rows of one segment (4 tiles of 16)
// and a range of the blocks of K (split-K over KS workgroups when the rows
// alone give too few workgroups).  Its W waves (mfma_waves) take the range's
// slabs in turn (wave w: slabs w, w + W, ...); a slab is the next 64 bytes of all 64 rows
// (2 q8_0 blocks or 4 q4 blocks).  A wave loads a slab with 16-byte loads that
// run along the rows (a quarter-wave covers 64 contiguous bytes of each of four
// rows), together with the slab's scales and the A operands of its blocks, one
// slab ahead of the arithmetic; it puts the slab in its own LDS region (rows 80
// bytes apart, so that the 64 lanes of an operand read hit 64 different banks)
// and feeds the instructions from there.
// The waves' partial sums meet in LDS and are added in wave order, hi part then
// lo part.  With split-K each workgroup stores its partial sums and a second
// launch adds the KS partial sums of each output in split order and finishes
// the rows (the kernel boundary orders the two; no fence inside a launch).
// Tall linears that need no split but leave some compute units one workgroup
// more than others take the even spread instead: each unit gets the same
// number of 16-row tiles (to one), in 2 to 4 tile workgroups, and the slab
// loop is compiled per tile count, so a shorter workgroup issues less.
// ---------------------------------------------------------------------------
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
constexpr int kRowStride = 80;  // LDS bytes per slab row
constexpr int kRsrcWord3 = 0x00020000;  // buffer resource flags: raw 32-bit data

template <int QT>
struct SlabFmt {
  static constexpr int S = QT == QBL_FMT_Q8 ? 2 : 4;           // blocks per slab
  static constexpr int kBpb = QT == QBL_FMT_Q8 ? 32 : 16;      // weight bytes per block
  static constexpr int kScE = QT == QBL_FMT_Q8 ? 2 : 4;        // q8_0 d, q4_sm (d | m << 16)
  static constexpr int kScLoads = QT == QBL_FMT_Q4K ? 0 : S;    // 64 S scale values / 64 lanes
  // float32 scales and minima (q4) of the slab, [block j][row], rows of
  // block j at 80 j: the stash's writes and the minimum operand's reads (lane
  // -> block l / 16, row l % 16) both fall on 64 different banks
  static constexpr int kDmStride = 80;
  static constexpr int kScOff = 64 * kRowStride;
  static constexpr int kMOff = kScOff + S * kDmStride * 4;
  static constexpr int kWave = kMOff + (QT == QBL_FMT_Q8 ? 0 : S * kDmStride * 4);  // LDS bytes per wave
};

// What a wave loads for one slab.
template <int QT>
struct SlabRegs {
  using F = SlabFmt<QT>;
  u32x4 w[4];
  uint32_t sc[F::kScLoads > 0 ? F::kScLoads : 1];
  u32x4 hd;                // q4_K: the row's super-block header (lane = row)
  u32x4 xf[F::S];
  float xa = 0.0f;         // q4: X of block l / 16 of the slab, batch row l % 16 (the minimum operand)
};

struct MfmaSplit {
  int ks;                  // workgroups per 64 rows, splitting the blocks
  int per;                 // blocks per split (a multiple of the slab)
  float* partial;          // ks > 1: [seg][ks][8][n] partial sums
  int64_t poff[kMaxSegs];  // segment offsets into partial (floats)
  // bal_k > 0 (one segment, no split): the rows' 16-row tiles spread evenly over
  // bal_c compute units, bal_k workgroups per unit (see tiles_of)
  int bal_k, bal_c, bal_t;
  const float* tpart;      // the prep launch's shrink partial sums [P][T][8]
  int P, T;
};
constexpr int kMaxT = 512;   // summed rank of a linear's list (the attach limit)

// Rows of workgroup wg under the even spread: the dispatcher fills compute
// units breadth first, so workgroups wg, wg + c, wg + 2c, ... share unit wg % c.
// Unit u owns a contiguous run of t / c (+1 for the first t % c units) tiles,
// split over its k workgroups the same way.  First tile and tile count.
__device__ __forceinline__ void tiles_of(int bal_k, int c, int bal_t, int wg, int& first, int& nt) {
  const int u = wg % c, s = wg / c;
  const int tu = bal_t / c + (u < bal_t % c ? 1 : 0);
  const int u0 = u * (bal_t / c) + min(u, bal_t % c);
  nt = tu / bal_k + (s < tu % bal_k ? 1 : 0);
  first = u0 + s * (tu / bal_k) + min(s, tu % bal_k);
}

// Output (b, n) of segment g from its base sum s (before the 2^e_b scale):
// scale, then the adapters in list order, then the store.
__device__ __forceinline__ void finish_output(const GemvArgs& a, const GemvSeg& g, const int* ex, int b, int n,
                                              float s, const float* tl, int T) {  // t[b][j] at tl[b T + j]
  float v = ldexpf(s, ex[b]);
  for (int i = 0; i < g.lora.n_ad; ++i) {
    const int rk = g.lora.rank[i];
    float p = 0.0f;
    if (rk == 0) {  // sparse delta: row n's entries against x[b]
      const float* xb = a.x + (int64_t)b * a.x_stride;
      const uint32_t e1 = g.lora.rp[i][n + 1];
      for (uint32_t e = g.lora.rp[i][n]; e < e1; ++e) p = fmaf(h2f(g.lora.sv[i][e]), xb[g.lora.ci[i][e]], p);
    } else {
      const float* Br = g.lora.B[i] + (int64_t)n * rk;
      const float* tb = tl + b * T + g.lora.toff[i];
#pragma unroll 8
      for (int q = 0; q < rk; ++q) p = fmaf(Br[q], tb[q], p);
    }
    v = fmaf(g.lora.scale[i], p, v);
  }
  g.y[(int64_t)b * g.y_stride + n] = v;
}

// Leading scalar arguments (preloaded into SGPRs at wave launch, so the first
// slab loads wait for no argument fetch): segment 0's weights and scales, the
// staged inputs and block sums, K, segment 0's height, blocks per split, the
// even spread's tile count and a packed word (ks | nseg << 5 | bal_k << 7 |
// bal_c << 10); they repeat fields of a and sp.
__host__ __device__ constexpr int mfma_pack(int ks, int nseg, int bal_k, int bal_c) {
  return ks | nseg << 5 | bal_k << 7 | bal_c << 10;
}

template <int QT>
__global__ __launch_bounds__(64 * mfma_waves<QT>(), 4) void gemv_mfma_kernel(
    const uint8_t* p_qs, const void* p_sc, const u32x4* frag, const float* xsum, int p_k, int p_n, int p_per,
    int p_balt, int p_pack, GemvArgs a, MfmaSplit sp, const int* ex) {
  using F = SlabFmt<QT>;
  constexpr int S = F::S;
  constexpr int kWaves = mfma_waves<QT>(), kMfmaThreads = 64 * kWaves;
  // the slab regions (reused after the slab loop for the waves' sums, 4 KiB per
  // wave), then the shrink results t[b][j] (without split-K)
  constexpr int kSlabLds = kWaves * F::kWave > kWaves * 4096 ? kWaves * F::kWave : kWaves * 4096;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kSlabLds + 8 * kMaxT * 4];
  float* tl = reinterpret_cast<float*>(lds + kSlabLds);
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int wg = blockIdx.x;
  const int ksn = p_pack & 31, nseg = (p_pack >> 5) & 3, bal_k = (p_pack >> 7) & 7, bal_c = p_pack >> 10;
  int si = 0, wgb = 0, n_rows = p_n;
  const uint8_t* qs = p_qs;
  const void* scp = p_sc;
  if (nseg > 1) {  // several segments: which one holds wg, and its arrays (read from a)
    asm volatile("");
    si = (nseg > 2 && wg >= a.seg[2].wg_begin) ? 2 : wg >= a.seg[1].wg_begin ? 1 : 0;
    wgb = a.seg[si].wg_begin;
    qs = a.seg[si].qs;
    scp = a.seg[si].sc;
    n_rows = a.seg[si].n;
  }
  const GemvSeg& g = a.seg[si];
  const int local = wg - wgb;
  const int rg = local / ksn, ks = local % ksn;
  // 64 rows (4 tiles of 16) per workgroup, or fewer under the even spread
  int row0 = rg * 64, nt = 4;
  if (bal_k > 0) {
    int first;
    tiles_of(bal_k, bal_c, p_balt, wg, first, nt);
    row0 = 16 * first;
  }
  // loads of rows past the workgroup's tiles go past the buffer end: they
  // return zero without a memory access (buffers and slab offsets stay below
  // 2^31 bytes, so the sum stays below 2^32)
  constexpr uint32_t kPastEnd = 0x80000000u;
  const int K = p_k, nblk = K / 32;
  const int kb0 = min(nblk, ks * p_per), kb1 = min(nblk, kb0 + p_per);
  const int nsl = (kb1 - kb0 + S - 1) / S;
  const int64_t rbytes = Fmt<QT>::row_bytes(K);

  unsigned char* W = lds + wave * F::kWave;
  float* DL = reinterpret_cast<float*>(W + F::kScOff);
  float* ML = reinterpret_cast<float*>(W + F::kMOff);

  // Slab loads are buffer loads: a per-lane byte offset fixed for the whole
  // loop plus the slab's offset (wave-uniform).  Reads past the end of a
  // buffer return zero; rows past n and blocks past the range land there or in
  // the next row, and neither is used.
  const uint32_t n32 = (uint32_t)n_rows, nb32 = (uint32_t)nblk;
  const __amdgpu_buffer_rsrc_t qs_r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(qs), 0,
                                                                         (int)(n32 * (uint32_t)rbytes), kRsrcWord3);
  uint32_t sc_bytes;
  if constexpr (QT == QBL_FMT_Q4K) sc_bytes = n32 * (uint32_t)(K / 256) * 16u;
  else sc_bytes = n32 * nb32 * (uint32_t)F::kScE;
  const __amdgpu_buffer_rsrc_t sc_r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(scp), 0, (int)sc_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t fr_r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4*>(frag), 0, (int)(nb32 * 1024u), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t xs_r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(xsum), 0, (int)(nb32 * 64u), kRsrcWord3);
  uint32_t w_off[4], s_off[F::kScLoads > 0 ? F::kScLoads : 1];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w_off[i] = i < nt ? (uint32_t)(row0 + 16 * i + (lane >> 2)) * (uint32_t)rbytes + 16u * (lane & 3) : kPastEnd;
#pragma unroll
  for (int i = 0; i < F::kScLoads; ++i) {
    const int e = 64 * i + lane, rl = e / S, j = e % S;
    s_off[i] = rl < 16 * nt ? ((uint32_t)(row0 + rl) * nb32 + (uint32_t)j) * (uint32_t)F::kScE : kPastEnd;
  }
  const uint32_t h_off = lane < 16 * nt ? (uint32_t)(row0 + lane) * (uint32_t)(K / 256) * 16u : kPastEnd;

  // NT: the tiles the slab loop covers (a compile-time count, so that a
  // workgroup with fewer tiles also issues fewer instructions)
  auto issue = [&](SlabRegs<QT>& r, int sl, auto ntc) {
    constexpr int NT = decltype(ntc)::value;
    const int b0 = kb0 + S * sl;  // wave-uniform
#pragma unroll
    for (int i = 0; i < NT; ++i)
      r.w[i] = __builtin_amdgcn_raw_buffer_load_b128(qs_r, w_off[i], b0 * F::kBpb, 0);
    if constexpr (QT == QBL_FMT_Q4K) {
      r.hd = __builtin_amdgcn_raw_buffer_load_b128(sc_r, h_off, (b0 / 8) * 16, 0);
    } else {
#pragma unroll
      for (int i = 0; i < F::kScLoads; ++i) {
        if constexpr (QT == QBL_FMT_Q8)
          r.sc[i] = __builtin_amdgcn_raw_buffer_load_b16(sc_r, s_off[i], b0 * 2, 0);
        else
          r.sc[i] = __builtin_amdgcn_raw_buffer_load_b32(sc_r, s_off[i], b0 * 4, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < S; ++j) r.xf[j] = __builtin_amdgcn_raw_buffer_load_b128(fr_r, 16u * lane, (b0 + j) * 1024, 0);
    if constexpr (QT != QBL_FMT_Q8)
      r.xa = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(xs_r, 4u * lane, b0 * 64, 0));
  };
  // the loaded slab into this wave's LDS region; scales and minima as float32
  auto stash = [&](const SlabRegs<QT>& r, int sl, auto ntc) {
    constexpr int NT = decltype(ntc)::value;
#pragma unroll
    for (int i = 0; i < NT; ++i)
      *reinterpret_cast<u32x4*>(W + (16 * i + (lane >> 2)) * kRowStride + 16 * (lane & 3)) = r.w[i];
    if constexpr (QT == QBL_FMT_Q4K) {  // lane = row: step and offset of the slab's sub-blocks
      const uint4 h = make_uint4(r.hd.x, r.hd.y, r.hd.z, r.hd.w);
#pragma unroll
      for (int j = 0; j < S; ++j) {
        float D, M;
        q4k_step_offset(h, (kb0 + S * sl + j) & 7, D, M);
        DL[j * F::kDmStride + lane] = D;
        ML[j * F::kDmStride + lane] = -M;
      }
    } else {
#pragma unroll
      for (int i = 0; i < F::kScLoads; ++i) {
        const int e = 64 * i + lane, rl = e / S, j = e % S;
        DL[j * F::kDmStride + rl] = h2f(r.sc[i]);
        if constexpr (QT != QBL_FMT_Q8) ML[j * F::kDmStride + rl] = h2f(r.sc[i] >> 16);
      }
    }
  };

  f32x4v acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = (f32x4v){0.0f, 0.0f, 0.0f, 0.0f};
  const f32x4v zero = {0.0f, 0.0f, 0.0f, 0.0f};

  auto slabs = [&](auto ntc) {
    constexpr int NT = decltype(ntc)::value;
    SlabRegs<QT> r;
    if (wave < nsl) issue(r, wave, ntc);
    // the shrink results, behind the first slab loads: into LDS for this
    // workgroup's rows, or (split-K) one value per thread of the first
    // workgroups into a.t for the reduce launch
    if (ksn == 1) {
      for (int i = tid; i < 8 * sp.T; i += kMfmaThreads) {
        const int j = i >> 3, b = i & 7;
        if (b < a.batch) tl[b * sp.T + j] = t_value(sp.tpart, sp.P, sp.T, j, b);
      }
    } else {
      for (int i = wg * kMfmaThreads + tid; i < 8 * sp.T; i += a.grid * kMfmaThreads) {
        const int j = i >> 3, b = i & 7;
        if (b < a.batch) const_cast<float*>(a.t)[(int64_t)b * sp.T + j] = t_value(sp.tpart, sp.P, sp.T, j, b);
      }
    }
    for (int sl = wave; sl < nsl; sl += kWaves) {
      stash(r, sl, ntc);
      u32x4 xf[S];
#pragma unroll
      for (int j = 0; j < S; ++j) xf[j] = r.xf[j];
      const float xa = r.xa;
      if (sl + kWaves < nsl) issue(r, sl + kWaves, ntc);
      const int nb = min(S, kb1 - (kb0 + S * sl));
#pragma unroll
      for (int j = 0; j < S; ++j) {
        if (j >= nb) break;
        const half8 xv = __builtin_bit_cast(half8, xf[j]);
        f32x4v o[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const unsigned char* wr = W + (16 * t + col) * kRowStride;
          half8 wv;
          if constexpr (QT == QBL_FMT_Q8) {
            const u32x2 w = *reinterpret_cast<const u32x2*>(wr + 32 * j + 8 * grp);
            wv = codes_q8(w.x, w.y);
          } else {
            wv = codes_q4(*reinterpret_cast<const uint32_t*>(wr + 16 * j + 4 * grp));
          }
          o[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv, wv, zero, 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const float d = DL[j * F::kDmStride + 16 * t + col];
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[t][q] = fmaf(d, o[t][q], acc[t][q]);
        }
      }
      // the slab's minimum terms (q4): block grp of the slab (none past nb), row col
      if constexpr (QT != QBL_FMT_Q8)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float m = grp < nb ? ML[(grp & (S - 1)) * F::kDmStride + 16 * t + col] : 0.0f;
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa, m, acc[t], 0, 0, 0);
      }
    }
  };
  // nt is 4 without the even spread, 2 to 4 with it (rows past nt read as zero)
  if (nt >= 4) slabs(std::integral_constant<int, 4>{});
  else if (nt == 3) slabs(std::integral_constant<int, 3>{});
  else slabs(std::integral_constant<int, 2>{});

  // the waves' sums (the slab regions are reused: wait until every wave is done with them)
  __syncthreads();
  f32x4v* part = reinterpret_cast<f32x4v*>(lds);  // [wave][tile][lane]
#pragma unroll
  for (int t = 0; t < 4; ++t) part[(wave * 4 + t) * 64 + lane] = acc[t];
  __syncthreads();

  // Rows of the workgroup: thread -> (batch row b, row rr), consecutive threads
  // on consecutive rows.  Hi of row b sits in lane 16 (b / 4) + col, element
  // b % 4; lo in lane 16 (2 + b / 4) + col.
  auto wg_sum = [&](int b, int rr) {
    const int t = rr >> 4, c = rr & 15, j = b & 3;
    const int lh = 16 * (b >> 2) + c, ll = lh + 32;
    float hi = part[t * 64 + lh][j], lo = part[t * 64 + ll][j];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      hi += part[(w * 4 + t) * 64 + lh][j];
      lo += part[(w * 4 + t) * 64 + ll][j];
    }
    return hi + lo;
  };
  if (ksn == 1) {  // thread -> (row rr, batch row b), b fastest: 8 lanes share a row of each B_i
    for (int idx = tid; idx < 64 * 8; idx += kMfmaThreads) {
      const int b = idx & 7, rr = idx >> 3, n = row0 + rr;
      if (b < a.batch && rr < 16 * nt && n < g.n) finish_output(a, g, ex, b, n, wg_sum(b, rr), tl, sp.T);
    }
    return;
  }
  float* pbase = sp.partial + sp.poff[si];
  for (int idx = tid; idx < 64 * 8; idx += kMfmaThreads) {
    const int b = idx >> 6, rr = idx & 63, n = row0 + rr;
    if (b < a.batch && n < g.n) pbase[((int64_t)ks * 8 + b) * g.n + n] = wg_sum(b, rr);
  }
}

// Split-K: output (b, n) = the ks partial sums in split order, finished.  One
// thread per output, batch row fastest (8 lanes share a row of each B_i);
// 32 rows per workgroup over the rows of all segments.
__global__ __launch_bounds__(256) void split_reduce_kernel(GemvArgs a, MfmaSplit sp, const int* ex) {
  const int b = threadIdx.x & 7;
  int n = blockIdx.x * 32 + (threadIdx.x >> 3);
  int si = 0;
  while (si + 1 < a.nseg && n >= a.seg[si].n) n -= a.seg[si++].n;
  const GemvSeg& g = a.seg[si];
  if (n >= g.n || b >= a.batch) return;
  const float* p = sp.partial + sp.poff[si] + (int64_t)b * g.n + n;
  float s = 0.0f;
  for (int q = 0; q < sp.ks; ++q) s += p[(int64_t)q * 8 * g.n];
  finish_output(a, g, ex, b, n, s, a.t, sp.T);
}

// Workgroups per 64 rows: none split when the rows alone give 1.5 workgroups
// per compute unit (256 of them), else about as many workgroups as the chip
// holds at once (4 per compute unit), each keeping at least 8 slabs.
int cu_count() {
  static std::atomic<int> cached{0};
  int n = cached.load(std::memory_order_relaxed);
  if (!n) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 1;
    cached.store(n, std::memory_order_relaxed);
  }
  return n;
}

int split_ks(int64_t row_groups, int nblk, int slab, int waves) {
  if (row_groups >= 384) return 1;
  const int64_t want = 4096 / waves / row_groups;
  const int64_t most = std::max<int64_t>(1, (nblk + slab - 1) / slab / 8);
  return (int)std::max<int64_t>(1, std::min<int64_t>({want, most, 16}));
}

template <int QT>
hipError_t launch_qt(GemvArgs& a, const PrepEntry* ent, int n_ent, int T, void* stage, int ks_force,
                     const LaunchCtx& prep_lc, const LaunchCtx& lc) {
  const int nblk = a.k / 32, P = (a.k + kScanK - 1) / kScanK;
  char* st = static_cast<char*>(stage);
  u32x4* frag = reinterpret_cast<u32x4*>(st);
  float* xsum = reinterpret_cast<float*>(st + (int64_t)nblk * 1024);
  int* ex = reinterpret_cast<int*>(xsum + (int64_t)nblk * 16);
  float* tpart = reinterpret_cast<float*>(st + mfma_stage_only_bytes(a.k));
  ScanArgs sa{};
  sa.x = a.x;
  sa.x_stride = a.x_stride;
  sa.batch = a.batch;
  sa.k = a.k;
  sa.T = T;
  sa.n_ent = n_ent;
  sa.nrw = (nblk + kRowBlocks - 1) / kRowBlocks;
  for (int i = 0; i < n_ent; ++i) sa.ent[i] = ent[i];
  sa.tpart = tpart;
  sa.frag = frag;
  sa.xsum = xsum;
  sa.ex = ex;
  const int shrink_wgs = T > 0 ? P * ((T + kScanJ - 1) / kScanJ) : 0;
  QBL_LAUNCH(prep8_kernel<QT>, dim3(8 * sa.nrw + shrink_wgs), dim3(256), 0, prep_lc, sa.x, sa.frag, sa.xsum, sa.tpart,
             (int)sa.x_stride, sa.batch, sa.k, sa.nrw, sa.T, sa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int S = SlabFmt<QT>::S;
  int64_t row_groups = 0;
  for (int i = 0; i < a.nseg; ++i) row_groups += (a.seg[i].n + 63) / 64;
  MfmaSplit sp{};
  sp.tpart = tpart;
  sp.P = P;
  sp.T = T;
  sp.ks = ks_force > 0 ? ks_force : split_ks(row_groups, nblk, S, mfma_waves<QT>());
  const int nslab = (nblk + S - 1) / S;
  sp.per = (nslab + sp.ks - 1) / sp.ks * S;
  sp.partial = reinterpret_cast<float*>(st + mfma_stage_only_bytes(a.k) + mfma_scan_bytes(a.k, T));
  int wg = 0;
  int64_t po = 0, rows = 0;
  for (int i = 0; i < a.nseg; ++i) {
    a.seg[i].wg_begin = wg;
    wg += (a.seg[i].n + 63) / 64 * sp.ks;
    sp.poff[i] = po;
    po += (int64_t)sp.ks * 8 * a.seg[i].n;
    rows += a.seg[i].n;
  }
  if (sp.ks > 1 && po * 4 > mfma_partial_bytes(row_groups * 64)) return hipErrorInvalidValue;
  // Even spread: with 64-row workgroups some compute units hold one more
  // workgroup than others (the 70B gate/up: 448 workgroups on 256 units, 192 of
  // them holding two and finishing ~1.7x later).  One segment without split: k
  // workgroups per unit share the unit's ceil(tiles / units) tiles, taken
  // where that lowers the most tiles any unit holds.
  if (sp.ks == 1 && a.nseg == 1) {
    const int c = cu_count(), t = (a.seg[0].n + 15) / 16;
    const int most_even = (t + c - 1) / c, k = (most_even + 3) / 4;
    const int most_now = 4 * ((wg + c - 1) / c);
    if (k >= 2 && k <= 7 && most_even < most_now) {  // k fits the packed argument's 3 bits
      sp.bal_k = k;
      sp.bal_c = c;
      sp.bal_t = t;
      wg = k * c;
    }
  }
  a.grid = wg;
  const int pack = mfma_pack(sp.ks, a.nseg, sp.bal_k, sp.bal_c);
  if (sp.ks == 1) {
    QBL_LAUNCH(gemv_mfma_kernel<QT>, dim3(wg), dim3(64 * mfma_waves<QT>()), 0, lc, a.seg[0].qs, a.seg[0].sc, frag,
               xsum, a.k, a.seg[0].n, sp.per, sp.bal_t, pack, a, sp, ex);
    return hipGetLastError();
  }
  // the timing events of lc go around both launches
  LaunchCtx first = lc, second = lc;
  first.stop = nullptr;
  second.start = nullptr;
  QBL_LAUNCH(gemv_mfma_kernel<QT>, dim3(wg), dim3(64 * mfma_waves<QT>()), 0, first, a.seg[0].qs, a.seg[0].sc, frag,
             xsum, a.k, a.seg[0].n, sp.per, sp.bal_t, pack, a, sp, ex);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  QBL_LAUNCH(split_reduce_kernel, dim3((unsigned)((rows + 31) / 32)), dim3(256), 0, second, a, sp, ex);
  return hipGetLastError();
}

}  // namespace

// Staging layout: A operands [nblk][64] x 16 bytes, block sums [nblk][16]
// floats, 8 exponents; the prep launch's partial shrink sums [P][T][8]; then
// the split-K partial sums.
int64_t mfma_stage_only_bytes(int k) {
  const int64_t nblk = k / 32;
  return (nblk * (1024 + 64) + 32 + 255) / 256 * 256;
}
int64_t mfma_scan_bytes(int k, int T) {
  const int64_t P = (k + kScanK - 1) / kScanK;
  return (P * 8 * 4 * (int64_t)T + 255) / 256 * 256;
}
int64_t mfma_partial_bytes(int64_t rows) { return rows * 8 * 16 * 4; }  // up to 16 splits
int64_t mfma_stage_bytes(int64_t rows, int k, int T) {
  return mfma_stage_only_bytes(k) + mfma_scan_bytes(k, T) +
         (mfma_partial_bytes((rows + 63) / 64 * 64) + 255) / 256 * 256;
}

hipError_t launch_gemv_mfma(GemvArgs& a, const PrepEntry* ent, int n_ent, int T, void* stage, int ks,
                            const LaunchCtx& prep_lc, const LaunchCtx& lc) {
  (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
  if (a.batch < 2 || a.batch > 8 || a.nseg < 1 || a.nseg > kMaxSegs || !stage) return hipErrorInvalidValue;
  if (a.k < 32 || a.k % (a.qtype == QBL_FMT_Q4K ? 256 : 32) || a.x_stride % 4 || a.x_stride >= ((int64_t)1 << 31))
    return hipErrorInvalidValue;
  if (reinterpret_cast<uintptr_t>(stage) % 256 || reinterpret_cast<uintptr_t>(a.x) % 16) return hipErrorInvalidValue;
  if (ks < 0 || ks > 16 || n_ent < 0 || n_ent > kMaxPrepEntries || T < 0 || T > kMaxT) return hipErrorInvalidValue;
  int rk = 0;
  for (int i = 0; i < n_ent; ++i) {
    if (ent[i].toff != rk || ent[i].rank <= 0) return hipErrorInvalidValue;
    rk += ent[i].rank;
  }
  // the GEMV's buffer loads address a segment's weights and scales with 32-bit
  // byte offsets: each must stay below 2^31 bytes
  const int64_t rbytes = a.qtype == QBL_FMT_Q8 ? a.k : a.k / 2;
  const int64_t sbytes = a.qtype == QBL_FMT_Q8 ? a.k / 16 : a.qtype == QBL_FMT_Q4 ? a.k / 8 : a.k / 16;
  for (int i = 0; i < a.nseg; ++i)
    if ((int64_t)(a.seg[i].n + 63) / 64 * 64 * rbytes >= (int64_t)1 << 31 ||
        (int64_t)(a.seg[i].n + 63) / 64 * 64 * sbytes >= (int64_t)1 << 31)
      return hipErrorInvalidValue;
  if (rk != T || (T > 0 && !a.t)) return hipErrorInvalidValue;
  switch (a.qtype) {
    case QBL_FMT_Q8: return launch_qt<QBL_FMT_Q8>(a, ent, n_ent, T, stage, ks, prep_lc, lc);
    case QBL_FMT_Q4: return launch_qt<QBL_FMT_Q4>(a, ent, n_ent, T, stage, ks, prep_lc, lc);
    case QBL_FMT_Q4K: return launch_qt<QBL_FMT_Q4K>(a, ent, n_ent, T, stage, ks, prep_lc, lc);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qbl
