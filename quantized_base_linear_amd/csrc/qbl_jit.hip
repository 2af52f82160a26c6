// Prefill path for gfx950: per-layer just-in-time materialisation feeding
// bf16 matrix cores.
//
// "Deep Technical Design: Exact, Atomic, Reversible Specialist Overlays",
// section 8: with many tokens the layer is a GEMM, and materialising the layer
// is amortised over the tokens; section 1 and section 5: the merged layer lives
// only in scratch, is used for this layer's forward pass and discarded, and the
// quantized base is never rewritten.  Here the scratch is on chip: each
// workgroup builds one 128 x 64 tile of
//
//   W_eff = bf16( f32(dequant(W_q)) + sum_i bf16(s_i B_i) bf16(A_i) )
//
// in LDS per K-step (the low-rank sum itself on MFMA), and multiplies the
// staged bf16 X tile against it with v_mfma_f32_32x32x16_bf16, accumulating
// in float32.  No W_eff element ever reaches HBM.
//
// MFMA 32x32x16 lane layout (wave64): operand A row i = lane % 32 holds
// k = 8*(lane/32) .. +7; operand B column j = lane % 32 holds the same k range;
// result element v of a lane is row 8*(v/4) + 4*(lane/32) + v%4, column lane % 32.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <algorithm>

#include "qbl_device.h"
#include "qbl_kernels.h"

namespace qbl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int JBM = 256;          // output rows (tokens) per workgroup
constexpr int JBN = 128;          // output columns per workgroup
constexpr int JBK = 64;           // K per step
constexpr int JLD = JBK + 8;      // LDS row pitch in bf16 (16 B pad: conflict-free 16 B reads)
constexpr int JTHREADS = 512;     // 8 waves: 4 along M x 2 along N, 64 x 64 outputs each
constexpr int JRMAX = 4;          // rank steps of 16 kept in registers (total rank <= 64)

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// ---------------------------------------------------------------------------
// Stage the adapter factors once per call in the workspace, as bf16 with the
// scale folded into B:  At[k][t] = bf16(A_cat[t][k]),  sB[n][t] = bf16(f32(s_i B_i[n][j]))
// where t runs over the concatenated ranks (zero beyond the total rank).
// ---------------------------------------------------------------------------
// At goes through an LDS tile of 64 ranks x 16 inputs per workgroup: each thread
// reads 4 consecutive inputs of one rank row of A (16 bytes) and writes 4
// consecutive ranks of one row of At.  The adapter loop runs over j uniformly, so
// the factor pointers are scalar loads.
constexpr int kStageT = 64, kStageK = 16;
__device__ __forceinline__ void stage_at_tile(const JitArgs& a, int tp, int kx, int ty) {
  __shared__ float tile[kStageT][kStageK + 1];
  const int k0 = kx * kStageK, t0 = ty * kStageT;
  {
    const int tt = threadIdx.x >> 2, kq = 4 * (threadIdx.x & 3), t = t0 + tt;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    int base = 0;
    for (int j = 0; j < a.n_ad; ++j) {
      if (t >= base && t < base + a.rank[j] && k0 + kq < a.k)
        v = *reinterpret_cast<const float4*>(a.A[j] + (int64_t)(t - base) * a.k + k0 + kq);
      base += a.rank[j];
    }
    tile[tt][kq] = v.x;
    tile[tt][kq + 1] = v.y;
    tile[tt][kq + 2] = v.z;
    tile[tt][kq + 3] = v.w;
  }
  __syncthreads();
  uint16_t* At = a.ws;
  const int kk = threadIdx.x >> 4, tq = 4 * (threadIdx.x & 15), k = k0 + kk;
  if (k < a.k && t0 + tq < tp) {
    const uint32_t lo = bf16_rne(tile[tq][kk]) | ((uint32_t)bf16_rne(tile[tq + 1][kk]) << 16);
    const uint32_t hi = bf16_rne(tile[tq + 2][kk]) | ((uint32_t)bf16_rne(tile[tq + 3][kk]) << 16);
    *reinterpret_cast<uint2*>(At + (int64_t)k * tp + t0 + tq) = make_uint2(lo, hi);
  }
}

// sB[n][t] = bf16(f32(s_j B_j[n][t - base_j])), element o = n * tp + t per
// thread (32-bit index arithmetic; the adapter loop over j is uniform)
__device__ __forceinline__ void stage_sb_elem(const JitArgs& a, int tp, uint32_t o) {
  if (o >= (uint32_t)a.n * (uint32_t)tp) return;
  const int n = (int)(o / (uint32_t)tp), t = (int)(o % (uint32_t)tp);
  const int64_t nat = (int64_t)a.k * tp;
  uint16_t* sB = a.ws + ((nat * 2 + 255) / 256 * 256) / 2;
  float v = 0.0f;
  int base = 0;
  for (int j = 0; j < a.n_ad; ++j) {
    if (t >= base && t < base + a.rank[j]) v = a.scale[j] * a.B[j][(int64_t)n * a.rank[j] + (t - base)];
    base += a.rank[j];
  }
  sB[o] = bf16_rne(v);
}

// Every rank a multiple of 8: elements o = 8 g .. 8 g + 7 lie in one row and in
// one adapter's part (or all in the zero padding), so a thread stages them with
// two 16-byte loads of B and one 16-byte store, each value rounded as above.
__device__ __forceinline__ void stage_sb_vec8(const JitArgs& a, int tp, uint32_t g) {
  if (g >= (uint32_t)a.n * (uint32_t)tp / 8u) return;  // (tp is a multiple of 16)
  const uint32_t o = 8u * g;
  const int n = (int)(o / (uint32_t)tp), t = (int)(o % (uint32_t)tp);
  const int64_t nat = (int64_t)a.k * tp;
  uint16_t* sB = a.ws + ((nat * 2 + 255) / 256 * 256) / 2;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int base = 0;
  for (int j = 0; j < a.n_ad; ++j) {
    if (t >= base && t < base + a.rank[j]) {
      const float4* p = reinterpret_cast<const float4*>(a.B[j] + (int64_t)n * a.rank[j] + (t - base));
      const float4 lo = p[0], hi = p[1];
      const float s = a.scale[j];
      v[0] = s * lo.x, v[1] = s * lo.y, v[2] = s * lo.z, v[3] = s * lo.w;
      v[4] = s * hi.x, v[5] = s * hi.y, v[6] = s * hi.z, v[7] = s * hi.w;
    }
    base += a.rank[j];
  }
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = bf16_rne(v[2 * i]) | ((uint32_t)bf16_rne(v[2 * i + 1]) << 16);
  *reinterpret_cast<uint4*>(sB + o) = make_uint4(w[0], w[1], w[2], w[3]);
}

// One launch for both: workgroups [0, at_wgs) stage At tiles (ceil(k/16) along
// k, then the rank tiles), the rest sB, 256 elements each (VEC8: 2048, eight
// per thread).
template <bool VEC8>
__global__ __launch_bounds__(256) void stage_lora_kernel(JitArgs a, int tp, int at_kt, int at_wgs) {
  const int b = blockIdx.x;
  if (b < at_wgs) stage_at_tile(a, tp, b % at_kt, b / at_kt);
  else if (VEC8) stage_sb_vec8(a, tp, (uint32_t)(b - at_wgs) * 256u + threadIdx.x);
  else stage_sb_elem(a, tp, (uint32_t)(b - at_wgs) * 256u + threadIdx.x);
}

// ---------------------------------------------------------------------------
// The fused JIT GEMM.  RS = rank steps of 16 (0: no adapters; 1..JRMAX: held
// in registers; JRMAX+1: more, streamed 64 ranks at a time).
//
// The X and W_eff tiles are double-buffered in LDS: during K-step k every wave
// issues its MFMAs on buffer k & 1 and, in the same stretch of code, builds its
// block of W_eff(k+1) and stages X(k+1) into the other buffer, so the matrix
// cores and the dequantisation arithmetic overlap; one barrier per K-step.
// bf16 rounding (round to nearest even) uses the hardware conversion.
// ---------------------------------------------------------------------------
constexpr int kXsElems = JBM * JLD;
constexpr int kWsElems = JBN * JLD;
constexpr int kALD = 16 * JRMAX + 8;         // LDS pitch of a staged At row (bf16)
constexpr int kAsElems = JBK * kALD;         // one K-step of At (rank <= 64)
constexpr size_t kJitLds = 2 * (size_t)(kXsElems + kWsElems + kAsElems) * sizeof(uint16_t);

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// two floats to bf16 (round to nearest even), lo in the low half: one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// FULL: every tile lies inside the matrix (M a multiple of 256, K of 64): the
// K-step body has no branches, one basic block that the scheduler interleaves.
template <int QT, int RS, bool FULL>
__global__ __launch_bounds__(JTHREADS) void jit_kernel(JitArgs a, int tp) {
  extern __shared__ __attribute__((aligned(16))) uint16_t jit_lds[];
  uint16_t* Xs0 = jit_lds;
  uint16_t* Ws0 = jit_lds + 2 * kXsElems;
  uint16_t* As0 = Ws0 + 2 * kWsElems;  // At rows of a K-step, staged once per workgroup

  // the wave index is uniform; conditions derived from it become scalar branches
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 31, h = lane >> 5;
  const int N = a.n, K = a.k, M = a.m;
  const int n0 = blockIdx.x * JBN, m0 = blockIdx.y * JBM;
  const int nblk = K / 32;
  const int nk = (K + JBK - 1) / JBK;

  // W-tile construction role: 32 k x 32 n block (kb, nb) of the 64 x 128 tile
  const int kb = w & 1, nb = w >> 1;
  const int nrow = min(n0 + 32 * nb + col, N - 1);
  // main GEMM role: 64 x 64 outputs at (wm, wn)
  const int wm = w & 3, wn = w >> 2;

  const int64_t nat = (int64_t)K * tp;
  const uint16_t* At = a.ws;
  const uint16_t* sB = a.ws + ((nat * 2 + 255) / 256 * 256) / 2;
  constexpr int RREG = RS <= JRMAX ? RS : JRMAX;

  bf16x8 sbf[RREG > 0 ? RREG : 1];
  if constexpr (RS > 0 && RS <= JRMAX) {
#pragma unroll
    for (int r = 0; r < RS; ++r) sbf[r] = ld_bf16x8(sB + (int64_t)nrow * tp + 16 * r + 8 * h);
  }

  // Operands of K-step s in registers (Ops(s)): the X tile and the quantised
  // weights of step s, and the At rows of step s + 1.  Two sets: at K-step ks
  // the set holding Ops(ks + 1) is consumed and reloaded with Ops(ks + 3) while
  // Ops(ks + 2), issued one step earlier, is still in flight.  Every load is
  // unconditional (clamped in-bounds addresses; what lies outside the matrix is
  // zeroed or skipped where it is used), so the compiler's in-order wait counts
  // keep the later set in flight.
  struct Ops {
    uint32_t scv;
    uint4 hd;  // q4_K: the super-block header of the lane's block
    uint4 qv;  // 16 consecutive weights of this lane's row: 16 bytes (q8_0) or 8 (q4_sm, q4_K)
    uint4 xr[4];
    uint4 atr;
  };
  Ops opa, opb;
  // At of a K-step: 64 rows of tp bf16, one 16-byte piece per thread
  constexpr bool kAtRegs = RS > 0 && RS <= JRMAX;
  const int arow = tid / (tp > 0 ? tp / 8 : 1), apiece = tid % (tp > 0 ? tp / 8 : 1);
  const bool aload = kAtRegs && tid < 8 * tp;
  auto load_at = [&](uint4& r, int k0) {
    if constexpr (kAtRegs) {
      const int k = aload ? min(k0 + arow, K - 1) : 0;
      r = *reinterpret_cast<const uint4*>(At + (int64_t)k * tp + (aload ? 8 * apiece : 0));
    }
  };
  // At row k_local = 16 h' + v of a 32-row half goes to LDS row 8 (v / 4) + 4 h' + v % 4:
  // the LoRA MFMA's output row r then holds k_local = perm(r), and lane (col, h)
  // holds k_local = 16 h + v in dsum[v], 16 contiguous k, the same k its single
  // 16-byte load of quantised weights covers.
  auto store_at = [&](const uint4& r, int b) {
    const int half = arow >> 5, kl = arow & 31, hh = kl >> 4, v = kl & 15;
    const int lrow = 32 * half + 8 * (v >> 2) + 4 * hh + (v & 3);
    if (aload) *reinterpret_cast<uint4*>(As0 + b * kAsElems + lrow * kALD + 8 * apiece) = r;
  };

  // K offset of K-step st (steps past the end build tiles nobody reads)
  auto koff = [&](int st) { return st * JBK; };

  auto prefetch = [&](Ops& o, int st) {
    const int k0 = koff(st);
    const int kbase = min(k0 + 32 * kb, K - 32);
    if (QT == QBL_FMT_Q8) {
      o.scv = reinterpret_cast<const uint16_t*>(a.sc)[(int64_t)nrow * nblk + kbase / 32];
      o.qv = *reinterpret_cast<const uint4*>(a.qs + (int64_t)nrow * K + kbase + 16 * h);
    } else {
      if constexpr (QT == QBL_FMT_Q4K)
        o.hd = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.sc) +
                                               ((int64_t)nrow * (K / 256) + kbase / 256) * 16);
      else
        o.scv = reinterpret_cast<const uint32_t*>(a.sc)[(int64_t)nrow * nblk + kbase / 32];
      const uint2 q2 = *reinterpret_cast<const uint2*>(a.qs + (int64_t)nrow * (K / 2) + (kbase + 16 * h) / 2);
      o.qv = make_uint4(q2.x, q2.y, 0u, 0u);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int idx = tid + JTHREADS * c;
      const int row = idx >> 3, c16 = idx & 7;
      const int m = min(m0 + row, M - 1), kk = min(k0 + 8 * c16, K - 8);
      o.xr[c] = *reinterpret_cast<const uint4*>(a.X + (int64_t)m * K + kk);
    }
    load_at(o.atr, koff(st + 1));
  };

  // The low-rank sum of this wave's 32 x 32 block of W_eff at K-step k0, from
  // the At rows staged in As[b]: lane (col, h) gets k = 16 h + v in dsum[v].
  auto lora = [&](int k0, int b) {
    f32x16 dsum;
#pragma unroll
    for (int v = 0; v < 16; ++v) dsum[v] = 0.0f;
    if constexpr (kAtRegs) {
      const uint16_t* arow_p = As0 + b * kAsElems + (32 * kb + col) * kALD + 8 * h;
#pragma unroll
      for (int r = 0; r < RS; ++r)
        dsum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_bf16x8(arow_p + 16 * r), sbf[r], dsum, 0, 0, 0);
    } else if constexpr (RS > JRMAX) {
      const int kbase = min(k0 + 32 * kb, K - 32);
      const int prow = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);  // the same row permutation
      for (int r = 0; r < tp / 16; ++r) {
        const bf16x8 af = ld_bf16x8(At + (int64_t)(kbase + prow) * tp + 16 * r + 8 * h);
        const bf16x8 bf = ld_bf16x8(sB + (int64_t)nrow * tp + 16 * r + 8 * h);
        dsum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, dsum, 0, 0, 0);
      }
    }
    return dsum;
  };

  // this wave's 32 x 32 block of W_eff for K-step at k0 (low-rank sum dsum), and
  // the X tile, into buffer b
  auto build = [&](const Ops& o, int k0, int b, const f32x16& dsum) {
    const uint4* xr = o.xr;
    const uint32_t qw[4] = {o.qv.x, o.qv.y, o.qv.z, o.qv.w};
    const uint32_t scv = o.scv;
    uint16_t* wrow = Ws0 + b * kWsElems + (32 * nb + col) * JLD + 32 * kb + 16 * h;
    // a K block past the matrix contributes zeros (the wave's condition, uniform:
    // a scalar branch, no per-element selects)
    if (FULL || k0 + 32 * kb < K) {
      float d, mn;
      if constexpr (QT == QBL_FMT_Q4K) {  // the block is sub-block (k / 32) % 8 of its super-block
        float D, M;
        q4k_step_offset(o.hd, ((k0 + 32 * kb) / 32) & 7, D, M);
        d = D;
        mn = -M;
      } else {
        d = h2f(scv);
        mn = QT == QBL_FMT_Q8 ? -128.0f * d : h2f(scv >> 16);
      }
      // lane (col, h): weights k = 16 h + v, v = 0..15, of row col
      uint32_t packed[8];
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        float wv[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          // q8_0: d (u - 128) = fma(d, u, -128 d), u the offset-binary byte; q4_sm: fma(d, q, m);
          // q4_K: fma(D, q, -M).  Each is float32(dequant) (products of at most 21
          // significant bits, then one rounding for the q4 formats), as in the recipe.
          const int e = v + j;
          float deq;
          if (QT == QBL_FMT_Q8)
            deq = d * (float)((qw[e >> 2] >> (8 * (e & 3))) & 0xFFu) + mn;
          else
            deq = fmaf(d, (float)((qw[e >> 3] >> (4 * (e & 7))) & 0xFu), mn);
          wv[j] = RS > 0 ? deq + dsum[e] : deq;
        }
        packed[v >> 1] = pack_bf16(wv[0], wv[1]);
      }
      *reinterpret_cast<uint4*>(wrow) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
      *reinterpret_cast<uint4*>(wrow + 8) = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    } else {
      *reinterpret_cast<uint4*>(wrow) = make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(wrow + 8) = make_uint4(0u, 0u, 0u, 0u);
    }
    // the X tile: stored as loaded when it lies inside the matrix (the workgroup's
    // condition, uniform), else with the parts outside zeroed
    uint16_t* xs = Xs0 + b * kXsElems;
    if (FULL || (m0 + JBM <= M && k0 + JBK <= K)) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int idx = tid + JTHREADS * c;
        *reinterpret_cast<uint4*>(xs + (idx >> 3) * JLD + 8 * (idx & 7)) = xr[c];
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int idx = tid + JTHREADS * c;
        const int row = idx >> 3, c16 = idx & 7;
        const bool xin = m0 + row < M && k0 + 8 * c16 < K;
        *reinterpret_cast<uint4*>(xs + row * JLD + 8 * c16) = xin ? xr[c] : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // At of steps 0 and 1 into LDS first; then step 0's tiles
  {
    uint4 r0 = make_uint4(0u, 0u, 0u, 0u), r1 = r0;
    load_at(r0, koff(0));
    load_at(r1, koff(1));
    store_at(r0, 0);
    store_at(r1, 1);
  }
  __syncthreads();
  prefetch(opa, 0);
  build(opa, koff(0), 0, lora(koff(0), 0));
  // Ops(1) strictly before Ops(2): the loop's wait counts assume the older set
  // was issued first (the barrier keeps the scheduler from swapping them)
  prefetch(opa, 1);
  __builtin_amdgcn_sched_barrier(0);
  prefetch(opb, 2);
  __syncthreads();

  // One K-step: the low-rank sum of the next W tile first (its MFMAs overlap the
  // main ones), the MFMAs on buffer cur, then the next step's tiles from `next`
  // (Ops(ks + 1)) into the other buffer, At(ks + 2) into As[cur], and `next`
  // reloaded with Ops(ks + 3).
  auto step = [&](int ks, Ops& next) {
    const int cur = ks & 1;
    const f32x16 dsum = lora(koff(ks + 1), cur ^ 1);  // At(ks + 1) in As[cur ^ 1]
    // the low-rank MFMAs go out first and alone: the build that uses their sum
    // then comes after the main MFMAs, by which time the chain has finished
    if constexpr (FULL) __builtin_amdgcn_sched_barrier(0);
    const uint16_t* xs = Xs0 + cur * kXsElems;
    const uint16_t* ws = Ws0 + cur * kWsElems;
#pragma unroll
    for (int kk = 0; kk < JBK / 16; ++kk) {
      bf16x8 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = ld_bf16x8(xs + (64 * wm + 32 * i + col) * JLD + 16 * kk + 8 * h);
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = ld_bf16x8(ws + (64 * wn + 32 * j + col) * JLD + 16 * kk + 8 * h);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    // (unconditional, so the body is one block the scheduler can interleave with
    // the MFMAs; past the end they build tiles nobody reads)
    build(next, koff(ks + 1), cur ^ 1, dsum);
    store_at(next.atr, cur);  // At(ks + 2): As[cur] was last read by the low-rank sum of step ks - 1
    prefetch(next, ks + 3);
    if constexpr (FULL) {
      // one MFMA, then a few vector instructions: the dequantisation of the next
      // tile runs while the matrix core works
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
    }
    __syncthreads();
  };
  // two steps per iteration with no exit between them (an exit there would merge
  // into the loop head and shorten the compiler's wait counts); an odd last step after
  int ks = 0;
  for (; ks + 1 < nk; ks += 2) {
    step(ks, opa);
    step(ks + 1, opb);
  }
  if (ks < nk) step(ks, opa);

  // ---- write Y (float32)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + 64 * wn + 32 * j + col;
      if (n >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + 64 * wm + 32 * i + 8 * (v / 4) + 4 * h + (v % 4);
        if (m < M) a.Y[(int64_t)m * N + n] = acc[i][j][v];
      }
    }
}

// ---------------------------------------------------------------------------
// The same GEMM for full tiles with the waves split by role: 8 waves issue the
// main MFMAs (64 x 64 outputs each, as above) and stage the X tile (loads two
// steps ahead, stores: no arithmetic); 8 builder waves load the quantised
// weights and the A-factor rows two steps ahead and build each W_eff tile
// (a 32 x 32 block per wave, the low-rank sum on their own MFMAs).
// Both roles meet at the one barrier per K-step of the double-buffered layout,
// so the matrix cores of a SIMD keep working while its builder wave does the
// vector work of the next step.
// ---------------------------------------------------------------------------
constexpr int JWS_MFMA = 8, JWS_BUILD = 8, JWS_THREADS = (JWS_MFMA + JWS_BUILD) * 64;

// SG (q8_0 with K a multiple of 256): a builder's scales come 8 blocks, 16 bytes,
// at a time, once per 4 K-steps (see below).
template <int QT, int RS, bool SG>
__global__ __launch_bounds__(JWS_THREADS) void jit_ws_kernel(JitArgs a, int tp) {
  static_assert(RS <= JRMAX, "ranks held in registers");
  extern __shared__ __attribute__((aligned(16))) uint16_t jit_lds[];
  uint16_t* Xs0 = jit_lds;
  uint16_t* Ws0 = jit_lds + 2 * kXsElems;
  uint16_t* As0 = Ws0 + 2 * kWsElems;

  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 31, h = lane >> 5;
  const int N = a.n, K = a.k;
  const int n0 = blockIdx.x * JBN, m0 = blockIdx.y * JBM;
  const int nblk = K / 32;
  const int nk = K / JBK;  // K is a multiple of the K-step here

  if (w < JWS_MFMA) {
    // ---- MFMA role: 64 x 64 outputs at (wm, wn)
    const int wm = w & 3, wn = w >> 2;
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    // X tile of K-step st: 256 rows x 64 bf16, 4 16-byte pieces per lane (plain
    // arrays and macros: held in registers, two sets, as the builders' operands)
    uint4 xa0, xa1, xa2, xa3, xb0, xb1, xb2, xb3;
    // piece c of a lane: row (tid + 512 c) / 8, 16-byte column (tid + 512 c) % 8
    const uint16_t* xg = a.X + (int64_t)(m0 + (tid >> 3)) * K + 8 * (tid & 7);
    const int64_t xrow64 = (int64_t)64 * K;  // 512 pieces = 64 rows further
    const int xl = (tid >> 3) * JLD + 8 * (tid & 7);
#define QBL_XLOAD(R, ST)                                                                 \
  do {                                                                                   \
    const int k0_ = min((ST), nk - 1) * JBK; /* steps past the end reload the last one */ \
    R##0 = *reinterpret_cast<const uint4*>(xg + k0_);                                    \
    R##1 = *reinterpret_cast<const uint4*>(xg + xrow64 + k0_);                           \
    R##2 = *reinterpret_cast<const uint4*>(xg + 2 * xrow64 + k0_);                       \
    R##3 = *reinterpret_cast<const uint4*>(xg + 3 * xrow64 + k0_);                       \
  } while (0)
#define QBL_XSTORE(R, B)                                                  \
  do {                                                                    \
    uint16_t* xs_ = Xs0 + (B) * kXsElems + xl;                            \
    *reinterpret_cast<uint4*>(xs_) = R##0;                                \
    *reinterpret_cast<uint4*>(xs_ + 64 * JLD) = R##1;                     \
    *reinterpret_cast<uint4*>(xs_ + 128 * JLD) = R##2;                    \
    *reinterpret_cast<uint4*>(xs_ + 192 * JLD) = R##3;                    \
  } while (0)
// One K-step: per 16-K group, the group's four operand reads, two MFMAs, the
// store of one X(ks + 1) piece and the reload of that piece's register with
// X(ks + 3), two MFMAs (the LDS write and the load issue hide under the matrix
// core instead of queueing before the barrier).
#define QBL_XPIECE(NEXT, C, XSN, K3)                                                        \
  do {                                                                                      \
    *reinterpret_cast<uint4*>((XSN) + (C) * 64 * JLD) = NEXT##C;                            \
    NEXT##C = *reinterpret_cast<const uint4*>(xg + (C) * xrow64 + (K3));                    \
  } while (0)
#define QBL_MSTEP(KS, NEXT)                                                                              \
  do {                                                                                                   \
    const int cur = (KS) & 1;                                                                            \
    const uint16_t* xs = Xs0 + cur * kXsElems;                                                           \
    const uint16_t* ws = Ws0 + cur * kWsElems;                                                           \
    uint16_t* xsn = Xs0 + (cur ^ 1) * kXsElems + xl;                                                     \
    const int k3 = min((KS) + 3, nk - 1) * JBK; /* steps past the end reload the last one */             \
    _Pragma("unroll") for (int kk = 0; kk < JBK / 16; ++kk) {                                            \
      bf16x8 af[2], bf[2];                                                                               \
      _Pragma("unroll") for (int i = 0; i < 2; ++i) af[i] =                                             \
          ld_bf16x8(xs + (64 * wm + 32 * i + col) * JLD + 16 * kk + 8 * h);                              \
      _Pragma("unroll") for (int j = 0; j < 2; ++j) bf[j] =                                             \
          ld_bf16x8(ws + (64 * wn + 32 * j + col) * JLD + 16 * kk + 8 * h);                              \
      _Pragma("unroll") for (int i = 0; i < 2; ++i) _Pragma("unroll") for (int j = 0; j < 2; ++j)       \
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);          \
      if (kk == 0) QBL_XPIECE(NEXT, 0, xsn, k3);                                                         \
      if (kk == 1) QBL_XPIECE(NEXT, 1, xsn, k3);                                                         \
      if (kk == 2) QBL_XPIECE(NEXT, 2, xsn, k3);                                                         \
      if (kk == 3) QBL_XPIECE(NEXT, 3, xsn, k3);                                                         \
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0); /* LDS reads */                                 \
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0); /* MFMA */                                      \
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0); /* LDS write */                                 \
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); /* global load */                               \
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0); /* MFMA */                                      \
    }                                                                                                    \
    __syncthreads();                                                                                     \
  } while (0)
    __syncthreads();  // the builders' At(0), At(1)
    QBL_XLOAD(xa, 0);
    QBL_XSTORE(xa, 0);
    QBL_XLOAD(xa, 1);
    __builtin_amdgcn_sched_barrier(0);  // X(1) strictly before X(2) (the loop's wait counts)
    QBL_XLOAD(xb, 2);
    __syncthreads();  // step 0's tiles
    int ks = 0;
    for (; ks + 1 < nk; ks += 2) {
      QBL_MSTEP(ks, xa);
      QBL_MSTEP(ks + 1, xb);
    }
    if (ks < nk) QBL_MSTEP(ks, xa);
#undef QBL_MSTEP
#undef QBL_XPIECE
#undef QBL_XSTORE
#undef QBL_XLOAD
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + 64 * wn + 32 * j + col;
        if (n >= N) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + 64 * wm + 32 * i + 8 * (v / 4) + 4 * h + (v % 4);
          a.Y[(int64_t)m * N + n] = acc[i][j][v];
        }
      }
    return;
  }

  // ---- builder role: wave bw builds the 32 x 32 block (kb, nb) = (bw & 1,
  // bw >> 1) of each W tile, and with the other builders stages At
  const int bw = w - JWS_MFMA, bt = tid - JWS_MFMA * 64;  // 0..7, 0..511
  const int kb = bw & 1, nb = bw >> 1;
  const int nrow = min(n0 + 32 * nb + col, N - 1);
  const int64_t nat = (int64_t)K * tp;
  const uint16_t* At = a.ws;
  const uint16_t* sB = a.ws + ((nat * 2 + 255) / 256 * 256) / 2;
  bf16x8 sbf[RS > 0 ? RS : 1];
  if constexpr (RS > 0) {
#pragma unroll
    for (int r = 0; r < RS; ++r) sbf[r] = ld_bf16x8(sB + (int64_t)nrow * tp + 16 * r + 8 * h);
  }
  // Operands of K-step s (Ops(s)): the lane's 16-weight run and its scale, and
  // its At piece of step s + 1; loaded two steps ahead as unconditional clamped
  // loads (exact in-order wait counts).
  struct Ops {
    uint32_t scv;
    uint4 hd;
    uint4 qv;
    uint4 atr;
  };
  Ops opa, opb;
  const int apr = tp > 0 ? tp / 8 : 1;  // 16-byte pieces per At row
  const bool aok = RS > 0 && bt < 8 * tp;
  const int arow = aok ? bt / apr : 0, apc = aok ? bt % apr : 0;
  auto load_at = [&](uint4& r, int k0) __attribute__((always_inline)) {
    if constexpr (RS > 0) r = *reinterpret_cast<const uint4*>(At + (int64_t)min(k0 + arow, K - 1) * tp + 8 * apc);
  };
  // At row k_local = 16 h' + v of a 32-row half goes to LDS row 8 (v / 4) + 4 h' + v % 4
  // (see jit_kernel): lane (col, h) then holds k_local = 16 h + v in dsum[v]
  auto store_at = [&](const uint4& r, int b) __attribute__((always_inline)) {
    if constexpr (RS > 0) {
      const int half = arow >> 5, kl = arow & 31, hh = kl >> 4, v = kl & 15;
      const int lrow = 32 * half + 8 * (v >> 2) + 4 * hh + (v & 3);
      if (aok) *reinterpret_cast<uint4*>(As0 + b * kAsElems + lrow * kALD + 8 * apc) = r;
    }
  };
  // SG: the scales of K-steps 4g .. 4g + 3 (this builder's blocks 2 st + kb)
  // are one 16-byte run of its row, blocks 8g .. 8g + 7.  sgc holds the run of
  // the group being built; the next group's run is loaded into sgn with the
  // operands of step 4g + 3, three steps before its first use, and moves to sgc
  // when step 4g + 4 is built.  A step's phase st % 4 is passed as a constant
  // where the caller knows it (ph >= 0).
  uint4 sgc = make_uint4(0u, 0u, 0u, 0u), sgn = sgc;
  auto load_sg = [&](uint4& r, int g) __attribute__((always_inline)) {
    if constexpr (SG)
      r = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.sc) + (int64_t)nrow * nblk +
                                          8 * min(g, nblk / 8 - 1));
  };
  auto prefetch = [&](Ops& o, int st, int ph = -1) __attribute__((always_inline)) {
    const int k0 = min(st, nk - 1) * JBK;  // steps past the end reload the last one
    const int kbase = k0 + 32 * kb;
    if (QT == QBL_FMT_Q8) {
      if constexpr (SG) {
        if ((ph >= 0 ? ph : st & 3) == 3) load_sg(sgn, (st >> 2) + 1);
      } else {
        o.scv = reinterpret_cast<const uint16_t*>(a.sc)[(int64_t)nrow * nblk + kbase / 32];
      }
      o.qv = *reinterpret_cast<const uint4*>(a.qs + (int64_t)nrow * K + kbase + 16 * h);
    } else {
      if constexpr (QT == QBL_FMT_Q4K)
        o.hd = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.sc) +
                                               ((int64_t)nrow * (K / 256) + kbase / 256) * 16);
      else
        o.scv = reinterpret_cast<const uint32_t*>(a.sc)[(int64_t)nrow * nblk + kbase / 32];
      const uint2 q2 = *reinterpret_cast<const uint2*>(a.qs + (int64_t)nrow * (K / 2) + (kbase + 16 * h) / 2);
      o.qv = make_uint4(q2.x, q2.y, 0u, 0u);
    }
    load_at(o.atr, min(st + 1, nk - 1) * JBK);
  };
  // block (kb, nb) of the W tile of K-step k0 into buffer b; the low-rank sum
  // from the At rows in As[b]
  auto build = [&](const Ops& o, int k0, int b, int ph = -1) __attribute__((always_inline)) {
    f32x16 dsum;
#pragma unroll
    for (int v = 0; v < 16; ++v) dsum[v] = 0.0f;
    if constexpr (RS > 0) {
      const uint16_t* arow_p = As0 + b * kAsElems + (32 * kb + col) * kALD + 8 * h;
#pragma unroll
      for (int r = 0; r < RS; ++r)
        dsum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_bf16x8(arow_p + 16 * r), sbf[r], dsum, 0, 0, 0);
    }
    float d, mn;
    if constexpr (QT == QBL_FMT_Q4K) {
      float D, M;
      q4k_step_offset(o.hd, ((k0 + 32 * kb) / 32) & 7, D, M);
      d = D;
      mn = -M;
    } else {
      uint32_t scv = o.scv;
      if constexpr (SG) {  // block 2 st + kb of the run of group st / 4: dword st % 4, half kb
        const int st = k0 / JBK, p = ph >= 0 ? ph : st & 3;
        if (p == 0 && st > 0) sgc = sgn;
        const uint32_t dw = p == 0 ? sgc.x : p == 1 ? sgc.y : p == 2 ? sgc.z : sgc.w;
        scv = kb ? dw >> 16 : dw;
      }
      d = h2f(scv);
      mn = QT == QBL_FMT_Q8 ? -128.0f * d : h2f(scv >> 16);
    }
    const uint32_t qw[4] = {o.qv.x, o.qv.y, o.qv.z, o.qv.w};
    uint32_t packed[8];
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      float wv[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // as in jit_kernel: float32(dequant), plus the low-rank sum, one bf16 rounding
        const int e = v + j;
        float deq;
        if (QT == QBL_FMT_Q8)
          deq = d * (float)((qw[e >> 2] >> (8 * (e & 3))) & 0xFFu) + mn;
        else
          deq = fmaf(d, (float)((qw[e >> 3] >> (4 * (e & 7))) & 0xFu), mn);
        wv[j] = RS > 0 ? deq + dsum[e] : deq;
      }
      packed[v >> 1] = pack_bf16(wv[0], wv[1]);
    }
    uint16_t* wrow = Ws0 + b * kWsElems + (32 * nb + col) * JLD + 32 * kb + 16 * h;
    *reinterpret_cast<uint4*>(wrow) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    *reinterpret_cast<uint4*>(wrow + 8) = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  };

  {
    uint4 r0 = make_uint4(0u, 0u, 0u, 0u), r1 = r0;
    load_at(r0, 0);
    load_at(r1, min(1, nk - 1) * JBK);
    store_at(r0, 0);
    store_at(r1, 1);
  }
  __syncthreads();
  load_sg(sgc, 0);
  prefetch(opa, 0);
  build(opa, 0, 0);
  prefetch(opa, 1);
  __builtin_amdgcn_sched_barrier(0);  // Ops(1) strictly before Ops(2) (the loop's wait counts)
  prefetch(opb, 2);
  __syncthreads();
  // step ks: the next W tile (step ks + 1) from `next` into the other buffer,
  // At(ks + 2) into As[cur], `next` reloaded with Ops(ks + 3); the MFMA waves
  // work on step ks and stage X(ks + 1)
  auto step = [&](int ks, Ops& next, int ph = -1) __attribute__((always_inline)) {
    const int cur = ks & 1;
    build(next, (ks + 1) * JBK, cur ^ 1, ph < 0 ? -1 : (ph + 1) & 3);
    store_at(next.atr, cur);
    prefetch(next, ks + 3, ph < 0 ? -1 : (ph + 3) & 3);
    __syncthreads();
  };
  int ks = 0;
  if constexpr (SG) {  // four steps per iteration, phases fixed: each body's scale work is the same every time
    for (; ks + 3 < nk; ks += 4) {
      step(ks, opa, 0);
      step(ks + 1, opb, 1);
      step(ks + 2, opa, 2);
      step(ks + 3, opb, 3);
    }
  }
  for (; ks + 1 < nk; ks += 2) {
    step(ks, opa);
    step(ks + 1, opb);
  }
  if (ks < nk) step(ks, opa);
}

int rank_pad(int t) { return t <= 0 ? 0 : t <= 16 * JRMAX ? (t + 15) / 16 * 16 : (t + 63) / 64 * 64; }

template <int QT, int RS, bool FULL>
hipError_t launch_full(const JitArgs& a, int tp, const LaunchCtx& lc) {
  // (the two M-blocks of an N tile are 112 = 0 mod 8 workgroups apart for the
  // prefill shape, so they share an XCD and its L2 copy of the weight rows)
  const dim3 grid((a.n + JBN - 1) / JBN, (a.m + JBM - 1) / JBM);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&jit_kernel<QT, RS, FULL>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kJitLds);
  if (e != hipSuccess) return e;
  QBL_LAUNCH((jit_kernel<QT, RS, FULL>), grid, dim3(JTHREADS), kJitLds, lc, a, tp);
  return hipGetLastError();
}

template <int QT, int RS, bool SG>
hipError_t launch_ws_sg(const JitArgs& a, int tp, const LaunchCtx& lc) {
  const dim3 grid((a.n + JBN - 1) / JBN, a.m / JBM);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&jit_ws_kernel<QT, RS, SG>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kJitLds);
  if (e != hipSuccess) return e;
  QBL_LAUNCH((jit_ws_kernel<QT, RS, SG>), grid, dim3(JWS_THREADS), kJitLds, lc, a, tp);
  return hipGetLastError();
}

template <int QT, int RS>
hipError_t launch_ws(const JitArgs& a, int tp, const LaunchCtx& lc) {
  // q8_0 rows whose scale arrays are 16-byte aligned (K a multiple of 256) take
  // the scales 8 blocks at a time
  if constexpr (QT == QBL_FMT_Q8)
    if (a.k % 256 == 0) return launch_ws_sg<QT, RS, true>(a, tp, lc);
  return launch_ws_sg<QT, RS, false>(a, tp, lc);
}

template <int QT, int RS>
hipError_t launch_rs(const JitArgs& a, int tp, const LaunchCtx& lc) {
  if (a.m % JBM == 0 && a.k % JBK == 0) {
    if constexpr (RS <= JRMAX) return launch_ws<QT, RS>(a, tp, lc);
    return launch_full<QT, RS, true>(a, tp, lc);
  }
  return launch_full<QT, RS, false>(a, tp, lc);
}

template <int QT>
hipError_t launch_q(const JitArgs& a, int tp, const LaunchCtx& lc) {
  switch (tp / 16) {
    case 0: return launch_rs<QT, 0>(a, tp, lc);
    case 1: return launch_rs<QT, 1>(a, tp, lc);
    case 2: return launch_rs<QT, 2>(a, tp, lc);
    case 3: return launch_rs<QT, 3>(a, tp, lc);
    case 4: return launch_rs<QT, 4>(a, tp, lc);
    default: return launch_rs<QT, JRMAX + 1>(a, tp, lc);
  }
}

}  // namespace

int64_t jit_workspace_bytes(int n, int k, int total_rank) {
  const int64_t tp = rank_pad(total_rank);
  if (tp == 0) return 0;
  return ((int64_t)k * tp * 2 + 255) / 256 * 256 + ((int64_t)n * tp * 2 + 255) / 256 * 256;
}

hipError_t launch_jit(const JitArgs& a, const LaunchCtx& lc) {
  (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
  if (a.k % 32 || a.n < 1 || a.m < 1) return hipErrorInvalidValue;
  const int tp = rank_pad(a.total_rank);
  if (tp > 0) {
    if ((int64_t)a.n * tp >= (int64_t)1 << 32 || a.k % 4) return hipErrorInvalidValue;
    const int at_kt = (a.k + kStageK - 1) / kStageK, at_wgs = at_kt * ((tp + kStageT - 1) / kStageT);
    bool vec8 = true;
    for (int j = 0; j < a.n_ad; ++j) vec8 = vec8 && a.rank[j] % 8 == 0;
    const int64_t per_wg = vec8 ? 2048 : 256;
    const int64_t sb_wgs = ((int64_t)a.n * tp + per_wg - 1) / per_wg;
    if (vec8)
      hipLaunchKernelGGL(stage_lora_kernel<true>, dim3((unsigned)(at_wgs + sb_wgs)), dim3(256), 0, lc.stream, a, tp,
                         at_kt, at_wgs);
    else
      hipLaunchKernelGGL(stage_lora_kernel<false>, dim3((unsigned)(at_wgs + sb_wgs)), dim3(256), 0, lc.stream, a,
                         tp, at_kt, at_wgs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  switch (a.qtype) {
    case QBL_FMT_Q8: return launch_q<QBL_FMT_Q8>(a, tp, lc);
    case QBL_FMT_Q4: return launch_q<QBL_FMT_Q4>(a, tp, lc);
    case QBL_FMT_Q4K: return a.k % 256 ? hipErrorInvalidValue : launch_q<QBL_FMT_Q4K>(a, tp, lc);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qbl
