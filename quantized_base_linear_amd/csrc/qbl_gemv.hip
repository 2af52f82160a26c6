// Decode-path kernels for gfx950 (wave64, CDNA4).
//
//  prep_kernel : the input glue (sum of parallel projections, RMS scale) and the
//                LoRA shrink t_i = A_i x for every adapter of the next launch.
//  gemv_kernel : the fused dequant-GEMV over q8_0 / q4_sm blocks with the LoRA
//                expand s_i * B_i t_i applied in the same output write.
//
// The method is the dual path of "Deep Technical Design: Exact, Atomic,
// Reversible Specialist Overlays" (section 1: base and overlay as parallel
// streams; section 8: batch-one decode is a bandwidth-bound GEMV, and the
// adapter rows are used while the base block is being consumed), with the
// shrink/expand split of the overlay page's "Native/WASM Kernel Implications"
// (x A^T first, then the rank-r product).
//
// Every reduction has a fixed order (no atomics), and launch shapes depend only
// on tensor shapes, so a call repeated with the same inputs returns the same bits.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "qbl_kernels.h"

namespace qbl {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kLdsFloats = 16384;  // x tile budget per workgroup (64 KiB)

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over the 64 lanes of a wave, returned to every lane.  Within each row of
// 16 lanes: mirror, half-mirror and two quad permutations (each pair of lanes
// adds the same two operands, so all 16 lanes end with the same value); the
// four row sums are then combined in a fixed order.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0x140>(v);  // row_mirror
  v += dpp_mov<0x141>(v);  // row_half_mirror
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return __half2float(__ushort_as_half((unsigned short)(bits16 & 0xFFFFu)));
}

__device__ __forceinline__ float ub(uint32_t v, int byte) {
  return (float)((v >> (8 * byte)) & 0xFFu);  // selected into v_cvt_f32_ubyteN
}

// ---------------------------------------------------------------------------
// prep: xin = c * ((v0 + v1) + v2); t[b][toff + j] = A[j] . xin[b]
// ---------------------------------------------------------------------------
__device__ __forceinline__ float prep_in(const PrepArgs& a, int b, int k) {
  const int64_t o = (int64_t)b * a.v_stride + k;
  float s = a.v[0][o];
  if (a.nv > 1) s += a.v[1][o];
  if (a.nv > 2) s += a.v[2][o];
  return s;
}

__global__ __launch_bounds__(kThreads) void prep_kernel(PrepArgs a) {
  __shared__ float red[kWaves];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int K = a.k;
  float c = 1.0f;
  if (a.rms) {  // batch 1: one scale for the summed vector
    float ss = 0.0f;
    for (int k = tid; k < K; k += kThreads) {
      const float s = prep_in(a, 0, k);
      ss = fmaf(s, s, ss);
    }
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    c = 1.0f / sqrtf(tot / (float)K + 1e-6f);
  }

  // shrink: one A row per wave
  const int row = blockIdx.x * kWaves + wave;
  if (row < a.rows_total) {
    int e = 0, base = 0;
    while (base + a.ent[e].rank <= row) {
      base += a.ent[e].rank;
      ++e;
    }
    const int j = row - base;
    const float* Ar = a.ent[e].A + (int64_t)j * K;
    for (int b = 0; b < a.batch; ++b) {
      float p = 0.0f;
      for (int k = lane; k < K; k += 64) p = fmaf(Ar[k], a.rms ? c * prep_in(a, b, k) : prep_in(a, b, k), p);
      p = wave_sum(p);
      if (lane == 0) a.t[(int64_t)b * a.T + a.ent[e].toff + j] = p;
    }
  }

  // this workgroup's slice of xin
  if (a.xin) {
    const int per = (K + gridDim.x - 1) / gridDim.x;
    const int k0 = blockIdx.x * per, k1 = min(K, k0 + per);
    for (int b = 0; b < a.batch; ++b)
      for (int k = k0 + tid; k < k1; k += kThreads)
        a.xin[(int64_t)b * K + k] = a.rms ? c * prep_in(a, b, k) : prep_in(a, b, k);
  }
}

// ---------------------------------------------------------------------------
// gemv: y[b][row] = sum over the row's blocks of dequant(block) . x[b]
//                   then + s_i * (B_i[row] . t_i[b]) for each adapter, in order.
//
// Workgroup = 4 waves; each wave owns RPW consecutive rows and walks the whole
// input: lane l takes the 16-byte chunks l, l+64, l+128, ... of each of its rows
// (q8_0: 16 weights; q4_sm: 32 weights = one block).  All of a wave's weight
// loads for a tile are issued before any is consumed, so a small matrix has its
// whole byte stream in flight at once.  The input x is staged in LDS one tile
// at a time, with the 16-byte slots of each chunk rotated so that the 8 lanes
// served together by an LDS read touch 8 different bank groups, plus per-chunk
// sums of x for the integer-offset tricks in dot_q8 / the q4_sm minimum.
// ---------------------------------------------------------------------------
template <int QT>
struct Fmt {
  static constexpr int kWeightsPerChunk = QT == QBL_FMT_Q8 ? 16 : 32;
  static constexpr int kSlots = kWeightsPerChunk / 4;
  // rotation of slot j of chunk c
  __device__ static __forceinline__ int slot(int c, int j) {
    return (j + (QT == QBL_FMT_Q8 ? (c >> 1) : c)) & (kSlots - 1);
  }
};

// Sum_j q_j x_j over one q8_0 chunk of 16 int8 weights.  Each byte is biased
// to unsigned (xor 0x80) so it converts with v_cvt_f32_ubyte; the bias is
// removed with the chunk's x sum: sum (u-128) x = sum u x - 128 sum x.
__device__ __forceinline__ float dot_q8(const uint4 q, const float4* xv, float xsum) {
  const uint32_t u[4] = {q.x ^ 0x80808080u, q.y ^ 0x80808080u, q.z ^ 0x80808080u,
                         q.w ^ 0x80808080u};
  float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; w += 2) {
    s0 = fmaf(ub(u[w], 0), xv[w].x, s0);
    s0 = fmaf(ub(u[w], 1), xv[w].y, s0);
    s0 = fmaf(ub(u[w], 2), xv[w].z, s0);
    s0 = fmaf(ub(u[w], 3), xv[w].w, s0);
    s1 = fmaf(ub(u[w + 1], 0), xv[w + 1].x, s1);
    s1 = fmaf(ub(u[w + 1], 1), xv[w + 1].y, s1);
    s1 = fmaf(ub(u[w + 1], 2), xv[w + 1].z, s1);
    s1 = fmaf(ub(u[w + 1], 3), xv[w + 1].w, s1);
  }
  return fmaf(-128.0f, xsum, s0 + s1);
}

// Sum_j q_j x_j over one q4_sm block: byte i holds q_{2i} (low nibble) and
// q_{2i+1} (high nibble), so 32-bit word w covers weights 8w .. 8w+7.
__device__ __forceinline__ float dot_q4(const uint4 q, const float4* xv) {
  const uint32_t v[4] = {q.x, q.y, q.z, q.w};
  float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = v[w] & 0x0F0F0F0Fu, hi = (v[w] >> 4) & 0x0F0F0F0Fu;
    const float4 xa = xv[2 * w], xb = xv[2 * w + 1];
    s0 = fmaf(ub(lo, 0), xa.x, s0);
    s1 = fmaf(ub(hi, 0), xa.y, s1);
    s0 = fmaf(ub(lo, 1), xa.z, s0);
    s1 = fmaf(ub(hi, 1), xa.w, s1);
    s0 = fmaf(ub(lo, 2), xb.x, s0);
    s1 = fmaf(ub(hi, 2), xb.y, s1);
    s0 = fmaf(ub(lo, 3), xb.z, s0);
    s1 = fmaf(ub(hi, 3), xb.w, s1);
  }
  return s0 + s1;
}

template <int QT, int BB, int CPL>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs a) {
  extern __shared__ float lds[];
  using F = Fmt<QT>;
  constexpr int WPC = F::kWeightsPerChunk;
  constexpr int NS = F::kSlots;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wg = blockIdx.x;
  const int s = (a.nseg > 2 && wg >= a.seg[2].wg_begin) ? 2 : (a.nseg > 1 && wg >= a.seg[1].wg_begin) ? 1 : 0;
  const GemvSeg& g = a.seg[s];
  const int n = g.n;
  const int row = (wg - g.wg_begin) * kWaves + wave;  // one row per wave
  const int lrow = min(row, n - 1);                    // rows past n load row n-1, store nothing
  const int K = a.k, KT = a.kt, B = a.batch;
  const int tile_chunks = KT / WPC;
  float* xs = lds;                        // [BB][KT]
  float* xsum = xs + BB * KT;             // [BB][KT / WPC]
  float* ts = xsum + BB * tile_chunks;    // [B][T]
  const int T = a.t_stride;
  const int nblk = K / 32;
  const int64_t row_bytes = QT == QBL_FMT_Q8 ? (int64_t)K : (int64_t)K / 2;
  const uint8_t* qrow = g.qs + (int64_t)lrow * row_bytes;

  if (g.lora.n_ad > 0)
    for (int i = tid; i < B * T; i += kThreads) ts[i] = a.t[i];

  float acc[BB];
#pragma unroll
  for (int b = 0; b < BB; ++b) acc[b] = 0.0f;

  for (int k0 = 0; k0 < K; k0 += KT) {
    const int kt = min(KT, K - k0);
    const int CT = kt / WPC;
    const int c0 = k0 / WPC;

    // weight stream first: every load of this tile in flight before any use
    uint4 q[CPL];
    uint32_t sc[CPL];
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      const int c = min(lane + 64 * u, CT - 1);
      q[u] = *reinterpret_cast<const uint4*>(qrow + (int64_t)(c0 + c) * 16);
      if (QT == QBL_FMT_Q8)
        sc[u] = reinterpret_cast<const uint16_t*>(g.sc)[(int64_t)lrow * nblk + ((c0 + c) >> 1)];
      else
        sc[u] = reinterpret_cast<const uint32_t*>(g.sc)[(int64_t)lrow * nblk + c0 + c];
    }

    __syncthreads();  // the previous tile is consumed
    const int nf4 = kt / 4;
    for (int i = tid; i < BB * nf4; i += kThreads) {
      const int b = i / nf4, f = i - b * nf4;
      const int c = f / NS, j = f - c * NS;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (b < B) v = *reinterpret_cast<const float4*>(a.x + (int64_t)b * a.x_stride + k0 + 4 * f);
      *reinterpret_cast<float4*>(xs + b * KT + c * WPC + 4 * F::slot(c, j)) = v;
    }
    __syncthreads();
    for (int i = tid; i < BB * CT; i += kThreads) {
      const int b = i / CT, c = i - b * CT;
      const float* p = xs + b * KT + c * WPC;
      float sum = 0.0f;
#pragma unroll
      for (int e = 0; e < WPC; ++e) sum += p[e];
      xsum[b * tile_chunks + c] = sum;
    }
    __syncthreads();

#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      const int c = lane + 64 * u;
      if (c < CT) {
        float d, m = 0.0f;
        if (QT == QBL_FMT_Q8) {
          d = h2f(sc[u]);
        } else {
          d = h2f(sc[u]);
          m = h2f(sc[u] >> 16);
        }
#pragma unroll
        for (int b = 0; b < BB; ++b) {
          const float* xc = xs + b * KT + c * WPC;
          float4 xv[NS];
#pragma unroll
          for (int j = 0; j < NS; ++j) xv[j] = *reinterpret_cast<const float4*>(xc + 4 * F::slot(c, j));
          const float xsc = xsum[b * tile_chunks + c];
          if (QT == QBL_FMT_Q8) {
            acc[b] = fmaf(d, dot_q8(q[u], xv, xsc), acc[b]);
          } else {
            acc[b] = fmaf(d, dot_q4(q[u], xv), acc[b]);
            acc[b] = fmaf(m, xsc, acc[b]);
          }
        }
      }
    }
  }

  // epilogue: base sum complete, then the adapters in list order
  if (row < n) {
#pragma unroll
    for (int b = 0; b < BB; ++b) {
      if (b >= B) break;
      float y = wave_sum(acc[b]);
      for (int i = 0; i < g.lora.n_ad; ++i) {
        const int r = g.lora.rank[i];
        const float* Br = g.lora.B[i] + (int64_t)row * r;
        const float* ti = ts + b * T + g.lora.toff[i];
        float p = 0.0f;
        for (int j = lane; j < r; j += 64) p = fmaf(Br[j], ti[j], p);
        y = fmaf(g.lora.scale[i], wave_sum(p), y);
      }
      if (lane == 0) g.y[(int64_t)b * g.y_stride + row] = y;
    }
  }
}

template <int QT, int BB, int CPL>
hipError_t launch_one(GemvArgs& a, hipStream_t st) {
  using F = Fmt<QT>;
  const size_t lds = sizeof(float) * ((size_t)BB * a.kt + (size_t)BB * (a.kt / F::kWeightsPerChunk) +
                                      (size_t)a.batch * a.t_stride);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  if (lds > 64 * 1024) {
    static bool raised = false;  // one attribute call per instantiation
    if (!raised) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_kernel<QT, BB, CPL>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      if (e != hipSuccess) return e;
      raised = true;
    }
  }
  hipLaunchKernelGGL((gemv_kernel<QT, BB, CPL>), dim3(a.grid), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <int QT, int BB>
hipError_t launch_cpl(GemvArgs& a, int cpl, hipStream_t st) {
  if (cpl <= 1) return launch_one<QT, BB, 1>(a, st);
  if (cpl <= 2) return launch_one<QT, BB, 2>(a, st);
  if (cpl <= 4) return launch_one<QT, BB, 4>(a, st);
  if (cpl <= 8) return launch_one<QT, BB, 8>(a, st);
  if (cpl <= 12) return launch_one<QT, BB, 12>(a, st);
  return launch_one<QT, BB, 16>(a, st);
}

template <int QT>
hipError_t launch_batch(GemvArgs& a, int bb, int cpl, hipStream_t st) {
  switch (bb) {
    case 1: return launch_cpl<QT, 1>(a, cpl, st);
    case 2: return launch_cpl<QT, 2>(a, cpl, st);
    case 4: return launch_cpl<QT, 4>(a, cpl, st);
    default: return launch_cpl<QT, 8>(a, cpl, st);
  }
}

}  // namespace

hipError_t launch_prep(const PrepArgs& a, hipStream_t st) {
  const int rows_wg = (a.rows_total + kWaves - 1) / kWaves;
  int grid = rows_wg;
  if (a.xin) grid = max(grid, (a.k + 2047) / 2048);
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(prep_kernel, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gemv(GemvArgs& a, hipStream_t st) {
  const int bb = a.batch <= 1 ? 1 : a.batch <= 2 ? 2 : a.batch <= 4 ? 4 : 8;
  const int wpc = a.qtype == QBL_FMT_Q8 ? 16 : 32;
  // x tile: whole input when it fits the LDS budget, else multiples of 64 chunks
  const int quant = 64 * wpc;
  int kt = a.k;
  if ((int64_t)bb * kt > kLdsFloats) kt = max(quant, (kLdsFloats / bb) / quant * quant);
  a.kt = kt;
  const int cpl = (kt / wpc + 63) / 64;
  int wg = 0;
  for (int i = 0; i < a.nseg; ++i) {
    a.seg[i].wg_begin = wg;
    wg += (a.seg[i].n + kWaves - 1) / kWaves;
  }
  a.grid = wg;
  return a.qtype == QBL_FMT_Q8 ? launch_batch<QBL_FMT_Q8>(a, bb, cpl, st)
                               : launch_batch<QBL_FMT_Q4>(a, bb, cpl, st);
}

}  // namespace qbl
