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

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return __half2float(__ushort_as_half((unsigned short)(bits16 & 0xFFFFu)));
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// ---------------------------------------------------------------------------
// Stage the adapter factors once per call in the workspace, as bf16 with the
// scale folded into B:  At[k][t] = bf16(A_cat[t][k]),  sB[n][t] = bf16(f32(s_i B_i[n][j]))
// where t runs over the concatenated ranks (zero beyond the total rank).
// ---------------------------------------------------------------------------
__global__ void stage_lora_kernel(JitArgs a, int tp) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nat = (int64_t)a.k * tp, nsb = (int64_t)a.n * tp;
  uint16_t* At = a.ws;
  uint16_t* sB = a.ws + ((nat * 2 + 255) / 256 * 256) / 2;
  if (i < nat) {
    const int k = (int)(i / tp), t = (int)(i % tp);
    float v = 0.0f;
    int base = 0;
    for (int j = 0; j < a.n_ad; ++j) {
      if (t >= base && t < base + a.rank[j]) v = a.A[j][(int64_t)(t - base) * a.k + k];
      base += a.rank[j];
    }
    At[i] = bf16_rne(v);
  } else if (i < nat + nsb) {
    const int64_t o = i - nat;
    const int n = (int)(o / tp), t = (int)(o % tp);
    float v = 0.0f;
    int base = 0;
    for (int j = 0; j < a.n_ad; ++j) {
      if (t >= base && t < base + a.rank[j]) v = a.scale[j] * a.B[j][(int64_t)n * a.rank[j] + (t - base)];
      base += a.rank[j];
    }
    sB[o] = bf16_rne(v);
  }
}

// ---------------------------------------------------------------------------
// The fused JIT GEMM.  RS = rank steps of 16 (0: no adapters; 1..JRMAX: held
// in registers; JRMAX+1: more, streamed 64 ranks at a time).
// ---------------------------------------------------------------------------
template <int QT, int RS>
__global__ __launch_bounds__(JTHREADS) void jit_kernel(JitArgs a, int tp) {
  __shared__ __attribute__((aligned(16))) uint16_t Xs[JBM * JLD];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[JBN * JLD];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int col = lane & 31, h = lane >> 5;
  const int N = a.n, K = a.k, M = a.m;
  const int n0 = blockIdx.x * JBN, m0 = blockIdx.y * JBM;
  const int nblk = K / 32;

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

  // prefetched operands of the next K-step
  uint4 xr[4];
  uint32_t qd[4];
  uint32_t scv = 0;
  bf16x8 atf[RREG > 0 ? RREG : 1];

  auto prefetch = [&](int k0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int idx = tid + JTHREADS * c;
      const int row = idx >> 3, c16 = idx & 7;
      const int m = m0 + row, kk = k0 + 8 * c16;
      xr[c] = (m < M && kk < K) ? *reinterpret_cast<const uint4*>(a.X + (int64_t)m * K + kk)
                                : make_uint4(0u, 0u, 0u, 0u);
    }
    const int kbase = k0 + 32 * kb;
    if (kbase < K) {
      if (QT == QBL_FMT_Q8) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
          qd[g] = *reinterpret_cast<const uint32_t*>(a.qs + (int64_t)nrow * K + kbase + 8 * g + 4 * h);
        scv = reinterpret_cast<const uint16_t*>(a.sc)[(int64_t)nrow * nblk + kbase / 32];
      } else {
#pragma unroll
        for (int g = 0; g < 4; ++g)
          qd[g] = *reinterpret_cast<const uint16_t*>(a.qs + (int64_t)nrow * (K / 2) + (kbase + 8 * g + 4 * h) / 2);
        scv = reinterpret_cast<const uint32_t*>(a.sc)[(int64_t)nrow * nblk + kbase / 32];
      }
      if constexpr (RS > 0 && RS <= JRMAX) {
#pragma unroll
        for (int r = 0; r < RS; ++r) atf[r] = ld_bf16x8(At + (int64_t)(kbase + col) * tp + 16 * r + 8 * h);
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

  prefetch(0);
  for (int k0 = 0; k0 < K; k0 += JBK) {
    // ---- build this wave's 32 x 32 block of W_eff in LDS
    const int kbase = k0 + 32 * kb;
    uint16_t* wrow = Ws + (32 * nb + col) * JLD + 32 * kb + 4 * h;
    if (kbase < K) {
      f32x16 dsum;
#pragma unroll
      for (int v = 0; v < 16; ++v) dsum[v] = 0.0f;
      if constexpr (RS > 0 && RS <= JRMAX) {
#pragma unroll
        for (int r = 0; r < RS; ++r) dsum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(atf[r], sbf[r], dsum, 0, 0, 0);
      } else if constexpr (RS > JRMAX) {
        for (int r = 0; r < tp / 16; ++r) {
          const bf16x8 af = ld_bf16x8(At + (int64_t)(kbase + col) * tp + 16 * r + 8 * h);
          const bf16x8 bf = ld_bf16x8(sB + (int64_t)nrow * tp + 16 * r + 8 * h);
          dsum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, dsum, 0, 0, 0);
        }
      }
      const float d = h2f(scv);
      const float mn = QT == QBL_FMT_Q8 ? 0.0f : h2f(scv >> 16);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float wv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float deq;
          if (QT == QBL_FMT_Q8)
            deq = d * (float)((int)((qd[g] >> (8 * j)) & 0xFFu) - 128);  // offset-binary byte; exact in float32
          else
            deq = fmaf(d, (float)((qd[g] >> (4 * j)) & 0xFu), mn);           // float32(d q + m)
          wv[j] = RS > 0 ? deq + dsum[4 * g + j] : deq;
        }
        const uint32_t lo = (uint32_t)bf16_rne(wv[0]) | ((uint32_t)bf16_rne(wv[1]) << 16);
        const uint32_t hi = (uint32_t)bf16_rne(wv[2]) | ((uint32_t)bf16_rne(wv[3]) << 16);
        *reinterpret_cast<uint2*>(wrow + 8 * g) = make_uint2(lo, hi);
      }
    } else {
#pragma unroll
      for (int g = 0; g < 4; ++g) *reinterpret_cast<uint2*>(wrow + 8 * g) = make_uint2(0u, 0u);
    }
    // ---- stage the X tile
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int idx = tid + JTHREADS * c;
      const int row = idx >> 3, c16 = idx & 7;
      *reinterpret_cast<uint4*>(Xs + row * JLD + 8 * c16) = xr[c];
    }
    __syncthreads();
    if (k0 + JBK < K) prefetch(k0 + JBK);  // overlaps the MFMA phase below

    // ---- main MFMA: 64 x 64 per wave, 4 k-steps of 16
#pragma unroll
    for (int ks = 0; ks < JBK / 16; ++ks) {
      bf16x8 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = ld_bf16x8(Xs + (64 * wm + 32 * i + col) * JLD + 16 * ks + 8 * h);
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = ld_bf16x8(Ws + (64 * wn + 32 * j + col) * JLD + 16 * ks + 8 * h);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

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

int rank_pad(int t) { return t <= 0 ? 0 : t <= 16 * JRMAX ? (t + 15) / 16 * 16 : (t + 63) / 64 * 64; }

template <int QT>
hipError_t launch_q(const JitArgs& a, int tp, const LaunchCtx& lc) {
  const dim3 grid((a.n + JBN - 1) / JBN, (a.m + JBM - 1) / JBM);
  const int rs = tp / 16;
  switch (rs) {
    case 0: QBL_LAUNCH((jit_kernel<QT, 0>), grid, dim3(JTHREADS), 0, lc, a, tp); break;
    case 1: QBL_LAUNCH((jit_kernel<QT, 1>), grid, dim3(JTHREADS), 0, lc, a, tp); break;
    case 2: QBL_LAUNCH((jit_kernel<QT, 2>), grid, dim3(JTHREADS), 0, lc, a, tp); break;
    case 3: QBL_LAUNCH((jit_kernel<QT, 3>), grid, dim3(JTHREADS), 0, lc, a, tp); break;
    case 4: QBL_LAUNCH((jit_kernel<QT, 4>), grid, dim3(JTHREADS), 0, lc, a, tp); break;
    default: QBL_LAUNCH((jit_kernel<QT, JRMAX + 1>), grid, dim3(JTHREADS), 0, lc, a, tp); break;
  }
  return hipGetLastError();
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
    const int64_t total = (int64_t)a.k * tp + (int64_t)a.n * tp;
    const int threads = 256;
    hipLaunchKernelGGL(stage_lora_kernel, dim3((unsigned)((total + threads - 1) / threads)), dim3(threads), 0,
                       lc.stream, a, tp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return a.qtype == QBL_FMT_Q8 ? launch_q<QBL_FMT_Q8>(a, tp, lc) : launch_q<QBL_FMT_Q4>(a, tp, lc);
}

}  // namespace qbl
