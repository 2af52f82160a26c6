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

#include <algorithm>
#include <atomic>
#include <utility>

#include "qbl_device.h"
#include "qbl_kernels.h"

namespace qbl {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kLdsFloats = 16384;      // GEMV x tile budget per workgroup (64 KiB)
constexpr int kPrepLdsFloats = 36864;  // prep input staging budget (144 KiB)
constexpr int kPrepAPre = 12;          // float4 of the A row held in registers per thread

// Workgroup-wide sum in a fixed order; every thread receives it.  `red` holds
// kWaves floats of LDS.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float s = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return s;
}

// ---------------------------------------------------------------------------
// prep: s = v0 + v1 + v2 (summed left to right), xin = c * s, with c the RMS
// scale 1/sqrt(mean(s^2) + 1e-6) when rms is set (batch 1) and 1 otherwise;
// t[b][toff + j] = A[j] . xin[b].
//
// Workgroup g stages the whole summed input in LDS (each workgroup its own
// copy: the inputs are tens of KiB and L2-resident), computes c, then takes
// A row g (all batch rows) and slice g of the xin output.  Every load is a
// 16-byte load, unrolled so many are in flight at once.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float4 prep_in4(const PrepArgs& a, int b, int f) {
  const int64_t o = (int64_t)b * a.v_stride + 4 * (int64_t)f;
  float4 s = *reinterpret_cast<const float4*>(a.v[0] + o);
  if (a.nv > 1) s = add4(s, *reinterpret_cast<const float4*>(a.v[1] + o));
  if (a.nv > 2) s = add4(s, *reinterpret_cast<const float4*>(a.v[2] + o));
  return s;
}

template <bool LDS>
__global__ __launch_bounds__(kThreads) void prep_kernel(PrepArgs a) {
  extern __shared__ float xs[];  // [batch][K] when LDS
  __shared__ float red[kWaves];
  const int tid = threadIdx.x;
  const int K = a.k, K4 = K / 4;
  const int g = blockIdx.x;

  // this workgroup's A row, requested before the input is staged so the two
  // memory round trips overlap
  int e = 0, j = 0;
  const float* Ar = nullptr;
  if (g < a.rows_total) {
    int base = 0;
    while (base + a.ent[e].rank <= g) {
      base += a.ent[e].rank;
      ++e;
    }
    j = g - base;
    Ar = a.ent[e].A + (int64_t)j * K;
  }
  const bool apre = Ar && K4 <= kThreads * kPrepAPre;
  float4 ap[kPrepAPre];
#pragma unroll
  for (int i = 0; i < kPrepAPre; ++i) {
    const int f = tid + kThreads * i;
    ap[i] = (apre && f < K4) ? *reinterpret_cast<const float4*>(Ar + 4 * f) : make_float4(0.f, 0.f, 0.f, 0.f);
  }

  // stage s (and accumulate sum s^2 of batch row 0)
  float ss = 0.0f;
  if (LDS) {
    for (int b = 0; b < a.batch; ++b) {
#pragma unroll 8
      for (int f = tid; f < K4; f += kThreads) {
        const float4 s = prep_in4(a, b, f);
        *reinterpret_cast<float4*>(xs + (int64_t)b * K + 4 * f) = s;
        if (b == 0) ss = fmaf(s.x, s.x, fmaf(s.y, s.y, fmaf(s.z, s.z, fmaf(s.w, s.w, ss))));
      }
    }
  } else if (a.rms) {
#pragma unroll 8
    for (int f = tid; f < K4; f += kThreads) {
      const float4 s = prep_in4(a, 0, f);
      ss = fmaf(s.x, s.x, fmaf(s.y, s.y, fmaf(s.z, s.z, fmaf(s.w, s.w, ss))));
    }
  }
  float c = 1.0f;
  if (a.rms) {
    const float tot = block_sum(ss, red);  // its barrier also publishes xs
    c = 1.0f / sqrtf(tot / (float)K + 1e-6f);
  } else if (LDS) {
    __syncthreads();
  }

  // shrink: A row g for every batch row
  if (Ar) {
    for (int b = 0; b < a.batch; ++b) {
      float p = 0.0f;
      if (apre) {
#pragma unroll
        for (int i = 0; i < kPrepAPre; ++i) {
          const int f = tid + kThreads * i;
          if (f < K4) {
            const float4 w = ap[i];
            float4 s = LDS ? *reinterpret_cast<const float4*>(xs + (int64_t)b * K + 4 * f) : prep_in4(a, b, f);
            if (a.rms) s = mul4(c, s);
            p = fmaf(w.x, s.x, p);
            p = fmaf(w.y, s.y, p);
            p = fmaf(w.z, s.z, p);
            p = fmaf(w.w, s.w, p);
          }
        }
      } else {
#pragma unroll 8
        for (int f = tid; f < K4; f += kThreads) {
          const float4 w = *reinterpret_cast<const float4*>(Ar + 4 * f);
          float4 s = LDS ? *reinterpret_cast<const float4*>(xs + (int64_t)b * K + 4 * f) : prep_in4(a, b, f);
          if (a.rms) s = mul4(c, s);
          p = fmaf(w.x, s.x, p);
          p = fmaf(w.y, s.y, p);
          p = fmaf(w.z, s.z, p);
          p = fmaf(w.w, s.w, p);
        }
      }
      p = block_sum(p, red);
      if (tid == 0) a.t[(int64_t)b * a.T + a.ent[e].toff + j] = p;
    }
  }

  // slice g of xin
  if (a.xin) {
    const int per = (K4 + gridDim.x - 1) / gridDim.x;
    const int f0 = g * per, f1 = min(K4, f0 + per);
    for (int b = 0; b < a.batch; ++b)
      for (int f = f0 + tid; f < f1; f += kThreads) {
        float4 s = LDS ? *reinterpret_cast<const float4*>(xs + (int64_t)b * K + 4 * f) : prep_in4(a, b, f);
        if (a.rms) s = mul4(c, s);
        *reinterpret_cast<float4*>(a.xin + (int64_t)b * K + 4 * f) = s;
      }
  }
}

// ---------------------------------------------------------------------------
// gemv: y[b][row] = sum over the row's blocks of dequant(block) . x[b]
//                   then + s_i * (B_i[row] . t_i[b]) for each adapter, in order.
//
// Workgroup = 4 waves; each wave owns RPW consecutive rows and walks the whole
// input: lane l takes the 16-byte chunks l, l+64, l+128, ... of each of its rows
// (q8_0: 16 weights; q4_sm: 32 weights = one block).  All of a wave's weight
// loads for a tile, and the B rows of its adapters, are issued before anything
// is consumed, so a small matrix has its whole byte stream in flight at once.
// The input x is staged in LDS one tile at a time, each thread staging whole
// chunks and their sums (used by the integer-offset tricks below); the 16-byte
// slots of each chunk are rotated so that the 8 lanes served together by an
// LDS read touch 8 different bank groups.
// ---------------------------------------------------------------------------
constexpr int kPrefetchAdapters = 2;  // B rows prefetched for lists of <= 2 adapters of rank <= 64

template <int QT, int BB, int CPL, int RPW>
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
  const int row0 = (wg - g.wg_begin) * (kWaves * RPW) + wave * RPW;
  const int K = a.k, KT = a.kt, B = a.batch;
  const int tile_chunks = KT / WPC;
  float* xs = lds;                        // [BB][KT]
  float* xsum = xs + BB * KT;             // [BB][KT / WPC]
  float* ts = xsum + BB * tile_chunks;    // [B][T]
  const int T = a.t_stride;
  const int64_t row_bytes = F::row_bytes(K);
  const int n_ad = g.lora.n_ad;
  const bool prefetch = g.lora.prefetch != 0;

  int lrow[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) lrow[r] = min(row0 + r, n - 1);  // rows past n load row n-1, store nothing

  // B rows of the (at most two) adapters, one value per lane
  float bpre[RPW][kPrefetchAdapters];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int i = 0; i < kPrefetchAdapters; ++i) {
      bpre[r][i] = 0.0f;
      if (prefetch && i < n_ad && lane < g.lora.rank[i])
        bpre[r][i] = g.lora.B[i][(int64_t)lrow[r] * g.lora.rank[i] + lane];
    }

  float acc[RPW][BB];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int b = 0; b < BB; ++b) acc[r][b] = 0.0f;

  for (int k0 = 0; k0 < K; k0 += KT) {
    const int kt = min(KT, K - k0);
    const int CT = kt / WPC;
    const int c0 = k0 / WPC;

    // this thread's chunks of x first (they gate the barrier), then the whole
    // weight stream of the wave, then x into LDS
    constexpr int XC = 1;  // x chunks per thread loaded ahead of the weights
    float4 xv_st[XC][NS];
#pragma unroll
    for (int h = 0; h < XC; ++h) {
      const int i = tid + kThreads * h;
      const int b = i / CT, c = i - b * CT;
#pragma unroll
      for (int j = 0; j < NS; ++j)
        xv_st[h][j] = (i < BB * CT && b < B)
                          ? *reinterpret_cast<const float4*>(a.x + (int64_t)b * a.x_stride + k0 + c * WPC + 4 * j)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    uint4 q[RPW][CPL];
    typename F::Sc sc[RPW][CPL];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const uint8_t* qrow = g.qs + (int64_t)lrow[r] * row_bytes;
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        const int c = min(lane + 64 * u, CT - 1);
        q[r][u] = stream_load16(qrow + (int64_t)(c0 + c) * 16);
        sc[r][u] = F::load_sc(g.sc, lrow[r], K, c0 + c);
      }
    }

    if (k0 > 0) __syncthreads();  // the previous tile is consumed
    if (k0 == 0 && n_ad > 0)
      for (int i = tid; i < B * T; i += kThreads) ts[i] = a.t[i];
    // stage whole chunks of x and their sums
    auto stage = [&](int i, const float4* v) {
      const int b = i / CT, c = i - b * CT;
      float sum = 0.0f;
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        sum += v[j].x;
        sum += v[j].y;
        sum += v[j].z;
        sum += v[j].w;
      }
#pragma unroll
      for (int j = 0; j < NS; ++j)
        *reinterpret_cast<float4*>(xs + b * KT + c * WPC + 4 * F::slot(c, j)) = v[j];
      xsum[b * tile_chunks + c] = sum;
    };
#pragma unroll
    for (int h = 0; h < XC; ++h)
      if (tid + kThreads * h < BB * CT) stage(tid + kThreads * h, xv_st[h]);
    for (int i = tid + kThreads * XC; i < BB * CT; i += kThreads) {
      const int b = i / CT, c = i - b * CT;
      float4 v[NS];
#pragma unroll
      for (int j = 0; j < NS; ++j)
        v[j] = b < B ? *reinterpret_cast<const float4*>(a.x + (int64_t)b * a.x_stride + k0 + c * WPC + 4 * j)
                     : make_float4(0.f, 0.f, 0.f, 0.f);
      stage(i, v);
    }
    __syncthreads();

#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      const int c = lane + 64 * u;
      if (c < CT) {
#pragma unroll
        for (int b = 0; b < BB; ++b) {
          const float* xc = xs + b * KT + c * WPC;
          float4 xv[NS];
#pragma unroll
          for (int j = 0; j < NS; ++j) xv[j] = *reinterpret_cast<const float4*>(xc + 4 * F::slot(c, j));
          const float xsc = xsum[b * tile_chunks + c];
#pragma unroll
          for (int r = 0; r < RPW; ++r) acc[r][b] = chunk_dot<QT>(acc[r][b], q[r][u], xv, xsc, sc[r][u], c0 + c);
        }
      }
    }
  }

  // epilogue: each lane adds s_i * B_i[row][j] * t_i[j] for its j to its
  // partial sum, adapters in list order; then one wave reduction per output
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int row = row0 + r;
    if (row >= n) break;
#pragma unroll
    for (int b = 0; b < BB; ++b) {
      if (b >= B) break;
      float v = acc[r][b];
      for (int i = 0; i < n_ad; ++i) {
        const int rk = g.lora.rank[i];
        if (rk == 0) {  // sparse delta: lanes strided over the row's entries
          const float* xb = a.x + (int64_t)b * a.x_stride;
          const float p = csr_row_dot(g.lora.ci[i], g.lora.sv[i], g.lora.rp[i][row], g.lora.rp[i][row + 1], lane,
                                      [&](uint32_t c) { return *gp(xb + c); });
          v = fmaf(g.lora.scale[i], p, v);
          continue;
        }
        const float* ti = ts + b * T + g.lora.toff[i];
        if (prefetch) {
          const float bv = i == 0 ? bpre[r][0] : bpre[r][1];
          if (lane < rk) v = fmaf(g.lora.scale[i], bv * ti[lane], v);
        } else {
          const float* Br = g.lora.B[i] + (int64_t)row * rk;
          float p = 0.0f;
          for (int j = lane; j < rk; j += 64) p = fmaf(Br[j], ti[j], p);
          v = fmaf(g.lora.scale[i], p, v);
        }
      }
      const float y = wave_sum(v);
      if (lane == 0) g.y[(int64_t)b * g.y_stride + row] = y;
    }
  }
}

// Dynamic LDS above 64 KiB needs a per-kernel opt-in; raise it to what this
// launch needs (static LDS of these kernels is at most 16 bytes).
constexpr size_t kMaxDynLds = 160 * 1024 - 256;

hipError_t allow_dyn_lds(const void* fn, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  if (bytes > kMaxDynLds) return hipErrorInvalidValue;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}


// ---------------------------------------------------------------------------
// Batch-1 kernel: glue + shrink + GEMV + expand in one launch.
//
// Layout of the work.  A workgroup of W waves splits the input dimension: the
// 16-byte chunks of a weight row are taken in blocks of 64 (one per lane), and
// wave w owns blocks w, w+W, w+2W, ...  Each lane loads the input values under
// its chunks once into registers and keeps them for every row the workgroup
// computes, so the input is read once per workgroup however many rows it has.
// Rows are streamed in groups of G, the next group's loads in flight while the
// current one is consumed; a row's partial sums are reduced within each wave,
// then across the W waves in LDS, in a fixed order.
//
// Glue.  The input is one vector s (the launcher sends inputs that are sums of
// several vectors to the prep + GEMV path), scaled by the RMS factor
// c = 1/sqrt(mean(s^2) + 1e-6) when rms is set; c multiplies the finished dot
// products.  With `sum` set, the segments (same height) are computed by the
// same workgroups and written as one vector y0 = y_seg0 + y_seg1 (+ y_seg2): the
// block's glue needs only the sum of parallel projections.
//
// Shrink.  t = c (A s), each value stored as one 64-bit word tagged with the
// launch's number.  GEMV workgroup i < rows_total computes t[i] from the input
// it holds anyway (one A row: its load rides with the first weight loads)
// before its own rows; only when a launch has fewer GEMV workgroups than A rows
// do separate workgroups [0, shrink_wgs) compute t, kRS rows of A each.
// (Separate shrink workgroups land as an extra workgroup on a few compute units
// and make those the last to finish: in the 7B block's q+k+v launch, 12 of
// them, 64 KiB of A each, ended the launch ~2.6 us after the other units.)
// The producers are dispatched first and never wait.  GEMV workgroups read t
// only after their row loop, waiting (bounded) until each word carries this
// launch's tag: the data is its own flag, so the hand-off needs no counters,
// fences or cache maintenance and nothing is reset afterwards.
// ---------------------------------------------------------------------------
constexpr int kB1MaxSlots = 64;   // output rows (over all segments) per workgroup
constexpr int kB1MaxT = kMaxSegs * 512;

template <int QT, int CPW>
struct B1Shape {
  static constexpr int kNS = Fmt<QT>::kSlots;
  static constexpr int kG = CPW >= 3 ? 1 : 2;                                   // rows per load group
  static constexpr int kRS = CPW * kNS >= 16 ? 1 : 16 / (CPW * kNS);           // A rows per shrink workgroup
  static constexpr bool kShrinkInGemv = CPW == 1;                               // GEMV workgroups compute t
};

// waves per SIMD the register budget targets: 4 waves, one q8_0 block of chunks
// per lane and two-row groups fit in 96 VGPRs, which lets 5 waves share a SIMD
template <int QT, int W, int CPW>
constexpr int b1_min_waves() { return W == 4 && CPW * Fmt<QT>::kSlots <= 4 ? 5 : 1; }

// v0, v1 or v2 by a wave-uniform index i < 3, as two conditional moves (a
// three-way ?: chain may be compiled into a table in scratch memory)
template <class T>
__device__ __forceinline__ T pick3(int i, T v0, T v1, T v2) {
  T r = v0;
  asm volatile("" : "+s"(r));
  r = i >= 1 ? v1 : r;
  asm volatile("" : "+s"(r));
  return i >= 2 ? v2 : r;
}

// Flags word of the batch-1 launch's leading scalar arguments.
__host__ __device__ constexpr int b1_flags(int sum, int nseg, int shrink_in_gemv, int shrink_wgs) {
  return sum | nseg << 3 | shrink_in_gemv << 5 | shrink_wgs << 8;
}

// The first scalar arguments (segment 0's weights and scales, the input, the
// row length, the first GEMV workgroup, rows per workgroup, segment 0's height,
// the flags word, the number of shrink values) repeat fields of f.  The
// library is compiled to preload leading scalar arguments into registers at
// wave launch, so the first weight and input loads wait for no argument
// fetch; everything else is read from f, and only behind uniform branches that
// the first loads do not take.
template <int QT, int W, int CPW, int G, bool XL>
__global__ __launch_bounds__(W * 64, (b1_min_waves<QT, W, CPW>())) void gemv_b1_kernel(
    const uint8_t* p_qs0, const void* p_sc0, const float* p_v0, int p_k, int p_first, int p_rows, int p_n0,
    int p_flags, int p_rt, FusedArgs f) {
  using F = Fmt<QT>;
  using S = B1Shape<QT, CPW>;
  constexpr int WPC = F::kWeightsPerChunk;
  constexpr int NS = F::kSlots;
  constexpr int RS = S::kRS;
  constexpr int NT = W * 64;
  constexpr int LG = G == 8 ? 3 : G == 4 ? 2 : G == 2 ? 1 : 0;
  __shared__ float red[W][kB1MaxSlots][4];  // per wave, slot, 16-lane row
  __shared__ float ssred[W];
  __shared__ float tred[W];
  __shared__ float tl[kB1MaxT];
  __shared__ float outl[kB1MaxSlots];

  const GemvArgs& a = f.g;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h_sum = p_flags & 1, h_nseg = (p_flags >> 3) & 3, h_sig = (p_flags >> 5) & 1;
  const int h_shrink = p_flags >> 8, h_sparse = p_first - h_shrink, h_rt = p_rt, h_R = p_rows, h_K = p_k;
  const int K = h_K, CT = K / WPC;
  const int64_t row_bytes = F::row_bytes(K);
  const bool shrinker = (int)blockIdx.x < h_shrink;
  const int wg = (int)blockIdx.x - h_shrink - h_sparse;
  // GEMV workgroup wg < rows_total computes t[wg] (no shrink workgroups; shapes
  // with one chunk per lane, where the A row's registers fit beside the first
  // weight loads)
  const bool trow = S::kShrinkInGemv && h_sig && !shrinker && wg >= 0 && wg < h_rt;

  // ---- sparse workgroups [shrink_wgs, shrink_wgs + sparse_wgs): a wave per
  // (segment, sparse adapter, row) item, its lanes strided over the row's
  // entries, gathering the unscaled input s (the RMS factor is
  // applied by the row's GEMV workgroup); one wave reduction per item, stored
  // as a tagged word like the shrink values.  They precede every GEMV
  // workgroup in dispatch order and never wait.
  if (!shrinker && wg < 0) {
    constexpr int kSpR = 2;  // items (rows) per wave at once (1, 3 and 4 measured slower)
    const int per = (f.sp_items + f.sparse_wgs - 1) / f.sparse_wgs;
    const int i0 = ((int)blockIdx.x - f.shrink_wgs) * per, i1 = min(f.sp_items, i0 + per);
    for (int g0 = i0 + kSpR * wave; g0 < i1; g0 += kSpR * W) {
      const uint32_t* col[kSpR];
      const uint16_t* val[kSpR];
      uint32_t e0[kSpR], e1[kSpR];
#pragma unroll
      for (int r = 0; r < kSpR; ++r) {
        const int item = g0 + r;
        int sg = 0, ad = 0;
        for (int q = 0; q < a.nseg; ++q)
          for (int i = 0; i < a.seg[q].lora.n_ad; ++i)
            if (f.sp_base[q][i] >= 0 && item >= f.sp_base[q][i] && item < f.sp_base[q][i] + a.seg[q].n) sg = q, ad = i;
        const LoraSeg& L = a.seg[sg].lora;
        col[r] = L.ci[ad];
        val[r] = L.sv[ad];
        e0[r] = e1[r] = 0;
        if (item < i1) {
          const int row = item - f.sp_base[sg][ad];
          e0[r] = L.rp[ad][row];
          e1[r] = L.rp[ad][row + 1];
        }
      }
      float p[kSpR];
      csr_rows_dot<kSpR, 4>(col, val, e0, e1, lane, [&](uint32_t c) { return *gp(p_v0 + c); }, p);
#pragma unroll
      for (int r = 0; r < kSpR; ++r) {
        const float w = wave_sum(p[r]);
        if (lane == 0 && g0 + r < i1)
          __hip_atomic_store(f.sp + g0 + r, ((uint64_t)f.tag << 32) | __float_as_uint(w), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    return;
  }

  // this lane's chunks
  int cidx[CPW];
  bool cval[CPW];
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int c = 64 * (u * W + wave) + lane;
    cval[u] = c < CT;
    // lanes past the row end read a valid chunk (their inputs are zero); for
    // q4_K the same lane of the last super-block, so that every quad still
    // holds one whole header (CT is a multiple of 8 there)
    cidx[u] = c < CT ? c : QT == QBL_FMT_Q4K ? CT - 8 + (lane & 7) : CT - 1;
  }

  // ---- the workgroup's rows (GEMV role)
  int sg0 = 0, row0 = 0, nslots = 0, R = h_R;
  if (!shrinker) {
    if (h_sum) {
      row0 = wg * R;
      nslots = R * h_nseg;
    } else {
      row0 = wg * R;
      nslots = R;
      if (h_nseg > 1) {  // several segments side by side: which one holds wg
        asm volatile("");
        const int wgb1 = a.seg[1].wg_begin, wgb2 = a.seg[2].wg_begin;
        sg0 = (h_nseg > 2 && wg >= wgb2) ? 2 : wg >= wgb1 ? 1 : 0;
        row0 = (wg - pick3(sg0, 0, wgb1, wgb2)) * R;
      }
    }
  }
  auto slot_seg = [&](int s) { return h_sum ? s / R : sg0; };
  auto slot_row = [&](int s) { return row0 + (h_sum ? s % R : s); };

  // ---- loads: the input (L2-resident), then the weight stream (or the A rows
  // when shrinking); the expand's B values are read after the row loop
  float4 xr[CPW][NS];
#pragma unroll
  for (int u = 0; u < CPW; ++u)
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      float4 t4 = make_float4(0.f, 0.f, 0.f, 0.f);
      if (cval[u]) {
        const int64_t o = (int64_t)cidx[u] * WPC + 4 * j;
        t4 = gload4(p_v0 + o);
      }
      xr[u][j] = t4;
    }

  using Sc = typename F::Sc;
  uint4 qa[G][CPW], qb[G][CPW];
  Sc sa[G][CPW], sb[G][CPW];
  float4 av[RS][CPW][NS];
  auto load_group = [&](uint4 (&q)[G][CPW], Sc (&sc)[G][CPW], int grp) {
#pragma unroll
    for (int r = 0; r < G; ++r) {
      const int s = grp * G + r;
      if (s < nslots) {
        const int sg = slot_seg(s);
        const uint8_t* qs = p_qs0;
        const void* scp = p_sc0;
        int n = p_n0;
        if (sg != 0) {  // segment 0's values come with the launch; the others from f
          asm volatile("");
          qs = pick3(sg, p_qs0, a.seg[1].qs, a.seg[2].qs);
          scp = pick3(sg, p_sc0, a.seg[1].sc, a.seg[2].sc);
          n = pick3(sg, p_n0, a.seg[1].n, a.seg[2].n);
        }
        const int row = min(slot_row(s), n - 1);
        const uint8_t* qrow = qs + (int64_t)row * row_bytes;
#pragma unroll
        for (int u = 0; u < CPW; ++u) {
          q[r][u] = stream_load16(qrow + (int64_t)cidx[u] * 16);
          sc[r][u] = F::load_sc(scp, row, K, cidx[u]);
        }
      }
    }
  };
  const int ngroups = (nslots + G - 1) / G;
  if (shrinker) {
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      const int arow = (int)blockIdx.x * RS + rs;
      const float* Ar = nullptr;
      if (arow < f.rows_total) {
        int e = 0, base = 0;
        while (base + f.ent[e].rank <= arow) {
          base += f.ent[e].rank;
          ++e;
        }
        Ar = f.ent[e].A + (int64_t)(arow - base) * K;
      }
#pragma unroll
      for (int u = 0; u < CPW; ++u)
#pragma unroll
        for (int j = 0; j < NS; ++j)
          av[rs][u][j] = Ar ? *reinterpret_cast<const float4*>(Ar + (int64_t)cidx[u] * WPC + 4 * j)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  } else {
    if (ngroups > 0) load_group(qa, sa, 0);
    if (ngroups > 1) load_group(qb, sb, 1);
    if (trow) {  // after the first weight loads: finding the A row reads the entry list
      int e = 0, base = 0;
      while (base + f.ent[e].rank <= wg) {
        base += f.ent[e].rank;
        ++e;
      }
      const float* Ar = f.ent[e].A + (int64_t)(wg - base) * K;
#pragma unroll
      for (int u = 0; u < CPW; ++u)
#pragma unroll
        for (int j = 0; j < NS; ++j) av[0][u][j] = *reinterpret_cast<const float4*>(Ar + (int64_t)cidx[u] * WPC + 4 * j);
    }
  }

  // ---- chunk sums and sum of squares of the input
  float xsm[CPW];
  float ss = 0.0f;
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const float4 t4 = xr[u][j];
      sum += t4.x;
      sum += t4.y;
      sum += t4.z;
      sum += t4.w;
      ss = fmaf(t4.x, t4.x, fmaf(t4.y, t4.y, fmaf(t4.z, t4.z, fmaf(t4.w, t4.w, ss))));
    }
    xsm[u] = sum;
  }
  float cscale = 1.0f;
  if (f.rms) {
    const float w = wave_sum(ss);
    if (lane == 0) ssred[wave] = w;
    __syncthreads();
    float tot = 0.0f;
#pragma unroll
    for (int i = 0; i < W; ++i) tot += ssred[i];
    cscale = 1.0f / sqrtf(tot / (float)K + 1e-6f);
  }

  if (shrinker) {
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      float p = 0.0f;
#pragma unroll
      for (int u = 0; u < CPW; ++u)
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          p = fmaf(av[rs][u][j].x, xr[u][j].x, p);
          p = fmaf(av[rs][u][j].y, xr[u][j].y, p);
          p = fmaf(av[rs][u][j].z, xr[u][j].z, p);
          p = fmaf(av[rs][u][j].w, xr[u][j].w, p);
        }
      p = wave_sum(p);
      if (lane == 0) red[wave][rs][0] = p;
    }
    __syncthreads();
    const int arow = (int)blockIdx.x * RS + tid;
    if (tid < RS && arow < f.rows_total) {
      float p = 0.0f;
#pragma unroll
      for (int i = 0; i < W; ++i) p += red[i][tid][0];
      const uint64_t word = ((uint64_t)f.tag << 32) | __float_as_uint(cscale * p);
      for (int c = 0; c < kTCopies; ++c)
        __hip_atomic_store(f.t + (int64_t)c * f.t_copy_stride + arow, word, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  if (trow) {  // t[wg], as a shrink workgroup would (inputs past the row end are zero)
    float p = 0.0f;
#pragma unroll
    for (int u = 0; u < CPW; ++u)
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        p = fmaf(av[0][u][j].x, xr[u][j].x, p);
        p = fmaf(av[0][u][j].y, xr[u][j].y, p);
        p = fmaf(av[0][u][j].z, xr[u][j].z, p);
        p = fmaf(av[0][u][j].w, xr[u][j].w, p);
      }
    p = wave_sum(p);
    if (lane == 0) tred[wave] = p;
    __syncthreads();
    if (tid == 0) {
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < W; ++i) s += tred[i];
      const uint64_t word = ((uint64_t)f.tag << 32) | __float_as_uint(cscale * s);
      for (int c = 0; c < kTCopies; ++c)
        __hip_atomic_store(f.t + (int64_t)c * f.t_copy_stride + wg, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // ---- row loop: two groups in flight; each group's rows reduced together
  auto compute_group = [&](const uint4 (&q)[G][CPW], const Sc (&sc)[G][CPW], int grp) {
    float p[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) p[r] = 0.0f;
#pragma unroll
    for (int r = 0; r < G; ++r) {
#pragma unroll
      for (int u = 0; u < CPW; ++u) p[r] = chunk_dot<QT>(p[r], q[r][u], xr[u], xsm[u], sc[r][u], cidx[u]);
    }
    reduce_rows16<G>(p, lane);
    const int r = (lane & 15) >> (4 - LG);
    const int s = grp * G + r;
    if ((lane & ((16 >> LG) - 1)) == 0 && s < nslots) red[wave][s][lane >> 4] = p[0];
  };
  // the first read of the shrink words goes out halfway through the row loop
  // (the shrink workgroups, dispatched first, are done by then), so its round
  // trip overlaps the remaining groups; a word still stale is read again at
  // the end
  constexpr int kTW = 2;
  const uint64_t* tcopy = f.t + (int64_t)(wg % kTCopies) * f.t_copy_stride;
  uint64_t tw[kTW];
  bool tw_out = false;
  auto issue_t = [&] {
#pragma unroll
    for (int m = 0; m < kTW; ++m) {
      const int j = tid + m * NT;
      tw[m] = j < f.rows_total ? __hip_atomic_load(tcopy + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
    }
    tw_out = true;
  };
  for (int grp = 0; grp < ngroups; grp += 2) {
    if (!tw_out && 2 * grp + 2 >= ngroups) issue_t();
    compute_group(qa, sa, grp);
    if (grp + 2 < ngroups) load_group(qa, sa, grp + 2);
    if (grp + 1 < ngroups) {
      compute_group(qb, sb, grp + 1);
      if (grp + 3 < ngroups) load_group(qb, sb, grp + 3);
    }
  }

  // ---- shrink values of this launch, then the row outputs
  HandoffWait hw(f.fail, f.wait_ticks);
  if (!tw_out) issue_t();
#pragma unroll
  for (int m = 0; m < kTW; ++m) {
    const int j = tid + m * NT;
    if (j < f.rows_total)
      tl[j] = (uint32_t)(tw[m] >> 32) == f.read_tag ? __uint_as_float((uint32_t)tw[m]) : tagged_get(tcopy + j, f.read_tag, hw);
  }
  for (int j = tid + kTW * NT; j < f.rows_total; j += NT) tl[j] = tagged_get(tcopy + j, f.read_tag, hw);

  // the first sparse value of each row, requested before the barrier so that
  // its round trip overlaps the wait there
  __shared__ uint64_t spl[XL ? kB1MaxSlots : 1];
  __shared__ int spf[XL ? kB1MaxSlots : 1];
  uint64_t spw = 0;
  int sp_first = -1;
  if (f.sp_items > 0 && tid < nslots) {
    const int sg = slot_seg(tid), row = slot_row(tid);
    for (int i = 0; i < a.seg[sg].lora.n_ad && sp_first < 0; ++i)
      if (f.sp_base[sg][i] >= 0) sp_first = i;
    if (sp_first >= 0 && row < a.seg[sg].n)
      spw = __hip_atomic_load(f.sp + f.sp_base[sg][sp_first] + row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if constexpr (XL) {  // for the row's lane group (below)
      spl[tid] = spw;
      spf[tid] = sp_first;
    }
  }
  __syncthreads();
  if (!XL && tid < nslots) {  // one thread per row (the launch's ranks are at most 32)
    const int s = tid;
    const GemvSeg& g = a.seg[slot_seg(s)];
    const int row = slot_row(s);
    float v = 0.0f;
#pragma unroll
    for (int i = 0; i < W; ++i) v += (red[i][s][0] + red[i][s][1]) + (red[i][s][2] + red[i][s][3]);
    v *= cscale;
    for (int i = 0; i < g.lora.n_ad; ++i) {
      const int rk = g.lora.rank[i];
      if (rk == 0) {
        float p = 0.0f;
        if (row < g.n) {
          const uint64_t* w = f.sp + f.sp_base[slot_seg(s)][i] + row;
          p = i == sp_first && (uint32_t)(spw >> 32) == f.read_tag ? __uint_as_float((uint32_t)spw)
                                                                  : tagged_get(w, f.read_tag, hw);
        }
        v = fmaf(g.lora.scale[i], cscale * p, v);
        continue;
      }
      const float* ti = tl + g.lora.toff[i];
      const float* Br = g.lora.B[i] + (int64_t)min(row, g.n - 1) * rk;
      float p = 0.0f;
      int j = 0;
      if (rk % 4 == 0) {  // 16-byte B loads, four in flight (the row is 16-byte aligned)
#pragma unroll 4
        for (; j < rk; j += 4) {
          const float4 b4 = gload4(Br + j);
          p = fmaf(b4.x, ti[j], p);
          p = fmaf(b4.y, ti[j + 1], p);
          p = fmaf(b4.z, ti[j + 2], p);
          p = fmaf(b4.w, ti[j + 3], p);
        }
      }
#pragma unroll 8
      for (; j < rk; ++j) p = fmaf(Br[j], ti[j], p);
      v = fmaf(g.lora.scale[i], p, v);
    }
    if (f.sum) outl[s] = v;
    else if (row < g.n) g.y[row] = v;
  }
  // With ranks above 32 (XL) each row finishes in a group of lps lanes (one per
  // 16 of the launch's largest rank, up to 16, as the workgroup's threads
  // allow): the lanes split each adapter's B row (16-byte pieces lps apart), so
  // every lane issues at most four loads at once, and a fixed xor tree adds
  // their partial sums (the same bits in every lane).  Launches whose ranks are
  // at most 32 run the kernel compiled without this path (carrying it cost the
  // rank-16 block step 0.6 us).
  int lps = f.expand_lanes;
  while (lps > 1 && lps * nslots > NT) lps >>= 1;
  const int s = tid / lps, q = tid & (lps - 1);
  if (XL && s < nslots) {
    const GemvSeg& g = a.seg[slot_seg(s)];
    const int row = slot_row(s);
    float v = 0.0f;
#pragma unroll
    for (int i = 0; i < W; ++i) v += (red[i][s][0] + red[i][s][1]) + (red[i][s][2] + red[i][s][3]);
    v *= cscale;
    for (int i = 0; i < g.lora.n_ad; ++i) {
      const int rk = g.lora.rank[i];
      if (rk == 0) {  // sparse: the group's first lane (only its v is stored)
        float p = 0.0f;
        if (q == 0 && row < g.n) {
          const uint64_t* w = f.sp + f.sp_base[slot_seg(s)][i] + row;
          const uint64_t sw = spl[s];
          p = i == spf[s] && (uint32_t)(sw >> 32) == f.read_tag ? __uint_as_float((uint32_t)sw)
                                                                  : tagged_get(w, f.read_tag, hw);
        }
        v = fmaf(g.lora.scale[i], cscale * p, v);
        continue;
      }
      const float* ti = tl + g.lora.toff[i];
      const float* Br = g.lora.B[i] + (int64_t)min(row, g.n - 1) * rk;
      float p = 0.0f;
      if (rk % 4 == 0) {  // 16-byte B loads (the row is 16-byte aligned), up to four issued together
        for (int j0 = 4 * q; j0 < rk; j0 += 16 * lps) {
          float4 b4[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            b4[u] = j0 + 4 * lps * u < rk ? gload4(Br + j0 + 4 * lps * u) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int j = j0 + 4 * lps * u;
            if (j < rk) {
              p = fmaf(b4[u].x, ti[j], p);
              p = fmaf(b4[u].y, ti[j + 1], p);
              p = fmaf(b4[u].z, ti[j + 2], p);
              p = fmaf(b4[u].w, ti[j + 3], p);
            }
          }
        }
      } else {
        for (int j = q; j < rk; j += lps) p = fmaf(Br[j], ti[j], p);
      }
      for (int o = lps >> 1; o > 0; o >>= 1) p += __shfl_xor(p, o);
      v = fmaf(g.lora.scale[i], p, v);
    }
    if (q == 0) {
      if (f.sum) outl[s] = v;
      else if (row < g.n) g.y[row] = v;
    }
  }
  if (f.sum) {
    __syncthreads();
    const int row = row0 + tid;
    if (tid < R && row < a.seg[0].n) {
      float y = outl[tid];
      for (int i = 1; i < a.nseg; ++i) y += outl[i * R + tid];
      a.seg[0].y[row] = y;
    }
  }
}

// Workgroups of gemv_b1_kernel<QT, W, CPW, G, XL> that one CU holds at once.
template <int QT, int W, int CPW, int G, bool XL>
int b1_resident_per_cu() {
  static std::atomic<int> cached{0};
  int n = cached.load(std::memory_order_relaxed);
  if (!n) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(&gemv_b1_kernel<QT, W, CPW, G, XL>), W * 64, 0) != hipSuccess ||
        n < 1)
      n = 1;
    cached.store(n, std::memory_order_relaxed);
  }
  return n;
}

int device_cus() {
  static std::atomic<int> cached{0};
  int n = cached.load(std::memory_order_relaxed);
  if (!n) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    cached.store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int QT, int W, int CPW, int G = B1Shape<QT, CPW>::kG>
hipError_t launch_b1_t(FusedArgs& f, const LaunchCtx& lc) {
  using S = B1Shape<QT, CPW>;
  GemvArgs& a = f.g;
  // The GEMV workgroups compute t when several share a compute unit (a separate
  // shrink workgroup would be an extra one on a unit with a full share of rows);
  // with one workgroup per unit, separate shrink workgroups take units of their
  // own and the rows spread over the others.  Separate ones also when there are
  // fewer GEMV workgroups than A rows.
  int max_rk = 0;
  for (int i = 0; i < a.nseg; ++i)
    for (int j = 0; j < a.seg[i].lora.n_ad; ++j) max_rk = std::max(max_rk, a.seg[i].lora.rank[j]);
  // lane groups for ranks above 32 (rank 32 measured no faster with them)
  f.expand_lanes = 1;
  if (max_rk > 32)
    while (f.expand_lanes < 16 && 16 * f.expand_lanes < max_rk) f.expand_lanes *= 2;
  const bool xl = f.expand_lanes > 1;
  const int per_cu = xl ? b1_resident_per_cu<QT, W, CPW, G, true>() : b1_resident_per_cu<QT, W, CPW, G, false>();
  f.shrink_wgs = 0;
  f.shrink_in_gemv = S::kShrinkInGemv && per_cu > 1 ? 1 : 0;
  if (!f.shrink_in_gemv) f.shrink_wgs = (f.rows_total + S::kRS - 1) / S::kRS;
  const int resident = per_cu * device_cus();
  const int rows_in = f.rows_per_wg;
  // sparse workgroups: their share of the round is twice their share of the
  // launch's bytes (a gathering workgroup moves about half the bytes per unit
  // time of a streaming one; measured on the 10 %-dense 7B block), at least one,
  // at most one per W items
  f.sparse_wgs = 0;
  if (f.sp_items > 0) {
    double dense = 0.0;
    for (int i = 0; i < a.nseg; ++i)
      dense += (double)a.seg[i].n * (double)(Fmt<QT>::row_bytes(a.k) + (QT == QBL_FMT_Q8 ? a.k / 16 : QT == QBL_FMT_Q4 ? a.k / 8 : a.k / 16));
    const double share = std::min(0.9, 2.0 * (double)f.sp_bytes / ((double)f.sp_bytes + dense));
    int sw = (int)(share * (double)(resident - f.shrink_wgs) + 0.5);
    sw = std::min(std::max(sw, 1), (f.sp_items + W - 1) / W);
    f.sparse_wgs = sw;
  }
  auto pick_rows = [&] {
    f.rows_per_wg = rows_in;
    if (f.rows_per_wg > 0) return;
    // one round: as many GEMV workgroups as the chip holds next to the shrink and sparse ones
    const int units = f.sum ? a.seg[0].n : [&] { int u = 0; for (int i = 0; i < a.nseg; ++i) u += a.seg[i].n; return u; }();
    const int slots = resident - f.shrink_wgs - f.sparse_wgs;
    const int rmax = kB1MaxSlots / (f.sum ? a.nseg : 1);
    int r = slots > 0 ? (units + slots - 1) / slots : rmax;
    f.rows_per_wg = r < 1 ? 1 : (r > rmax ? rmax : r);
  };
  auto gemv_wgs = [&] {
    int wg = 0;
    if (f.sum) {
      wg = (a.seg[0].n + f.rows_per_wg - 1) / f.rows_per_wg;
    } else {
      for (int i = 0; i < a.nseg; ++i) {
        a.seg[i].wg_begin = wg;
        wg += (a.seg[i].n + f.rows_per_wg - 1) / f.rows_per_wg;
      }
    }
    return wg;
  };
  pick_rows();
  int wg = gemv_wgs();
  if (f.shrink_in_gemv && wg < f.rows_total) {
    f.shrink_in_gemv = 0;
    f.shrink_wgs = (f.rows_total + S::kRS - 1) / S::kRS;
    pick_rows();
    wg = gemv_wgs();
  }
  a.grid = f.shrink_wgs + f.sparse_wgs + wg;
  const int flags = b1_flags(f.sum, a.nseg, f.shrink_in_gemv, f.shrink_wgs);
  if (xl)
    QBL_LAUNCH((gemv_b1_kernel<QT, W, CPW, G, true>), dim3(a.grid), dim3(W * 64), 0, lc, a.seg[0].qs, a.seg[0].sc,
               f.v[0], a.k, f.shrink_wgs + f.sparse_wgs, f.rows_per_wg, a.seg[0].n, flags, f.rows_total, f);
  else
    QBL_LAUNCH((gemv_b1_kernel<QT, W, CPW, G, false>), dim3(a.grid), dim3(W * 64), 0, lc, a.seg[0].qs, a.seg[0].sc,
               f.v[0], a.k, f.shrink_wgs + f.sparse_wgs, f.rows_per_wg, a.seg[0].n, flags, f.rows_total, f);
  return hipGetLastError();
}

// The workgroup shapes (W waves, CPW chunks per lane) of the batch-1 kernel.
// Up to one block of 64 chunks per lane, four waves suffice (K <= 4096 for
// q8_0); longer rows take more waves before more chunks per lane, which keeps
// more rows in flight per register.  Shapes whose registers would spill at
// their wave count are left out (q4 formats hold twice the inputs per chunk).
struct B1ShapeW { int w, cpw; };
constexpr B1ShapeW kB1ShapesQ8[] = {{4, 1},  {6, 1},  {8, 1},  {11, 1}, {12, 1}, {14, 1},
                                    {16, 1}, {12, 2}, {14, 2}, {16, 2}, {16, 3}};
constexpr B1ShapeW kB1ShapesQ4[] = {{4, 1}, {6, 1}, {8, 1}, {11, 1}, {12, 1}, {14, 1}, {16, 1}, {12, 2}};
constexpr int kB1MaxBlocksQ8 = 48, kB1MaxBlocksQ4 = 24;

// For a row of `blocks` blocks of 64 chunks: the shape with the fewest chunk
// slots (lanes past the row end do no useful work), then the fewest chunks per
// lane; -1 if none holds the row.
template <int N>
constexpr int b1_pick(const B1ShapeW (&t)[N], int blocks) {
  int best = -1;
  for (int i = 0; i < N; ++i) {
    if (t[i].w * t[i].cpw < blocks) continue;
    if (best < 0 || t[i].w * t[i].cpw < t[best].w * t[best].cpw) best = i;
  }
  return best;
}

template <int QT, int I>
hipError_t launch_b1_shape(FusedArgs& f, const LaunchCtx& lc) {
  constexpr B1ShapeW sh = QT == QBL_FMT_Q8 ? kB1ShapesQ8[I] : kB1ShapesQ4[I];
  return launch_b1_t<QT, sh.w, sh.cpw>(f, lc);
}

template <int QT, int... I>
hipError_t launch_b1_index(FusedArgs& f, const LaunchCtx& lc, int i, std::integer_sequence<int, I...>) {
  hipError_t e = hipErrorInvalidValue;
  ((i == I ? (e = launch_b1_shape<QT, I>(f, lc), true) : false) || ...);
  return e;
}

template <int QT>
hipError_t launch_b1_q(FusedArgs& f, const LaunchCtx& lc) {
  const int blocks = (f.g.k / Fmt<QT>::kWeightsPerChunk + 63) / 64;
  if constexpr (QT == QBL_FMT_Q8) {
    constexpr int n = sizeof(kB1ShapesQ8) / sizeof(kB1ShapesQ8[0]);
    return launch_b1_index<QT>(f, lc, b1_pick(kB1ShapesQ8, blocks), std::make_integer_sequence<int, n>{});
  } else {
    constexpr int n = sizeof(kB1ShapesQ4) / sizeof(kB1ShapesQ4[0]);
    return launch_b1_index<QT>(f, lc, b1_pick(kB1ShapesQ4, blocks), std::make_integer_sequence<int, n>{});
  }
}

template <int QT, int BB, int CPL, int RPW>
hipError_t launch_one(GemvArgs& a, const LaunchCtx& lc) {
  using F = Fmt<QT>;
  const size_t lds = sizeof(float) * ((size_t)BB * a.kt + (size_t)BB * (a.kt / F::kWeightsPerChunk) +
                                      (size_t)a.batch * a.t_stride);
  if (lds > kMaxDynLds) return hipErrorInvalidValue;
  hipError_t e = allow_dyn_lds(reinterpret_cast<const void*>(&gemv_kernel<QT, BB, CPL, RPW>), lds);
  if (e != hipSuccess) return e;
  int wg = 0;
  for (int i = 0; i < a.nseg; ++i) {
    a.seg[i].wg_begin = wg;
    wg += (a.seg[i].n + kWaves * RPW - 1) / (kWaves * RPW);
  }
  a.grid = wg;
  a.rpw = RPW;
  QBL_LAUNCH((gemv_kernel<QT, BB, CPL, RPW>), dim3(a.grid), dim3(kThreads), lds, lc, a);
  return hipGetLastError();
}

// rows per wave: enough weight loads in flight per wave without exhausting VGPRs
template <int QT, int BB, int CPL>
hipError_t launch_rpw(GemvArgs& a, const LaunchCtx& lc) {
  if constexpr (BB == 1 && CPL <= 8) return launch_one<QT, BB, CPL, 2>(a, lc);
  else return launch_one<QT, BB, CPL, 1>(a, lc);
}

// chunks per lane: only the variants the LDS tile of this batch bucket can need
template <int QT, int BB>
hipError_t launch_cpl(GemvArgs& a, int cpl, const LaunchCtx& lc) {
  constexpr int kMax = (kLdsFloats / BB) / Fmt<QT>::kWeightsPerChunk / 64;
  if (cpl <= 1) return launch_rpw<QT, BB, 1>(a, lc);
  if constexpr (kMax >= 2) if (cpl <= 2) return launch_rpw<QT, BB, 2>(a, lc);
  if constexpr (kMax >= 4) if (cpl <= 4) return launch_rpw<QT, BB, 4>(a, lc);
  if constexpr (kMax >= 8) if (cpl <= 8) return launch_rpw<QT, BB, 8>(a, lc);
  if constexpr (kMax >= 12) if (cpl <= 12) return launch_rpw<QT, BB, 12>(a, lc);
  if constexpr (kMax >= 16) if (cpl <= 16) return launch_rpw<QT, BB, 16>(a, lc);
  return hipErrorInvalidValue;
}

template <int QT>
hipError_t launch_batch(GemvArgs& a, int bb, int cpl, const LaunchCtx& lc) {
  switch (bb) {
    case 1: return launch_cpl<QT, 1>(a, cpl, lc);
    case 2: return launch_cpl<QT, 2>(a, cpl, lc);
    case 4: return launch_cpl<QT, 4>(a, cpl, lc);
    default: return launch_cpl<QT, 8>(a, cpl, lc);
  }
}

// y = v / sqrt(mean(v^2) + 1e-6) for one vector (n a multiple of 4): a single
// workgroup of 1024 threads; up to 16384 values stay in registers between the
// sum of squares and the scaled write (larger vectors are read twice).  The sum
// is formed per thread, then per wave (DPP), then over the 16 waves in order.
constexpr int kRmsThreads = 1024;
constexpr int kRmsHeld = 4;  // float4 per thread kept in registers

__global__ __launch_bounds__(kRmsThreads) void rms_kernel(const float* v, int n, float* y) {
  __shared__ float red[kRmsThreads / 64];
  const int tid = threadIdx.x, n4 = n / 4;
  float4 r[kRmsHeld];
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < kRmsHeld; ++i) {
    const int f = tid + kRmsThreads * i;
    r[i] = f < n4 ? gload4(v + 4 * (int64_t)f) : make_float4(0.f, 0.f, 0.f, 0.f);
    ss = fmaf(r[i].x, r[i].x, fmaf(r[i].y, r[i].y, fmaf(r[i].z, r[i].z, fmaf(r[i].w, r[i].w, ss))));
  }
  for (int f = tid + kRmsThreads * kRmsHeld; f < n4; f += kRmsThreads) {
    const float4 t = gload4(v + 4 * (int64_t)f);
    ss = fmaf(t.x, t.x, fmaf(t.y, t.y, fmaf(t.z, t.z, fmaf(t.w, t.w, ss))));
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int i = 0; i < kRmsThreads / 64; ++i) tot += red[i];
  const float c = 1.0f / sqrtf(tot / (float)n + 1e-6f);
#pragma unroll
  for (int i = 0; i < kRmsHeld; ++i) {
    const int f = tid + kRmsThreads * i;
    if (f < n4) *reinterpret_cast<float4*>(y + 4 * (int64_t)f) = mul4(c, r[i]);
  }
  for (int f = tid + kRmsThreads * kRmsHeld; f < n4; f += kRmsThreads)
    *reinterpret_cast<float4*>(y + 4 * (int64_t)f) = mul4(c, gload4(v + 4 * (int64_t)f));
}

template <bool LDS>
hipError_t launch_prep_t(const PrepArgs& a, int grid, size_t lds, const LaunchCtx& lc) {
  if (LDS) {
    hipError_t e = allow_dyn_lds(reinterpret_cast<const void*>(&prep_kernel<LDS>), lds);
    if (e != hipSuccess) return e;
  }
  QBL_LAUNCH((prep_kernel<LDS>), dim3(grid), dim3(kThreads), LDS ? lds : 0, lc, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prep(const PrepArgs& a, const LaunchCtx& lc) {
  (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
  if (a.k % 4) return hipErrorInvalidValue;
  int grid = a.rows_total;
  if (a.xin) grid = max(grid, (a.k + 2047) / 2048);
  if (grid < 1) grid = 1;
  const int64_t floats = (int64_t)a.batch * a.k;
  if (floats <= kPrepLdsFloats) return launch_prep_t<true>(a, grid, sizeof(float) * floats, lc);
  return launch_prep_t<false>(a, grid, 0, lc);
}

hipError_t launch_rms(const float* v, int n, float* y, const LaunchCtx& lc) {
  (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
  if (n < 4 || n % 4) return hipErrorInvalidValue;
  QBL_LAUNCH(rms_kernel, dim3(1), dim3(kRmsThreads), 0, lc, v, n, y);
  return hipGetLastError();
}

bool fused_supported(int qtype, int k) {
  const int wpc = qtype == QBL_FMT_Q8 ? 16 : 32;
  const int max_blocks = qtype == QBL_FMT_Q8 ? kB1MaxBlocksQ8 : kB1MaxBlocksQ4;
  return k % (qtype == QBL_FMT_Q4K ? 256 : 32) == 0 && (k / wpc + 63) / 64 <= max_blocks;
}

hipError_t launch_fused(FusedArgs& f, const LaunchCtx& lc) {
  (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
  GemvArgs& a = f.g;
  if (a.batch != 1 || f.nv != 1 || !fused_supported(a.qtype, a.k) || f.rows_total > kB1MaxT) return hipErrorInvalidValue;
  // the flags word (b1_flags) holds the shrink workgroup count in 24 bits
  if (f.rows_total > (1 << 23)) return hipErrorInvalidValue;
  for (int i = 0; i < a.nseg; ++i)
    if (f.sum && a.seg[i].n != a.seg[0].n) return hipErrorInvalidValue;
  // sparse items: every (segment, sparse adapter) has its n rows at sp_base, all below sp_items
  for (int i = 0; i < a.nseg; ++i)
    for (int j = 0; j < a.seg[i].lora.n_ad; ++j) {
      const bool sparse = a.seg[i].lora.rank[j] == 0;
      const int b = f.sp_base[i][j];
      if (sparse != (b >= 0) || (sparse && (b + a.seg[i].n > f.sp_items || !f.sp))) return hipErrorInvalidValue;
    }
  f.rows_per_wg = 0;  // chosen by the launcher from the kernel's occupancy
  switch (a.qtype) {
    case QBL_FMT_Q8: return launch_b1_q<QBL_FMT_Q8>(f, lc);
    case QBL_FMT_Q4: return launch_b1_q<QBL_FMT_Q4>(f, lc);
    case QBL_FMT_Q4K: return launch_b1_q<QBL_FMT_Q4K>(f, lc);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv(GemvArgs& a, const LaunchCtx& lc) {
  (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
  const int bb = a.batch <= 1 ? 1 : a.batch <= 2 ? 2 : a.batch <= 4 ? 4 : 8;
  const int wpc = a.qtype == QBL_FMT_Q8 ? 16 : 32;
  // x tile: whole input when it fits the LDS budget, else multiples of 64 chunks
  const int quant = 64 * wpc;
  int kt = a.k;
  if ((int64_t)bb * kt > kLdsFloats) kt = max(quant, (kLdsFloats / bb) / quant * quant);
  a.kt = kt;
  const int cpl = (kt / wpc + 63) / 64;
  for (int i = 0; i < a.nseg; ++i) {
    LoraSeg& L = a.seg[i].lora;
    L.prefetch = L.n_ad <= kPrefetchAdapters;
    for (int j = 0; j < L.n_ad; ++j)
      if (L.rank[j] > 64 || L.rank[j] == 0) L.prefetch = 0;
  }
  switch (a.qtype) {
    case QBL_FMT_Q8: return launch_batch<QBL_FMT_Q8>(a, bb, cpl, lc);
    case QBL_FMT_Q4: return launch_batch<QBL_FMT_Q4>(a, bb, cpl, lc);
    case QBL_FMT_Q4K: return launch_batch<QBL_FMT_Q4K>(a, bb, cpl, lc);
  }
  return hipErrorInvalidValue;
}

}  // namespace qbl
