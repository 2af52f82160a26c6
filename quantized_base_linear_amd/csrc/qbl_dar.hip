// Dequantize-add-requantize (DAR), for measuring the drift of the destructive
// merge that the overlay never performs ("We propose a content-addressed
// overlay system", "Quantized-Base Numerical Analysis"; "Deep Technical
// Design", "The Pathology of Dequantize-Add-Requantize (DAR) Error").
//
// One thread per 32-weight chunk (a q8_0 or q4_sm block, a q4_K sub-block).
// A wave covers 64 rows at one chunk (q4_K: 8 rows at the 8 chunks of one
// super-block, whose sub-blocks are then 8 consecutive lanes), so the A values
// of its chunks are shared by the whole wave: they are staged in the wave's LDS
// region kRB rank rows at a time, together with the kRB B values of the wave's
// rows (loaded four lanes to a row, then read back per lane), so that one
// memory round trip serves kRB steps of every lane's fma chain.  A thread
// forms the merged float32 weights of its chunk with one fixed recipe
//   w = f32(deq(W));  per adapter in list order:
//     low-rank  w = fma(s, u, w),  u = fma chain over j of B[r][j] * A[j][k]
//     sparse    w = fma(s, f32(v), w) at the row's entries in the chunk
// then applies the base format's quantiser (IEEE-rounded float32 divisions,
// round-half-away, fp16 round-to-nearest-even) and writes the canonical block
// bytes.  The base is only read.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "qbl_device.h"
#include "qbl_kernels.h"

namespace qbl {
namespace {

constexpr int kDarThreads = 256;
constexpr int kRB = 8;  // rank rows of A staged per round

__device__ __forceinline__ uint16_t f2h_bits(float f) { return __half_as_ushort(__float2half_rn(f)); }
__device__ __forceinline__ float h_bits2f(uint16_t b) { return __half2float(__ushort_as_half(b)); }
// std::min / std::max with the host quantiser's operand order
__device__ __forceinline__ float mn(float a, float b) { return b < a ? b : a; }
__device__ __forceinline__ float mx(float a, float b) { return a < b ? b : a; }

template <int QT>
__global__ __launch_bounds__(kDarThreads, 4) void dar_kernel(DarArgs a) {
#pragma clang fp contract(off)  // the codes depend on each rounding: only the fmas written out fuse
  constexpr int RW = QT == QBL_FMT_Q4K ? 8 : 64;  // rows per wave
  constexpr int CW = 64 / RW;                      // chunks per wave
  __shared__ f32x4 a_st[kDarThreads / 64][kRB][CW * 8];  // per wave: kRB rank rows of A at its chunks
  __shared__ f32x4 b_st[kDarThreads / 64][RW][kRB / 4 + 1];  // per wave: its rows' kRB B values (+ pad)
  const int cpr = a.k / 32;                        // chunks per row
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t wv = ((int64_t)blockIdx.x * kDarThreads + threadIdx.x) >> 6;
  const int64_t n_rw = (a.n + RW - 1) / RW;        // row groups
  const int rgrp = (int)(wv % n_rw), cgrp = (int)(wv / n_rw);
  if (cgrp * CW >= cpr) return;                    // whole waves past the end
  // lanes on rows past n work on the last row and store nothing (q4_K: whole
  // 8-lane groups, so the group exchanges below stay within valid data)
  const bool valid = rgrp * RW + lane / CW < a.n;
  const int row = min(rgrp * RW + lane / CW, a.n - 1), c = cgrp * CW + lane % CW;
  const int64_t t = (int64_t)row * cpr + c;        // the chunk's index in canonical order
  const int k0 = 32 * c;

  // ---- exact float32 dequantisation of the chunk
  float w[32];
  if constexpr (QT == QBL_FMT_Q8) {
    const float d = h_bits2f(reinterpret_cast<const uint16_t*>(a.sc)[(int64_t)row * cpr + c]);
    const uint8_t* q = a.qs + (int64_t)row * a.k + k0;
#pragma unroll
    for (int i = 0; i < 32; ++i) w[i] = d * (float)((int)q[i] - 128);
  } else {
    const uint8_t* q = a.qs + (int64_t)row * (a.k / 2) + 16 * c;
    float D, M;
    if constexpr (QT == QBL_FMT_Q4) {
      const uint32_t dm = reinterpret_cast<const uint32_t*>(a.sc)[(int64_t)row * cpr + c];
      D = h_bits2f((uint16_t)dm);
      M = -h_bits2f((uint16_t)(dm >> 16));
    } else {
      const uint32_t* h = reinterpret_cast<const uint32_t*>(a.sc) + ((int64_t)row * (a.k / 256) + (c >> 3)) * 4;
      q4k_step_offset(make_uint4(h[0], h[1], h[2], h[3]), c & 7, D, M);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      w[2 * i] = fmaf(D, (float)(q[i] & 0x0F), -M);
      w[2 * i + 1] = fmaf(D, (float)(q[i] >> 4), -M);
    }
  }

  // ---- the adapters' terms, in list order
  for (int i = 0; i < a.n_ad; ++i) {
    const float s = a.scale[i];
    if (a.rank[i] == 0) {
      // first entry of the row at or after k0 (columns strictly increase), then a merge walk
      uint32_t lo = a.rp[i][row], hi = a.rp[i][row + 1];
      while (lo < hi) {
        const uint32_t mid = lo + (hi - lo) / 2;
        if (a.ci[i][mid] < (uint32_t)k0) lo = mid + 1;
        else hi = mid;
      }
      const uint32_t end = a.rp[i][row + 1];
#pragma unroll
      for (int j = 0; j < 32; ++j)
        if (lo < end && a.ci[i][lo] == (uint32_t)(k0 + j)) {
          w[j] = fmaf(s, h_bits2f(a.sv[i][lo]), w[j]);
          ++lo;
        }
      continue;
    }
    const int rk = a.rank[i];
    const float* Br = a.B[i] + (int64_t)row * rk;
    const f32x4* Ab = reinterpret_cast<const f32x4*>(a.A[i] + 32 * cgrp * CW);  // the wave's first column
    float u[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) u[j] = 0.0f;
    for (int r0 = 0; r0 < rk; r0 += kRB) {
      const int nr = min(kRB, rk - r0);
      // rank rows r0 .. r0 + nr of A at the wave's CW chunks (CW * 8 float4 each)
#pragma unroll
      for (int q0 = 0; q0 < kRB * CW * 8; q0 += 64) {
        const int q = q0 + lane, rr = q / (CW * 8), f = q % (CW * 8);
        if (rr < nr) a_st[wave][rr][f] = *gp(Ab + (int64_t)(r0 + rr) * (a.k / 4) + f);
      }
      // the wave's RW rows x nr B values: 4 lanes per row with 16-byte loads when
      // the rows allow it (each lane then reads its row back), else per lane
      float b[kRB];
      const bool coalesced = rk % 4 == 0;
      if (coalesced) {
#pragma unroll
        for (int q0 = 0; q0 < RW * kRB / 4; q0 += 64) {
          const int q = q0 + lane, ro = q / (kRB / 4), part = q % (kRB / 4);
          const int grow = min(rgrp * RW + ro, a.n - 1);
          if (q < RW * kRB / 4 && 4 * part < nr)
            b_st[wave][ro][part] = *gp(reinterpret_cast<const f32x4*>(a.B[i] + (int64_t)grow * rk + r0) + part);
        }
      } else {
#pragma unroll
        for (int rr = 0; rr < kRB; ++rr) b[rr] = rr < nr ? *gp(Br + r0 + rr) : 0.0f;
      }
      // a wave's LDS writes and reads run in issue order; this keeps the
      // compiler from moving the reads above the writes
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (coalesced) {
#pragma unroll
        for (int p4 = 0; p4 < kRB / 4; ++p4) {
          const f32x4 v = b_st[wave][lane / CW][p4];
          b[4 * p4] = v.x, b[4 * p4 + 1] = v.y, b[4 * p4 + 2] = v.z, b[4 * p4 + 3] = v.w;
        }
      }
#pragma unroll
      for (int rr = 0; rr < kRB; ++rr) {
        if (rr >= nr) break;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const f32x4 a4 = a_st[wave][rr][(lane % CW) * 8 + j];
          u[4 * j] = fmaf(b[rr], a4.x, u[4 * j]);
          u[4 * j + 1] = fmaf(b[rr], a4.y, u[4 * j + 1]);
          u[4 * j + 2] = fmaf(b[rr], a4.z, u[4 * j + 2]);
          u[4 * j + 3] = fmaf(b[rr], a4.w, u[4 * j + 3]);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) w[j] = fmaf(s, u[j], w[j]);
  }

  // ---- the base format's quantiser, canonical bytes
  if constexpr (QT == QBL_FMT_Q8) {
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = mx(amax, fabsf(w[j]));
    const uint16_t dh = f2h_bits(__fdiv_rn(amax, 127.0f));
    const float d = h_bits2f(dh);
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out + t * 34);
    if (!valid) return;
    out[0] = dh;
#pragma unroll
    for (int j = 0; j < 32; j += 2) {
      uint32_t pair = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float q = d != 0.0f ? roundf(__fdiv_rn(w[j + h], d)) : 0.0f;
        q = fminf(127.0f, fmaxf(-127.0f, q));
        pair |= ((uint32_t)(uint8_t)(int8_t)(int)q) << (8 * h);
      }
      out[1 + j / 2] = (uint16_t)pair;
    }
  } else if constexpr (QT == QBL_FMT_Q4) {
    float lo = w[0], hi = w[0];
#pragma unroll
    for (int j = 1; j < 32; ++j) {
      lo = mn(lo, w[j]);
      hi = mx(hi, w[j]);
    }
    const uint16_t mh = f2h_bits(lo);
    const float m = h_bits2f(mh);
    const uint16_t dh = f2h_bits(__fdiv_rn(hi - m, 15.0f));
    const float d = h_bits2f(dh);
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out + t * 20);
    if (!valid) return;
    out[0] = dh;
    out[1] = mh;
#pragma unroll
    for (int j = 0; j < 32; j += 4) {
      uint32_t nib = 0;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        float q = d != 0.0f ? roundf(__fdiv_rn(w[j + h] - m, d)) : 0.0f;
        q = fminf(15.0f, fmaxf(0.0f, q));
        nib |= (uint32_t)(int)q << (4 * h);
      }
      out[2 + j / 4] = (uint16_t)nib;
    }
  } else {
    // sub-block span and offset, then the super-block maxima over the 8 lanes
    float lo = 0.0f, hi = w[0];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      lo = mn(lo, w[j]);
      hi = mx(hi, w[j]);
    }
    const float span = __fdiv_rn(hi - lo, 15.0f), off = 0.0f - lo;
    float smax = span, tmax = off;
#pragma unroll
    for (int x = 1; x < 8; x <<= 1) {
      smax = mx(smax, __shfl_xor(smax, x, 8));
      tmax = mx(tmax, __shfl_xor(tmax, x, 8));
    }
    smax = mx(0.0f, smax);
    tmax = mx(0.0f, tmax);
    const uint16_t dh = f2h_bits(__fdiv_rn(smax, 63.0f)), mh = f2h_bits(__fdiv_rn(tmax, 63.0f));
    const float d = h_bits2f(dh), dmin = h_bits2f(mh);
    const float sc = d != 0.0f ? fminf(63.0f, ceilf(__fdiv_rn(span, d))) : 0.0f;
    const float mc = dmin != 0.0f ? fminf(63.0f, roundf(__fdiv_rn(off, dmin))) : 0.0f;
    const float D = d * sc, M = dmin * mc;
    const int j8 = c & 7;
    uint8_t* blk = a.out + (t >> 3) * 144;
    uint16_t* nb = reinterpret_cast<uint16_t*>(blk + 16 + 16 * j8);
#pragma unroll
    for (int j = 0; j < 32; j += 4) {
      uint32_t nib = 0;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        float q = D != 0.0f ? roundf(__fdiv_rn(w[j + h] + M, D)) : 0.0f;
        q = fminf(15.0f, fmaxf(0.0f, q));
        nib |= (uint32_t)(int)q << (4 * h);
      }
      if (valid) nb[j / 4] = (uint16_t)nib;
    }
    // the 16 six-bit codes into lane 0 of the group: code i at field bit 6i
    const uint32_t codes = (uint32_t)sc | ((uint32_t)mc << 8);
    uint64_t f_lo = 0, f_hi = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t cj = __shfl(codes, j, 8);
      const uint64_t s6 = cj & 63u, m6 = (cj >> 8) & 63u;
      const int bs = 6 * j, bm = 48 + 6 * j;
      f_lo |= s6 << bs;                                   // bits 0..47
      if (bm < 64) f_lo |= m6 << bm;
      if (bm + 6 > 64) f_hi |= bm >= 64 ? m6 << (bm - 64) : m6 >> (64 - bm);
    }
    if (valid && j8 == 0) {
      uint16_t* hdr = reinterpret_cast<uint16_t*>(blk);
      hdr[0] = dh;
      hdr[1] = mh;
#pragma unroll
      for (int b = 0; b < 4; ++b) hdr[2 + b] = (uint16_t)(f_lo >> (16 * b));
#pragma unroll
      for (int b = 0; b < 2; ++b) hdr[6 + b] = (uint16_t)(f_hi >> (16 * b));
    }
  }
}

}  // namespace

hipError_t launch_dar(const DarArgs& a, const LaunchCtx& lc) {
  (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
  if (a.k % (a.qtype == QBL_FMT_Q4K ? 256 : 32) || a.n < 1) return hipErrorInvalidValue;
  const int rw = a.qtype == QBL_FMT_Q4K ? 8 : 64;
  const int64_t waves = (int64_t)(a.n + rw - 1) / rw * ((a.k / 32) / (64 / rw));
  const dim3 grid((unsigned)((waves * 64 + kDarThreads - 1) / kDarThreads));
  switch (a.qtype) {
    case QBL_FMT_Q8: QBL_LAUNCH((dar_kernel<QBL_FMT_Q8>), grid, dim3(kDarThreads), 0, lc, a); break;
    case QBL_FMT_Q4: QBL_LAUNCH((dar_kernel<QBL_FMT_Q4>), grid, dim3(kDarThreads), 0, lc, a); break;
    case QBL_FMT_Q4K: QBL_LAUNCH((dar_kernel<QBL_FMT_Q4K>), grid, dim3(kDarThreads), 0, lc, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qbl
