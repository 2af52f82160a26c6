// Device helpers shared by the decode-path kernels (gfx950, wave64).
// Internal to the library.
#pragma once
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "qbl_kernels.h"

namespace qbl {
namespace {

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// The value of lane (i of the quad) in every lane of each 4-lane quad:
// quad_perm [i,i,i,i] (0x00, 0x55, 0xAA, 0xFF).  All four lanes of a quad must be
// active.
template <int CTRL>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
  // bound_ctrl: no lane keeps an old value (every source lane is in its quad),
  // so no register needs clearing before the move
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
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

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Device pointers as global-address-space pointers.  A pointer the compiler
// cannot trace to a kernel argument (read from memory, e.g. a descriptor in
// LDS) is otherwise accessed with flat instructions, whose completion counts
// against both the vector-memory and the LDS counters: every LDS wait would then
// also wait for the weight loads in flight.
template <class T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* gp(const T* p) {
  return (const __attribute__((address_space(1))) T*)p;
}
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gpw(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16-byte load of 4 floats through a global-address-space pointer
__device__ __forceinline__ float4 gload4(const float* p) {
  const f32x4 v = *gp(reinterpret_cast<const f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

// 16-byte streaming load of weight bytes: read once, not worth keeping in cache.
__device__ __forceinline__ uint4 stream_load16(const uint8_t* p) {
  const u32x4 v = __builtin_nontemporal_load(gp(reinterpret_cast<const u32x4*>(p)));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ __forceinline__ float4 mul4(float c, float4 a) {
  return make_float4(c * a.x, c * a.y, c * a.z, c * a.w);
}

// ---------------------------------------------------------------------------
// 16-byte weight chunks: a q8_0 chunk is 16 weights (half a block), a q4_sm
// chunk is one whole 32-weight block, a q4_K chunk one 32-weight sub-block.
// In LDS the 16-byte slots of a chunk's input are rotated per chunk so that the
// lanes served together by an LDS read touch different bank groups.
//
// Scale data per chunk (Sc): q8_0 the block's fp16 d, q4_sm the block's
// (d | m << 16); q4_K dword (c & 3) of the chunk's 16-byte super-block header:
// the 4 lanes of a quad (consecutive chunks of one super-block) hold the whole
// header between them, and DPP quad broadcasts give every lane all of it.
// ---------------------------------------------------------------------------
template <int QT>
struct Fmt {
  static constexpr int kWeightsPerChunk = QT == QBL_FMT_Q8 ? 16 : 32;
  static constexpr int kSlots = kWeightsPerChunk / 4;
  using Sc = uint32_t;
  __device__ static __forceinline__ int slot(int c, int j) {
    return (j + (QT == QBL_FMT_Q8 ? (c >> 1) : c)) & (kSlots - 1);
  }
  static constexpr int64_t row_bytes(int k) { return QT == QBL_FMT_Q8 ? (int64_t)k : (int64_t)k / 2; }
  // scale data of chunk c (global chunk index along k) of a row
  __device__ static __forceinline__ Sc load_sc(const void* sc, int row, int k, int c) {
    if constexpr (QT == QBL_FMT_Q8)
      return *gp(reinterpret_cast<const uint16_t*>(sc) + (int64_t)row * (k / 32) + (c >> 1));
    else if constexpr (QT == QBL_FMT_Q4)
      return *gp(reinterpret_cast<const uint32_t*>(sc) + (int64_t)row * (k / 32) + c);
    else  // dword (c & 3) of the super-block header; the quad's 4 lanes hold all four
      return *gp(reinterpret_cast<const uint32_t*>(sc) + ((int64_t)row * (k / 256) + (c >> 3)) * 4 + (c & 3));
  }
};

// Step D and offset M of sub-block j of a q4_K super-block header h (w = D*q - M):
// h.x = d | dmin << 16; h.y, h.z, h.w = the 96-bit code field, scale code j at
// field bits 6j.., min code j at field bits 48 + 6j...  D and M are exact in float32.
__device__ __forceinline__ void q4k_step_offset(const uint4 h, int j, float& D, float& M) {
  const uint64_t lo = (uint64_t)h.y | ((uint64_t)h.z << 32);  // field bits 0..63
  const uint64_t hi = (uint64_t)h.z | ((uint64_t)h.w << 32);  // field bits 32..95
  const uint32_t sc = (uint32_t)(lo >> (6 * j)) & 63u;
  const uint32_t mc = (uint32_t)(hi >> (16 + 6 * j)) & 63u;
  D = h2f(h.x) * (float)sc;
  M = h2f(h.x >> 16) * (float)mc;
}

// Sum_j q_j x_j over one q8_0 chunk of 16 weights.  The device stores q8_0
// bytes offset-binary (u = q + 128), which convert with v_cvt_f32_ubyte; the
// offset is removed with the chunk's x sum: sum (u-128) x = sum u x - 128 sum x.
__device__ __forceinline__ float dot_q8(const uint4 q, const float4* xv, float xsum) {
  const uint32_t u[4] = {q.x, q.y, q.z, q.w};
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
// q_{2i+1} (high nibble), so 32-bit word w covers weights 8w .. 8w+7.  The low
// and the high nibbles of a word are spread into the bytes of one word each and
// converted two at a time by the gfx950 fp8 (e4m3) conversion: a byte c < 16 is
// the e4m3 value c 2^-9, so scale 2^9 gives the exact f16 integer c.  Each
// product is one v_fma_mix_f32 (f16 code times float32 input, float32 fma), so
// the sums are bitwise those of fmaf(float(c), x, s) in the same order.
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot_q4(const uint4 q, const float4* xv) {
  constexpr float kFp8Scale = 512.0f;  // 2^9
  const uint32_t v[4] = {q.x, q.y, q.z, q.w};
  float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = v[w] & 0x0F0F0F0Fu, hi = (v[w] >> 4) & 0x0F0F0F0Fu;
    const f16x2v l01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, kFp8Scale, false);
    const f16x2v l23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, kFp8Scale, true);
    const f16x2v h01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, kFp8Scale, false);
    const f16x2v h23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, kFp8Scale, true);
    const float4 xa = xv[2 * w], xb = xv[2 * w + 1];
    s0 = fmaf((float)l01[0], xa.x, s0);
    s1 = fmaf((float)h01[0], xa.y, s1);
    s0 = fmaf((float)l01[1], xa.z, s0);
    s1 = fmaf((float)h01[1], xa.w, s1);
    s0 = fmaf((float)l23[0], xb.x, s0);
    s1 = fmaf((float)h23[0], xb.y, s1);
    s0 = fmaf((float)l23[1], xb.z, s0);
    s1 = fmaf((float)h23[1], xb.w, s1);
  }
  return s0 + s1;
}

// p + (the chunk's dequantised weights . x) for chunk c (global index along k)
// with weights q, inputs xv, input sum xsum and scale data sc:
//   q8_0  p + d * (sum q x)                    (offset-binary bytes, see dot_q8)
//   q4_sm p + d * (sum q x) + m * (sum x)
//   q4_K  p + D * (sum q x) - M * (sum x)      (D, M of the chunk's sub-block)
template <int QT>
__device__ __forceinline__ float chunk_dot(float p, const uint4 q, const float4* xv, float xsum,
                                           const typename Fmt<QT>::Sc sc, int c) {
  if constexpr (QT == QBL_FMT_Q8) {
    return fmaf(h2f(sc), dot_q8(q, xv, xsum), p);
  } else if constexpr (QT == QBL_FMT_Q4) {
    p = fmaf(h2f(sc), dot_q4(q, xv), p);
    return fmaf(h2f(sc >> 16), xsum, p);
  } else {
    const uint4 h = make_uint4(quad_bcast<0x00>(sc), quad_bcast<0x55>(sc), quad_bcast<0xAA>(sc),
                               quad_bcast<0xFF>(sc));
    float D, M;
    q4k_step_offset(h, c & 7, D, M);
    p = fmaf(D, dot_q4(q, xv), p);
    return fmaf(-M, xsum, p);
  }
}

// Sum over entries [e0, e1) of one CSR row of fp16 val[e] * x(col[e]), this
// lane's share: entries e0 + lane, e0 + lane + 64, ...  Loads go out in rounds
// of 8 per lane (the column and value loads of a round first, then its 8
// gathers), so a row of up to 512 entries waits for two memory round trips.
// Entries past e1 read entry e0 with value 0.  xat(c) returns the input at
// column c.
template <class XAt>
__device__ __forceinline__ float csr_row_dot(const uint32_t* col, const uint16_t* val, uint32_t e0,
                                             uint32_t e1, int lane, XAt xat) {
  float p = 0.0f;
  for (uint32_t r0 = e0; r0 < e1; r0 += 8 * 64) {
    uint32_t c[8];
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t e = r0 + 64 * u + lane;
      const bool ok = e < e1;
      c[u] = *gp(col + (ok ? e : e0));
      v[u] = ok ? (uint32_t)*gp(val + e) : 0u;
    }
    float xv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) xv[u] = xat(c[u]);
#pragma unroll
    for (int u = 0; u < 8; ++u) p = fmaf(h2f(v[u]), xv[u], p);
  }
  return p;
}

// csr_row_dot for R rows at once, U loads per row and lane per round: the
// rounds' loads of all R rows go out together.  Each lane still visits its
// entries of a row in the same order (e0 + lane, e0 + lane + 64, ...), so every
// p[r] has the bits csr_row_dot gives; entries past a row's end are not loaded
// and add 0 * x(0).
template <int R, int U, class XAt>
__device__ __forceinline__ void csr_rows_dot(const uint32_t* const (&col)[R], const uint16_t* const (&val)[R],
                                             const uint32_t (&e0)[R], const uint32_t (&e1)[R], int lane, XAt xat,
                                             float (&p)[R]) {
  uint32_t len = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    p[r] = 0.0f;
    len = max(len, e1[r] - e0[r]);
  }
  for (uint32_t off = 0; off < len; off += 64 * U) {
    uint32_t c[R][U], v[R][U];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t e = e0[r] + off + 64 * u + lane;
        const bool ok = e < e1[r];
        c[r][u] = ok ? *gp(col[r] + e) : 0u;
        v[r][u] = ok ? (uint32_t)*gp(val[r] + e) : 0u;
      }
    float xv[R][U];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int u = 0; u < U; ++u) xv[r][u] = xat(c[r][u]);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int u = 0; u < U; ++u) p[r] = fmaf(h2f(v[r][u]), xv[r][u], p[r]);
  }
}

// Waits for values handed from one workgroup to others in the same launch.
// All waits of one thread share one deadline on the 100 MHz wall clock, set at
// its first wait that finds a stale word; past it the thread records the
// failure in the host-visible status word (one vector store to coherent host
// memory) and takes every later word as it finds it, without waiting.  So a
// broken hand-off costs a launch at most one budget, and the caller learns of
// it from the library (a run call or the status call) instead of from its
// numbers.
struct HandoffWait {
  uint32_t* fail;      // status word, device address of coherent host memory
  int64_t budget;      // wall-clock ticks one thread may spend waiting
  int64_t deadline;
  bool gave_up;
  __device__ HandoffWait(uint32_t* f, int64_t b) : fail(f), budget(b), deadline(-1), gave_up(false) {}
};

// One value handed over: a 64-bit word, the launch's (or phase's) tag in the
// high half and the float in the low half, read with device-coherent relaxed
// loads until the tag matches (bounded as above).
__device__ __forceinline__ float tagged_get(const uint64_t* p, uint32_t tag, HandoffWait& hw) {
  uint64_t w = __hip_atomic_load(gp(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((uint32_t)(w >> 32) == tag || hw.gave_up) return __uint_as_float((uint32_t)w);
  if (hw.deadline < 0) hw.deadline = wall_clock64() + hw.budget;
  for (;;) {
    __builtin_amdgcn_s_sleep(1);
    w = __hip_atomic_load(gp(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(w >> 32) == tag) break;
    if (wall_clock64() > hw.deadline) {
      hw.gave_up = true;
      __hip_atomic_store(hw.fail, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      break;
    }
  }
  return __uint_as_float((uint32_t)w);
}

// One DPP exchange-and-add step of the transposed row reduction: lanes whose
// bit (the partner distance) is clear keep the first half of the values, the
// others the second half; each adds its partner's copy of the half it keeps.
template <int CTRL, int N>
__device__ __forceinline__ void fold_half(float (&p)[8], bool upper) {
#pragma unroll
  for (int k = 0; k < N / 2; ++k) {
    const float send = upper ? p[k] : p[k + N / 2];
    const float keep = upper ? p[k + N / 2] : p[k];
    p[k] = keep + dpp_mov<CTRL>(send);
  }
}

// Reduces G per-lane partials (one per row) over each 16-lane row of the wave.
// Afterwards lane i of a 16-lane row holds the partial of row (i >> (4 - log2 G))
// in p[0]: lanes 0, 16/G, 2*16/G, ... hold rows 0, 1, 2, ...
template <int G>
__device__ __forceinline__ void reduce_rows16(float (&p)[8], int lane) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "G");
  const bool b3 = lane & 8, b2 = lane & 4, b1 = lane & 2;
  if constexpr (G == 8) {
    fold_half<0x140, 8>(p, b3);  // row_mirror: partner 15 - i
    fold_half<0x141, 4>(p, b2);  // row_half_mirror: partner 7 - i
    fold_half<0x4E, 2>(p, b1);   // quad_perm [2,3,0,1]: partner i ^ 2
    p[0] += dpp_mov<0xB1>(p[0]);  // quad_perm [1,0,3,2]
  } else if constexpr (G == 4) {
    fold_half<0x140, 4>(p, b3);
    fold_half<0x141, 2>(p, b2);
    p[0] += dpp_mov<0x4E>(p[0]);
    p[0] += dpp_mov<0xB1>(p[0]);
  } else if constexpr (G == 2) {
    fold_half<0x140, 2>(p, b3);
    p[0] += dpp_mov<0x141>(p[0]);
    p[0] += dpp_mov<0x4E>(p[0]);
    p[0] += dpp_mov<0xB1>(p[0]);
  } else {
    p[0] += dpp_mov<0x140>(p[0]);
    p[0] += dpp_mov<0x141>(p[0]);
    p[0] += dpp_mov<0x4E>(p[0]);
    p[0] += dpp_mov<0xB1>(p[0]);
  }
}

}  // namespace
}  // namespace qbl
