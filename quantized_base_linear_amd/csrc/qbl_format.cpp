// Host side of the block formats: quantisation, dequantisation, the repack
// into the device layout, and SHA-256 for the base-integrity digest.
//
// q8_0 follows "Deep Technical Design: Exact, Atomic, Reversible Specialist
// Overlays", section 5 (a block is 32 weights and one f16 scale); q4_sm is the
// 4-bit scale+minimum block (w = d*q + m) named in the same section.  The
// quantiser rules (scale from the block extreme, rounding half away from zero
// with the stored fp16 scale) are the library's reading of those passages and
// are listed in qbl.h.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

#include "../../include/qbl.h"
#include "qbl_host.h"

namespace qbl {

int default_threads() {
  unsigned n = std::thread::hardware_concurrency();
  if (const char* env = std::getenv("OMP_NUM_THREADS")) {
    const int e = std::atoi(env);
    if (e > 0 && (unsigned)e < n) n = (unsigned)e;
  }
  return n ? (int)n : 1;
}

void parallel_for(int64_t n, int nthreads, const std::function<void(int64_t)>& fn) {
  if (nthreads <= 0) nthreads = default_threads();
  if (n <= 0) return;
  if (nthreads == 1 || n == 1) {
    for (int64_t i = 0; i < n; ++i) fn(i);
    return;
  }
  if ((int64_t)nthreads > n) nthreads = (int)n;
  std::vector<std::thread> th;
  th.reserve(nthreads);
  const int64_t per = (n + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    const int64_t b = per * t, e = std::min(n, b + per);
    if (b >= e) break;
    th.emplace_back([=, &fn] {
      for (int64_t i = b; i < e; ++i) fn(i);
    });
  }
  for (auto& x : th) x.join();
}

namespace {

inline uint16_t to_half_bits(float f) {
  const _Float16 h = (_Float16)f;  // round to nearest even
  uint16_t u;
  std::memcpy(&u, &h, 2);
  return u;
}
inline float from_half_bits(uint16_t u) {
  _Float16 h;
  std::memcpy(&h, &u, 2);
  return (float)h;
}
inline bool half_finite(uint16_t u) { return (u & 0x7C00u) != 0x7C00u; }

// one q8_0 block; returns false if the scale overflows fp16
bool q8_block(const float* w, uint8_t* out) {
  float amax = 0.0f;
  for (int j = 0; j < 32; ++j) amax = std::max(amax, std::fabs(w[j]));
  const uint16_t dh = to_half_bits(amax / 127.0f);
  if (!half_finite(dh)) return false;
  const float d = from_half_bits(dh);
  out[0] = (uint8_t)(dh & 0xFF);
  out[1] = (uint8_t)(dh >> 8);
  for (int j = 0; j < 32; ++j) {
    float q = d != 0.0f ? std::round(w[j] / d) : 0.0f;
    q = std::min(127.0f, std::max(-127.0f, q));
    out[2 + j] = (uint8_t)(int8_t)(int)q;
  }
  return true;
}

bool q4_block(const float* w, uint8_t* out) {
  float lo = w[0], hi = w[0];
  for (int j = 1; j < 32; ++j) {
    lo = std::min(lo, w[j]);
    hi = std::max(hi, w[j]);
  }
  const uint16_t mh = to_half_bits(lo);
  if (!half_finite(mh)) return false;
  const float m = from_half_bits(mh);
  const uint16_t dh = to_half_bits((hi - m) / 15.0f);
  if (!half_finite(dh)) return false;
  const float d = from_half_bits(dh);
  out[0] = (uint8_t)(dh & 0xFF);
  out[1] = (uint8_t)(dh >> 8);
  out[2] = (uint8_t)(mh & 0xFF);
  out[3] = (uint8_t)(mh >> 8);
  uint8_t q[32];
  for (int j = 0; j < 32; ++j) {
    float v = d != 0.0f ? std::round((w[j] - m) / d) : 0.0f;
    v = std::min(15.0f, std::max(0.0f, v));
    q[j] = (uint8_t)(int)v;
  }
  for (int i = 0; i < 16; ++i) out[4 + i] = (uint8_t)(q[2 * i] | (q[2 * i + 1] << 4));
  return true;
}

// One q4_K super-block of 256 weights (include/qbl.h gives the layout): per
// 32-weight sub-block the smallest 6-bit scale code whose step covers the
// sub-block's range down to min(0, min w), the nearest 6-bit code for that
// offset, then 4-bit q.  Returns false if a super-scale overflows fp16.
bool q4k_block(const float* w, uint8_t* out) {
  float span[8], off[8], span_max = 0.0f, off_max = 0.0f;
  for (int j = 0; j < 8; ++j) {
    const float* v = w + 32 * j;
    float lo = 0.0f, hi = v[0];
    for (int i = 0; i < 32; ++i) {
      lo = std::min(lo, v[i]);
      hi = std::max(hi, v[i]);
    }
    span[j] = (hi - lo) / 15.0f;
    off[j] = 0.0f - lo;
    span_max = std::max(span_max, span[j]);
    off_max = std::max(off_max, off[j]);
  }
  const uint16_t dh = to_half_bits(span_max / 63.0f), mh = to_half_bits(off_max / 63.0f);
  if (!half_finite(dh) || !half_finite(mh)) return false;
  const float d = from_half_bits(dh), dmin = from_half_bits(mh);
  uint64_t field_lo = 0, field_hi = 0;  // the 96-bit code field, bits 0..63 and 64..95
  auto put_code = [&](int i, uint32_t c) {
    const int bit = 6 * i;
    if (bit < 64) field_lo |= (uint64_t)c << bit;
    if (bit + 6 > 64) field_hi |= bit >= 64 ? (uint64_t)c << (bit - 64) : (uint64_t)c >> (64 - bit);
  };
  out[0] = (uint8_t)(dh & 0xFF);
  out[1] = (uint8_t)(dh >> 8);
  out[2] = (uint8_t)(mh & 0xFF);
  out[3] = (uint8_t)(mh >> 8);
  for (int j = 0; j < 8; ++j) {
    const float sc = d != 0.0f ? std::min(63.0f, std::ceil(span[j] / d)) : 0.0f;
    const float mc = dmin != 0.0f ? std::min(63.0f, std::round(off[j] / dmin)) : 0.0f;
    put_code(j, (uint32_t)sc);
    put_code(8 + j, (uint32_t)mc);
    const float step = d * sc, offset = dmin * mc;
    uint8_t* nib = out + 16 + 16 * j;
    for (int i = 0; i < 16; ++i) {
      uint8_t pair = 0;
      for (int h = 0; h < 2; ++h) {
        float q = step != 0.0f ? std::round((w[32 * j + 2 * i + h] + offset) / step) : 0.0f;
        q = std::min(15.0f, std::max(0.0f, q));
        pair |= (uint8_t)((int)q << (4 * h));
      }
      nib[i] = pair;
    }
  }
  for (int b = 0; b < 8; ++b) out[4 + b] = (uint8_t)(field_lo >> (8 * b));
  for (int b = 0; b < 4; ++b) out[12 + b] = (uint8_t)(field_hi >> (8 * b));
  return true;
}

}  // namespace

int64_t block_weights(int qtype) { return qtype == QBL_Q4_K ? 256 : 32; }

// The 6-bit codes of sub-block j (scale, min) from a q4_K block's 12 code bytes.
void q4k_codes(const uint8_t* field, int j, uint32_t* sc, uint32_t* m) {
  uint64_t lo = 0, hi = 0;
  for (int b = 0; b < 8; ++b) lo |= (uint64_t)field[b] << (8 * b);
  for (int b = 0; b < 4; ++b) hi |= (uint64_t)field[8 + b] << (8 * b);
  auto code = [&](int i) -> uint32_t {
    const int bit = 6 * i;
    uint64_t v = bit < 64 ? lo >> bit : 0;
    if (bit + 6 > 64) v |= bit >= 64 ? hi >> (bit - 64) : hi << (64 - bit);
    return (uint32_t)(v & 63u);
  };
  *sc = code(j);
  *m = code(8 + j);
}

int quantize_rows(int qtype, const float* w, int64_t n, int64_t k, uint8_t* blocks, int nthreads) {
  const int64_t bb = qbl_block_bytes(qtype);
  const int64_t bw = block_weights(qtype);
  const int64_t nb = k / bw;
  std::vector<char> bad((size_t)n, 0);
  parallel_for(n, nthreads, [&](int64_t r) {
    const float* row = w + r * k;
    for (int64_t i = 0; i < k; ++i)
      if (!std::isfinite(row[i])) {
        bad[(size_t)r] = 1;
        return;
      }
    for (int64_t b = 0; b < nb; ++b) {
      uint8_t* dst = blocks + (r * nb + b) * bb;
      const float* src = row + bw * b;
      const bool ok = qtype == QBL_Q8_0 ? q8_block(src, dst) : qtype == QBL_Q4_SM ? q4_block(src, dst)
                                                                                 : q4k_block(src, dst);
      if (!ok) {
        bad[(size_t)r] = 2;
        return;
      }
    }
  });
  for (char c : bad) {
    if (c == 1) return QBL_E_NONFINITE;
    if (c == 2) return QBL_E_LIMIT;
  }
  return QBL_OK;
}

int dequantize_rows(int qtype, const uint8_t* blocks, int64_t n, int64_t k, float* out) {
  const int64_t bb = qbl_block_bytes(qtype);
  const int64_t bw = block_weights(qtype);
  const int64_t nb = k / bw;
  parallel_for(n, 0, [&](int64_t r) {
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t* p = blocks + (r * nb + b) * bb;
      const float d = from_half_bits((uint16_t)(p[0] | (p[1] << 8)));
      float* o = out + r * k + bw * b;
      if (qtype == QBL_Q4_K) {
        const float dmin = from_half_bits((uint16_t)(p[2] | (p[3] << 8)));
        for (int j = 0; j < 8; ++j) {
          uint32_t sc, m;
          q4k_codes(p + 4, j, &sc, &m);
          const float step = d * (float)sc, offset = dmin * (float)m;
          for (int i = 0; i < 16; ++i) {
            const uint8_t byte = p[16 + 16 * j + i];
            o[32 * j + 2 * i] = std::fma(step, (float)(byte & 0x0F), -offset);
            o[32 * j + 2 * i + 1] = std::fma(step, (float)(byte >> 4), -offset);
          }
        }
      } else if (qtype == QBL_Q8_0) {
        for (int j = 0; j < 32; ++j) o[j] = d * (float)(int8_t)p[2 + j];
      } else {
        const float m = from_half_bits((uint16_t)(p[2] | (p[3] << 8)));
        for (int i = 0; i < 16; ++i) {
          o[2 * i] = std::fma(d, (float)(p[4 + i] & 0x0F), m);
          o[2 * i + 1] = std::fma(d, (float)(p[4 + i] >> 4), m);
        }
      }
    }
  });
  return QBL_OK;
}

int64_t qs_bytes(int qtype, int64_t n, int64_t k) { return qtype == QBL_Q8_0 ? n * k : n * k / 2; }
int64_t sc_bytes(int qtype, int64_t n, int64_t k) {
  return qtype == QBL_Q8_0 ? n * (k / 32) * 2 : qtype == QBL_Q4_SM ? n * (k / 32) * 4 : n * (k / 256) * 16;
}

void repack_rows(int qtype, const uint8_t* blocks, int64_t n, int64_t k, uint8_t* qs, uint8_t* sc,
                 int nthreads) {
  const int64_t bb = qbl_block_bytes(qtype);
  const int64_t nb = k / block_weights(qtype);
  parallel_for(n, nthreads, [&](int64_t r) {
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t* p = blocks + (r * nb + b) * bb;
      if (qtype == QBL_Q4_K) {  // nibbles as they are; the 16-byte header beside them
        std::memcpy(qs + r * (k / 2) + 128 * b, p + 16, 128);
        std::memcpy(sc + (r * nb + b) * 16, p, 16);
      } else if (qtype == QBL_Q8_0) {  // offset-binary on the device: u = q + 128
        uint8_t* dst = qs + r * k + 32 * b;
        for (int j = 0; j < 32; ++j) dst[j] = (uint8_t)(p[2 + j] ^ 0x80u);
        std::memcpy(sc + (r * nb + b) * 2, p, 2);
      } else {
        std::memcpy(qs + r * (k / 2) + 16 * b, p + 4, 16);
        std::memcpy(sc + (r * nb + b) * 4, p, 4);  // d (low half) then m (high half)
      }
    }
  });
}

void unpack_rows(int qtype, const uint8_t* qs, const uint8_t* sc, int64_t n, int64_t k,
                 uint8_t* blocks) {
  const int64_t bb = qbl_block_bytes(qtype);
  const int64_t nb = k / block_weights(qtype);
  for (int64_t r = 0; r < n; ++r)
    for (int64_t b = 0; b < nb; ++b) {
      uint8_t* p = blocks + (r * nb + b) * bb;
      if (qtype == QBL_Q4_K) {
        std::memcpy(p, sc + (r * nb + b) * 16, 16);
        std::memcpy(p + 16, qs + r * (k / 2) + 128 * b, 128);
      } else if (qtype == QBL_Q8_0) {
        std::memcpy(p, sc + (r * nb + b) * 2, 2);
        const uint8_t* src = qs + r * k + 32 * b;
        for (int j = 0; j < 32; ++j) p[2 + j] = (uint8_t)(src[j] ^ 0x80u);
      } else {
        std::memcpy(p, sc + (r * nb + b) * 4, 4);
        std::memcpy(p + 4, qs + r * (k / 2) + 16 * b, 16);
      }
    }
}

// ---------------------------------------------------------------------------
// SHA-256, FIPS 180-4 section 6.2.
// ---------------------------------------------------------------------------
namespace {
constexpr uint32_t kK[64] = {
    0x428a2f98, 0x71374491, 0xb5c0fbcf, 0xe9b5dba5, 0x3956c25b, 0x59f111f1, 0x923f82a4, 0xab1c5ed5,
    0xd807aa98, 0x12835b01, 0x243185be, 0x550c7dc3, 0x72be5d74, 0x80deb1fe, 0x9bdc06a7, 0xc19bf174,
    0xe49b69c1, 0xefbe4786, 0x0fc19dc6, 0x240ca1cc, 0x2de92c6f, 0x4a7484aa, 0x5cb0a9dc, 0x76f988da,
    0x983e5152, 0xa831c66d, 0xb00327c8, 0xbf597fc7, 0xc6e00bf3, 0xd5a79147, 0x06ca6351, 0x14292967,
    0x27b70a85, 0x2e1b2138, 0x4d2c6dfc, 0x53380d13, 0x650a7354, 0x766a0abb, 0x81c2c92e, 0x92722c85,
    0xa2bfe8a1, 0xa81a664b, 0xc24b8b70, 0xc76c51a3, 0xd192e819, 0xd6990624, 0xf40e3585, 0x106aa070,
    0x19a4c116, 0x1e376c08, 0x2748774c, 0x34b0bcb5, 0x391c0cb3, 0x4ed8aa4a, 0x5b9cca4f, 0x682e6ff3,
    0x748f82ee, 0x78a5636f, 0x84c87814, 0x8cc70208, 0x90befffa, 0xa4506ceb, 0xbef9a3f7, 0xc67178f2};
inline uint32_t rotr(uint32_t x, int r) { return (x >> r) | (x << (32 - r)); }
}  // namespace

Sha256::Sha256() : h_{0x6a09e667, 0xbb67ae85, 0x3c6ef372, 0xa54ff53a, 0x510e527f, 0x9b05688c,
                      0x1f83d9ab, 0x5be0cd19},
                   len_(0), fill_(0) {}

void Sha256::block(const uint8_t* p) {
  uint32_t w[64];
  for (int i = 0; i < 16; ++i)
    w[i] = (uint32_t)p[4 * i] << 24 | (uint32_t)p[4 * i + 1] << 16 | (uint32_t)p[4 * i + 2] << 8 |
           (uint32_t)p[4 * i + 3];
  for (int i = 16; i < 64; ++i) {
    const uint32_t s0 = rotr(w[i - 15], 7) ^ rotr(w[i - 15], 18) ^ (w[i - 15] >> 3);
    const uint32_t s1 = rotr(w[i - 2], 17) ^ rotr(w[i - 2], 19) ^ (w[i - 2] >> 10);
    w[i] = w[i - 16] + s0 + w[i - 7] + s1;
  }
  uint32_t a = h_[0], b = h_[1], c = h_[2], d = h_[3], e = h_[4], f = h_[5], g = h_[6], h = h_[7];
  for (int i = 0; i < 64; ++i) {
    const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
    const uint32_t ch = (e & f) ^ (~e & g);
    const uint32_t t1 = h + S1 + ch + kK[i] + w[i];
    const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
    const uint32_t mj = (a & b) ^ (a & c) ^ (b & c);
    const uint32_t t2 = S0 + mj;
    h = g;
    g = f;
    f = e;
    e = d + t1;
    d = c;
    c = b;
    b = a;
    a = t1 + t2;
  }
  h_[0] += a;
  h_[1] += b;
  h_[2] += c;
  h_[3] += d;
  h_[4] += e;
  h_[5] += f;
  h_[6] += g;
  h_[7] += h;
}

void Sha256::update(const void* data, size_t n) {
  const uint8_t* p = static_cast<const uint8_t*>(data);
  len_ += n;
  if (fill_) {
    const size_t take = std::min(n, 64 - fill_);
    std::memcpy(buf_ + fill_, p, take);
    fill_ += take;
    p += take;
    n -= take;
    if (fill_ == 64) {
      block(buf_);
      fill_ = 0;
    }
  }
  while (n >= 64) {
    block(p);
    p += 64;
    n -= 64;
  }
  if (n) {
    std::memcpy(buf_, p, n);
    fill_ = n;
  }
}

void Sha256::final(uint8_t out[32]) {
  const uint64_t bits = len_ * 8;
  const uint8_t one = 0x80, zero = 0;
  update(&one, 1);
  while (fill_ != 56) update(&zero, 1);
  uint8_t be[8];
  for (int i = 0; i < 8; ++i) be[i] = (uint8_t)(bits >> (56 - 8 * i));
  update(be, 8);
  for (int i = 0; i < 8; ++i) {
    out[4 * i] = (uint8_t)(h_[i] >> 24);
    out[4 * i + 1] = (uint8_t)(h_[i] >> 16);
    out[4 * i + 2] = (uint8_t)(h_[i] >> 8);
    out[4 * i + 3] = (uint8_t)h_[i];
  }
}

}  // namespace qbl
