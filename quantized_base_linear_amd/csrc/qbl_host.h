// Host-side helpers of the library (not part of the C ABI).
#pragma once
#include <cstddef>
#include <cstdint>
#include <functional>
#include <string>

namespace qbl {

// FIPS 180-4 SHA-256.
class Sha256 {
 public:
  Sha256();
  void update(const void* data, size_t n);
  void final(uint8_t out[32]);

 private:
  void block(const uint8_t* p);
  uint32_t h_[8];
  uint8_t buf_[64];
  uint64_t len_;
  size_t fill_;
};

// Runs fn(i) for i in [0, n) on up to nthreads threads (<= 0: online cores).
void parallel_for(int64_t n, int nthreads, const std::function<void(int64_t)>& fn);
int default_threads();

// Host quantisers over canonical blocks (see qbl.h).  Return a qbl status.
int quantize_rows(int qtype, const float* w, int64_t n, int64_t k, uint8_t* blocks, int nthreads);
int dequantize_rows(int qtype, const uint8_t* blocks, int64_t n, int64_t k, float* out);

// Weights per canonical block: 32, or 256 for q4_K.
int64_t block_weights(int qtype);

// Canonical blocks -> device layout (host staging buffers):
//   q8_0 : qs offset-binary bytes u = q + 128 [n][k] and d fp16 [n][k/32]
//   q4_sm: qs packed nibbles [n][k/2] and dm uint32 (d | m << 16) [n][k/32]
//   q4_K : qs packed nibbles [n][k/2] and the 16-byte super-block header
//          (d, dmin, 12 code bytes) [n][k/256]
void repack_rows(int qtype, const uint8_t* blocks, int64_t n, int64_t k, uint8_t* qs, uint8_t* sc,
                 int nthreads);
// The inverse of repack_rows: device-layout arrays back to canonical blocks.
void unpack_rows(int qtype, const uint8_t* qs, const uint8_t* sc, int64_t n, int64_t k,
                 uint8_t* blocks);
int64_t qs_bytes(int qtype, int64_t n, int64_t k);
int64_t sc_bytes(int qtype, int64_t n, int64_t k);

}  // namespace qbl
