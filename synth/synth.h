/* Seeded synthetic input generator (SplitMix64 counter stream + Box-Muller).
 * Shared by the oracle tests and the GPU library's tests and benchmark; it
 * carries none of the method's arithmetic. */
#ifndef SYNTH_H
#define SYNTH_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif
/* i-th raw 64-bit draw of the SplitMix64 stream started at seed. */
uint64_t synth_splitmix64_at(uint64_t seed, uint64_t i);
/* Stream seed for a textual tag (FNV-1a 64, then SplitMix64 finalisation). */
uint64_t synth_seed_from_tag(const char* tag);
/* out[i] = float(mean + std * z_{offset+i}) for i < count, z the standard
 * normal stream of `seed`.  nthreads <= 0 picks the online core count (capped
 * by OMP_NUM_THREADS).  Returns 0, or -1 on a null output. */
int synth_normal_f32(uint64_t seed, uint64_t offset, uint64_t count, double mean, double std,
                     float* out, int nthreads);
/* out[i] = the 53-bit uniform in [0, 1) of draw offset+i of the stream. */
int synth_uniform_f64(uint64_t seed, uint64_t offset, uint64_t count, double* out);
#ifdef __cplusplus
}
#endif
#endif
