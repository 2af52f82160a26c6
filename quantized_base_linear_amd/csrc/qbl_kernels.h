// Launch interface between the host runtime and the gfx950 kernels.
// Internal to the library: not part of the C ABI.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

namespace qbl {

// Launch `kernel` on lc.stream, with lc's timing events when they are set.
#define QBL_LAUNCH(kernel, grid, block, lds, lc, ...)                                              \
  do {                                                                                             \
    if ((lc).start || (lc).stop)                                                                   \
      hipExtLaunchKernelGGL(kernel, grid, block, lds, (lc).stream, (lc).start, (lc).stop, 0,       \
                            __VA_ARGS__);                                                          \
    else                                                                                           \
      hipLaunchKernelGGL(kernel, grid, block, lds, (lc).stream, __VA_ARGS__);                      \
  } while (0)

constexpr int QBL_FMT_Q8 = 1;  // same values as QBL_Q8_0 / QBL_Q4_SM / QBL_Q4_K of the C ABI
constexpr int QBL_FMT_Q4 = 2;
constexpr int QBL_FMT_Q4K = 3;
constexpr int kMaxAdapters = 8;
constexpr int kMaxSegs = 3;                        // linears sharing one input in one launch
constexpr int kMaxPrepEntries = kMaxSegs * kMaxAdapters;

// The adapters of one linear in list order, as the expand needs them.  An
// entry of rank 0 is a sparse delta: row r's entries are rp[r] .. rp[r+1]-1,
// with columns ci[] and fp16 values sv[] (its toff and B are unused).
struct LoraSeg {
  int n_ad;
  int prefetch;              // set by launch_gemv: B rows loaded up front
  int toff[kMaxAdapters];    // offset of t_i within a batch row of the t buffer
  int rank[kMaxAdapters];
  float scale[kMaxAdapters];
  const float* B[kMaxAdapters];  // n_out x rank, row-major
  const uint32_t* rp[kMaxAdapters];
  const uint32_t* ci[kMaxAdapters];
  const uint16_t* sv[kMaxAdapters];
};

// One linear of a fused GEMV launch.
struct GemvSeg {
  const uint8_t* qs;   // q8_0: offset-binary bytes q + 128 [n][k]; q4_sm, q4_K: packed nibbles [n][k/2]
  const void* sc;      // q8_0: fp16 d [n][k/32]; q4_sm: uint32 (d | m << 16) [n][k/32];
                       // q4_K: 16-byte super-block header (d, dmin, 12 code bytes) [n][k/256]
  float* y;            // [batch][y_stride]
  int64_t y_stride;
  int n;
  int wg_begin;        // first workgroup of this segment
  LoraSeg lora;
};

struct GemvArgs {
  GemvSeg seg[kMaxSegs];
  int nseg;
  int qtype;
  int k;
  int kt;              // input-tile width staged in LDS
  int batch;
  int rpw;             // rows per wave
  const float* x;      // [batch][x_stride]
  int64_t x_stride;
  const float* t;      // [batch][t_stride] shrink results (may be null when no adapters)
  int t_stride;
  int grid;
};

// One (adapter, linear) pair whose shrink t = A x a prep launch computes.
struct PrepEntry {
  const float* A;      // rank x k
  int rank;
  int toff;
};

// Input glue + LoRA shrink.  xin = c * (v0 + v1 + v2) with c = rms scale or 1.
struct PrepArgs {
  const float* v[3];
  int nv;
  int rms;             // 1: c = 1/sqrt(mean(s^2) + 1e-6) of the summed vector (batch 1 only)
  int batch;
  int k;
  int64_t v_stride;    // between batch rows of the inputs
  float* xin;          // [batch][k] or null
  float* t;            // [batch][T] or null
  int T;
  int n_ent;
  int rows_total;      // sum of entry ranks
  PrepEntry ent[kMaxPrepEntries];
};

// Batch-1 GEMV with the glue and the shrink in the same launch.  The first
// GEMV workgroups compute one value of t each (or, when the launch has fewer
// GEMV workgroups than A rows, workgroups [0, shrink_wgs) compute t, kRS rows
// of A each) and store each value as one 64-bit word tagged with the launch's
// number; every GEMV workgroup reads t only after its row loop, waiting
// (bounded) until each word carries this launch's tag.  Input: s = v0 + v1 +
// v2, scaled by c (RMS or 1).
struct FusedArgs {
  GemvArgs g;          // segments (qs, sc, y, n, lora), nseg, qtype, k; wg_begin set by the launcher
  const float* v[3];
  int nv;
  int rms;
  int sum;             // 1: segments of equal height summed into seg[0].y
  int rows_per_wg;     // set by the launcher
  int n_ent;
  int rows_total;      // A rows = shrink results
  int has_sparse;      // 1: some segment has a sparse delta
  int shrink_wgs;      // set by the launcher
  int shrink_in_gemv;  // set by the launcher: 1 = no shrink workgroups; GEMV workgroup i < rows_total computes t[i]
  int sparse_wgs;      // set by the launcher (0 when sp_items == 0)
  int sp_items;        // sparse (segment, adapter, row) items: S x values handed to the GEMV workgroups
  int64_t sp_bytes;    // CSR bytes of the launch (for the launcher's split of the round)
  int sp_base[kMaxSegs][kMaxAdapters];  // first item of (segment, adapter), -1 unless the adapter is sparse
  uint64_t* sp;        // sp_items tagged words (launch number << 32 | float bits)
  int64_t wait_ticks;  // wall-clock ticks (100 MHz) a thread may spend waiting for handed-over values
  uint32_t* fail;      // status word a wait sets when it gives up (coherent host memory)
  uint32_t tag;        // this launch's number, never 0: written beside every handed-over value
  uint32_t read_tag;   // the number readers wait for: tag (another value only under test fault injection)
  int expand_lanes;    // set by the launcher: lanes per row in the expand (1, or for ranks above 32 one per 16 of the largest)
  uint64_t* t;         // kTCopies copies of the rows_total shrink results, (tag << 32) | float bits
  int64_t t_copy_stride;  // words between copies (see t_copy_stride())
  PrepEntry ent[kMaxPrepEntries];
};

// JIT prefill: Y[m][n] = sum_k X[m][k] * Weff[n][k], Weff built tile by tile.
struct JitArgs {
  int qtype;
  const uint8_t* qs;
  const void* sc;
  int n, k, m;
  const uint16_t* X;   // bf16 [m][k]
  float* Y;            // [m][n]
  int n_ad;
  const float* A[kMaxAdapters];  // rank x k fp32
  const float* B[kMaxAdapters];  // n x rank fp32
  int rank[kMaxAdapters];
  float scale[kMaxAdapters];
  int total_rank;
  uint16_t* ws;        // scratch for the staged bf16 factors (see launch_jit)
};

// Dequantize-add-requantize of one linear under an adapter list (a merge the
// overlay never performs; used to measure its drift): canonical blocks of
// Q(deq(W) + sum of the adapters' deltas) into out.  Adapter entries as in
// LoraSeg (rank 0: sparse delta rp/ci/sv; otherwise A rank x k and B n x rank).
struct DarArgs {
  int qtype;
  const uint8_t* qs;
  const void* sc;
  int n, k;
  int n_ad;
  int rank[kMaxAdapters];
  float scale[kMaxAdapters];
  const float* A[kMaxAdapters];
  const float* B[kMaxAdapters];
  const uint32_t* rp[kMaxAdapters];
  const uint32_t* ci[kMaxAdapters];
  const uint16_t* sv[kMaxAdapters];
  uint8_t* out;
};

// Where a kernel goes: the stream, and optionally a pair of events that the
// runtime attaches to the dispatch itself (hipExtLaunchKernelGGL) so that they
// time the kernel's execution.
struct LaunchCtx {
  hipStream_t stream = nullptr;
  hipEvent_t start = nullptr, stop = nullptr;
};

hipError_t launch_prep(const PrepArgs& a, const LaunchCtx& lc);
// y = v / sqrt(mean(v^2) + 1e-6), one vector of n floats (n a multiple of 4)
hipError_t launch_rms(const float* v, int n, float* y, const LaunchCtx& lc);
hipError_t launch_gemv(GemvArgs& a, const LaunchCtx& lc);
// Batch 2..8 on the matrix cores (no input glue): a prep launch (the inputs as
// f16 instruction operands with their per-row exponents, and the low-rank
// shrink summed by input range), timed by prep_lc, then the GEMV launch and,
// when K is split, a reduce launch (both timed by lc); the launch that finishes
// the rows adds the shrink's ranges in order (a.t is not used).  `stage`: mfma_stage_bytes(rows, k, T) bytes, rows = all
// output rows of the launch, 256-byte aligned.  ent: the shrink entries with
// toff = running sum of the ranks.  ks: workgroups per 64 rows splitting K
// (1..16; 0 picks it from the shape).
int64_t mfma_stage_only_bytes(int k);
int64_t mfma_scan_bytes(int k, int T);
int64_t mfma_partial_bytes(int64_t rows);
int64_t mfma_stage_bytes(int64_t rows, int k, int T);
hipError_t launch_gemv_mfma(GemvArgs& a, const PrepEntry* ent, int n_ent, int T, void* stage, int ks,
                            const LaunchCtx& prep_lc, const LaunchCtx& lc);
// false when the fused path cannot serve this shape (the caller then uses prep + gemv)
bool fused_supported(int qtype, int k);
hipError_t launch_fused(FusedArgs& f, const LaunchCtx& lc);
// The shrink results of a fused launch are stored kTCopies times, copy c read by
// GEMV workgroups c, c + kTCopies, ...: every workgroup reads them, and one copy
// would put all those reads on one memory channel.  Copies sit t_copy_stride(T)
// words apart (a 256-byte multiple plus 256 bytes, so they fall on different
// channels).
constexpr int kTCopies = 8;
inline int64_t t_copy_stride(int64_t rows) { return (rows + 31) / 32 * 32 + 32; }
hipError_t launch_jit(const JitArgs& a, const LaunchCtx& lc);

// The no-allocation variant of qbl_linear uses one file-scope device array per
// GPU as its workspace: kStaticScratchBytes (32 MiB) each.  static_scratch
// returns the current device's copy, setting it up on the device's first call
// (its address, then a clear enqueued on st; hipErrorStreamCaptureUnsupported
// if st is capturing then).
constexpr int64_t kStaticScratchBytes = 32ll << 20;
hipError_t static_scratch(hipStream_t st, void** out);

int64_t jit_workspace_bytes(int n, int k, int total_rank);
hipError_t launch_dar(const DarArgs& a, const LaunchCtx& lc);
// Read-only streaming probe: reads `bytes` (a multiple of 16) at buf once; the
// XOR of each workgroup's words goes to sink[workgroup] for probe_workgroups()
// workgroups.
int probe_workgroups(int sink_words);
hipError_t launch_hbm_probe(const void* buf, int64_t bytes, uint32_t* sink, int sink_words, const LaunchCtx& lc);

}  // namespace qbl
