/*
 * qbl: the dual-path quantized-base + LoRA linear on AMD Instinct MI355X (gfx950).
 *
 *   y = dequant(W_q) x + sum_i s_i B_i (A_i x)        adapters summed in list order
 *
 * over an immutable block-quantized base (q8_0 or q4_sm), plus a per-layer
 * just-in-time path for multi-token prefill that materialises
 * W_eff = dequant(W_q) + sum_i s_i B_i A_i in on-chip scratch, uses it and
 * discards it.
 *
 * The operations follow three pages on quantized-base adapter overlays:
 *  [overlay]  mikekappel.com, "We propose a content-addressed overlay system"
 *             (sections "Composition Identity and Manifest Schema", "Explicit
 *             Correctness and Atomicity Invariants", "Proposed Activation/
 *             Deactivation State Machine", "TDD and Fault-Injection Matrix",
 *             "Runtime Strategy Comparison Matrix", "Native/WASM Kernel
 *             Implications", "Clean Replacement Plan and Rejection Criteria");
 *  [design]   mikekappel.com, "Deep Technical Design: Exact, Atomic, Reversible
 *             Specialist Overlays" (sections 1, 2, 5, 6, 8, 9, 11);
 *  [lora]     contenox.com, "LoRA adapters" blueprint ("Backend Support
 *             Position", llama.cpp adapter API and its shape rules, "Runtime
 *             Identity and Cache Safety").
 *
 * Conventions for every call:
 *  - Every function returns a qbl_status (0 = QBL_OK, negative = error) unless
 *    stated.  On error nothing changed: no handle, composition or base byte is
 *    modified, out-parameters are left untouched, and qbl_last_error() returns
 *    a description (thread-local).  No C++ exception crosses this boundary.
 *  - "host" pointers are CPU memory; "device" pointers are GPU memory of the
 *    base's device (e.g. torch CUDA tensors).  Matrices are row-major, float32
 *    unless stated, contiguous, and at least 16-byte aligned.
 *  - stream is a hipStream_t passed as void* (NULL = the null stream).  Run
 *    calls only enqueue work on it and return without synchronising.
 *  - The library owns the device copies of bases and adapters; the caller owns
 *    x, y and the workspace.  Calls on one composition from several host threads
 *    are serialised by the library.
 */
#ifndef QBL_H
#define QBL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QBL_ABI_VERSION 2

typedef int32_t qbl_status;
#define QBL_OK 0
#define QBL_E_ARG (-1)        /* null pointer, bad index or count */
#define QBL_E_SHAPE (-2)      /* dimensions do not match the base */
#define QBL_E_FORMAT (-3)     /* unknown quantisation type, k not a multiple of 32, bad byte count */
#define QBL_E_NONFINITE (-4)  /* NaN/Inf in weights, adapter factors or scales */
#define QBL_E_NOMEM (-5)      /* device or host allocation failed */
#define QBL_E_BUDGET (-6)     /* workspace too small, or a base's device-memory budget exceeded */
#define QBL_E_BUSY (-7)       /* object still referenced */
#define QBL_E_DEVICE (-8)     /* a HIP runtime call failed */
#define QBL_E_FOREIGN (-9)    /* adapter bound to another base */
#define QBL_E_DUPLICATE (-10) /* the same handle twice in one list, or one linear twice in one adapter */
#define QBL_E_LIMIT (-11)     /* above a documented limit */
#define QBL_E_CHECKSUM (-12)  /* a device copy read back differs from the bytes sent */
#define QBL_E_INJECTED (-13)  /* a failure armed with qbl_fault_inject fired */
#define QBL_E_STATE (-14)     /* the call does not apply to the object's state */

/* Quantisation types.
 * QBL_Q8_0: blocks of 32 weights along k: one fp16 scale d and 32 int8 q,
 *   w = d*q ([design] section 5: 32 weights and one f16 scale, 8.5 bits per
 *   weight).  Canonical block bytes: [d as fp16 little-endian][q0..q31] = 34 B.
 * QBL_Q4_SM: blocks of 32 weights: fp16 scale d, fp16 min m, 32 unsigned
 *   4-bit q, w = d*q + m ([design] section 5: per-block scale and minimum).
 *   Canonical block bytes: [d][m][16 B; byte i = q[2i] | q[2i+1] << 4] = 20 B. */
#define QBL_Q8_0 1
#define QBL_Q4_SM 2
/* QBL_Q4_K: super-blocks of 256 weights in 8 sub-blocks of 32 ([design]
 *   section 5: a 6-bit scale and a 6-bit minimum per sub-block under two f16
 *   super-scales, 4.5 bits per weight).  Sub-block j has step D_j = d * sc_j and
 *   offset M_j = dmin * m_j (sc_j, m_j in 0..63) and w = D_j * q - M_j, q in 0..15.
 *   Canonical block bytes (144): [d fp16][dmin fp16][12 B: sixteen 6-bit codes,
 *   code i in bits 6i..6i+5 of the 96-bit little-endian field, codes 0..7 =
 *   sc_0..sc_7, 8..15 = m_0..m_7][128 B: sub-block j's 16 bytes at offset
 *   16 + 16j, byte i = q[32j + 2i] | q[32j + 2i + 1] << 4].  The page names the
 *   parts but not their bit layout; this layout is the library's. */
#define QBL_Q4_K 3

/* Limits. */
#define QBL_MAX_ADAPTERS 8     /* entries in one attached list */
#define QBL_MAX_RANK 256       /* rank of one adapter on one linear */
#define QBL_MAX_TOTAL_RANK 512 /* sum of ranks on one linear over an attached list */
#define QBL_MAX_BATCH 8        /* rows of x for qbl_linear */
#define QBL_MAX_K 65536        /* input features of a linear */

typedef struct qbl_base qbl_base;
typedef struct qbl_adapter qbl_adapter;
typedef struct qbl_comp qbl_comp;

/* Text of the calling thread's last error ("" if none).  Never NULL. */
const char* qbl_last_error(void);

/* QBL_ABI_VERSION of the built library (not a status). */
int32_t qbl_abi_version(void);

/* Bytes of one block of qtype (q8_0 34, q4_sm 20, q4_K 144); 0 for an unknown type. */
int64_t qbl_block_bytes(int32_t qtype);

/* Weights of one block of qtype (32, or 256 for q4_K); 0 for an unknown type.
 * A linear's k_in must be a multiple of it. */
int64_t qbl_block_weights(int32_t qtype);

/* Quantise a host float32 matrix w (n x k, k a multiple of qbl_block_weights)
 * into canonical blocks (host, n*k/qbl_block_weights*qbl_block_bytes bytes,
 * caller-owned).
 * q8_0: d = fp16(max|w|/127), q = round-half-away(w / d) with the stored d, clamped
 *   to [-127, 127]; an all-zero block gives d = 0, q = 0.
 * q4_sm: m = fp16(min w), d = fp16((max w - m)/15), q = round-half-away((w - m)/d)
 *   clamped to [0, 15]; q = 0 where d = 0.
 * q4_K: per sub-block lo = min(0, min w), hi = max w, s = (hi - lo)/15, t = 0 - lo;
 *   d = fp16(max s / 63), dmin = fp16(max t / 63); sc = min(63, ceil(s / d)),
 *   m = min(63, round-half-away(t / dmin)) (0 where the super-scale is 0);
 *   q = round-half-away((w + M)/D) clamped to [0, 15]; q = 0 where D = 0.
 * All arithmetic in float32.  nthreads <= 0 uses the online cores.
 * QBL_E_NONFINITE on NaN/Inf input, QBL_E_LIMIT if a scale, minimum or
 * super-scale would overflow fp16. */
qbl_status qbl_quantize(int32_t qtype, const float* w, int64_t n, int64_t k, void* blocks_out,
                        int32_t nthreads);

/* SHA-256 (FIPS 180-4) of n host bytes: the digest used by qbl_base_hash and
 * qbl_adapter_digest. */
qbl_status qbl_sha256(const void* data, int64_t n, uint8_t sha256_out[32]);

/* Dequantise canonical blocks (host) to float32 (host, n x k); q4_K as
 * fma(D, q, -M) in float32. */
qbl_status qbl_dequantize(int32_t qtype, const void* blocks, int64_t n, int64_t k, float* w_out);

/* ---------------------------------------------------------------- base --- */

/* One linear of a base: n_out x k_in weights as canonical blocks in host memory. */
typedef struct {
  int32_t qtype;
  int32_t reserved; /* must be 0 */
  int64_t n_out;
  int64_t k_in;
  const void* blocks; /* host, n_out * k_in/qbl_block_weights * qbl_block_bytes(qtype) bytes */
  int64_t nbytes;     /* must equal that size */
} qbl_linear_desc;

/* Load an immutable base of n_linears linears onto the current HIP device.
 * Linears are numbered 0..n_linears-1 in this order.  Block b of a stack is
 * linears 7b..7b+6 in the order q, k, v, o, gate, up, down; qbl_block and
 * qbl_decode check those shapes when called.  The library copies the blocks
 * (the caller may free them on return), repacks them into its device layout,
 * uploads them, reads every device copy back and compares it byte for byte with
 * what it sent (QBL_E_CHECKSUM on a difference: [design] section 6, checksum
 * verification of a staged block), records the base digest (qbl_base_digest)
 * and seals the bytes: no kernel ever receives a writable pointer to base bytes
 * ([design] section 2, the oracle invariant: base bytes stay bit-identical).
 * On any failure every allocation made so far is freed.  *out receives the
 * handle. */
qbl_status qbl_base_load(const qbl_linear_desc* descs, int32_t n_linears, qbl_base** out);

/* The base digest recorded at load, from the canonical blocks it was given:
 * SHA-256 (FIPS 180-4) over the concatenation, in linear order, of each
 * linear's SHA-256 over the 24-byte little-endian header
 * [int32 qtype][int32 0][int64 n_out][int64 k_in] followed by its canonical
 * blocks.  It names the exact quantised bytes and their format, the first
 * fields of a composition's identity ([overlay] "Composition Identity and
 * Manifest Schema": base hash and quantisation profile). */
qbl_status qbl_base_digest(const qbl_base* base, uint8_t sha256_out[32]);

/* The same digest computed now from the device bytes, re-read from the GPU and
 * translated back to canonical blocks.  It equals qbl_base_digest as long as
 * the device copy is intact, before and after any attach, clear or run
 * ([overlay] "Checksum Verification"; [design] section 2). */
qbl_status qbl_base_hash(qbl_base* base, uint8_t sha256_out[32]);

/* Number of linears, and one linear's type and shape. */
qbl_status qbl_base_count(const qbl_base* base, int32_t* n_linears);
qbl_status qbl_base_info(const qbl_base* base, int32_t linear, int32_t* qtype, int64_t* n_out,
                         int64_t* k_in);

/* Free a base.  QBL_E_BUSY while any adapter or composition still refers to it
 * (adapters are owned by the base they were loaded against, as in [lora]). */
qbl_status qbl_base_free(qbl_base* base);

/* Device-memory budget of a base: a cap on the device bytes held on its behalf,
 * its own arrays plus the arena of every adapter loaded against it that is
 * still alive.  0 = no cap (the default).  An adapter load that would take the
 * total above the cap fails with QBL_E_BUDGET before it allocates anything
 * ([overlay] "Bounded Resources" and the state machine's validation: the
 * composition must fit a fixed memory budget; [design] section 6 ALLOCATION: abort when the request exceeds what is
 * available).  Setting a cap below the bytes already held fails with
 * QBL_E_BUDGET and keeps the old cap. */
qbl_status qbl_base_set_budget(qbl_base* base, int64_t budget_bytes);

/* Bytes held now (base arrays + live adapter arenas) and the cap (0 = none). */
qbl_status qbl_base_memory(const qbl_base* base, int64_t* held_bytes, int64_t* budget_bytes);

/* ------------------------------------------------------------- adapters --- */

/* One LoRA factor pair on one linear of the base: A is rank x k_in, B is
 * n_out x rank, host float32 row-major ([overlay] "Memory, Byte, and Latency
 * Formulas": A in R^{r x n}, B in R^{m x r}).  Shapes must satisfy the
 * llama.cpp rule quoted in [lora]: A's columns = the base's inputs, B's rows =
 * the base's outputs, A's rows = B's columns = rank. */
typedef struct {
  int32_t linear;
  int32_t rank; /* 1..QBL_MAX_RANK */
  const float* A;
  const float* B;
} qbl_lora_desc;

/* Validate, stage and verify an adapter touching n >= 1 linears of base (no
 * linear twice), following [design] section 6: validation (shapes, ranks,
 * finite values, known linears: [design] section 11 deep compatibility checks;
 * [lora]: an adapter that matches zero layers is rejected), allocation of one
 * device arena within the base's budget, staging of every A and B into it, and
 * verification: each device copy is read back and compared byte for byte with
 * what was sent (QBL_E_CHECKSUM on a difference).  Any failure frees the arena
 * and leaves nothing behind.  The adapter is bound to base.  *out receives the
 * handle. */
qbl_status qbl_adapter_load(qbl_base* base, const qbl_lora_desc* descs, int32_t n,
                            qbl_adapter** out);

/* One sparse delta S on one linear of the base (n_out x k_in), in CSR form
 * ([design] "Sparse Overlay Bytes": DARE-masked task vectors stored as 4-byte
 * indices and 2-byte f16 values; [overlay] "Runtime Strategy Comparison
 * Matrix": a sparse overlay adds values only at its indices).  All host:
 *   row_ptr: n_out + 1 uint32, row_ptr[0] = 0, non-decreasing, row_ptr[n_out] = nnz;
 *   col:     nnz uint32 column indices, strictly increasing within each row, < k_in;
 *   val:     nnz fp16 bit patterns, finite.
 * col and val may be NULL when nnz = 0. */
typedef struct {
  int32_t linear;
  int32_t reserved; /* must be 0 */
  int64_t nnz;
  const uint32_t* row_ptr;
  const uint32_t* col;
  const uint16_t* val;
} qbl_sparse_desc;

/* Validate, stage and verify a sparse adapter touching n >= 1 linears (no
 * linear twice), like qbl_adapter_load.  The deep checks of [design] section
 * 11 are applied to every entry: row_ptr from 0 to nnz and non-decreasing
 * (QBL_E_SHAPE), columns inside the row (QBL_E_SHAPE) and strictly increasing
 * within each row (QBL_E_FORMAT), values finite (QBL_E_NONFINITE).  On the
 * decode path the adapter adds scale * (S x) to the output, in list order with
 * the other adapters; the prefill path refuses lists holding one
 * (QBL_E_FORMAT).  *out receives the handle, used like any other adapter. */
qbl_status qbl_adapter_load_sparse(qbl_base* base, const qbl_sparse_desc* descs, int32_t n,
                                   qbl_adapter** out);

/* SHA-256 of the adapter content: over the concatenation, in entry order, of
 * each entry's SHA-256 over, little-endian, [int32 linear][int32 rank] followed
 * by A's and then B's float32 bytes (low-rank), or [int32 linear][int32 -1]
 * [int64 nnz] followed by row_ptr, col and val (sparse). */
qbl_status qbl_adapter_digest(const qbl_adapter* adapter, uint8_t sha256_out[32]);

/* Drop the caller's reference.  Device memory lives on while an attached list
 * uses the adapter, and until the last enqueued run that read it completes. */
qbl_status qbl_adapter_free(qbl_adapter* adapter);

/* --------------------------------------------------------- compositions --- */

/* A composition: a base plus an ordered adapter list, initially empty.  An
 * empty list is the base-only path. */
qbl_status qbl_comp_create(qbl_base* base, qbl_comp** out);

/* Replace the composition's adapter list with list[0..n) and effective scales
 * scales[0..n) (alpha/rank already folded in, as [lora] describes for both
 * backends; any finite value, negative included), 0 <= n <= QBL_MAX_ADAPTERS.
 * Everything is validated before anything changes: every adapter bound to this
 * base (QBL_E_FOREIGN), no handle twice (QBL_E_DUPLICATE), scales finite, the
 * summed rank per linear within QBL_MAX_TOTAL_RANK.  Then a new immutable list
 * replaces the old one in a single atomic exchange ([overlay] "Atomic Update";
 * [design] section 6 COMMIT/SWAP), and the replaced list is kept as the
 * composition's previous list (qbl_comp_rollback).  Entries with scale 0 are
 * dropped, so an all-zero list runs exactly the base-only instructions.  Runs
 * already enqueued keep the list they captured.  Attaching the list already in
 * place changes nothing, not even the previous list ([overlay] "Idempotency"). */
qbl_status qbl_comp_attach(qbl_comp* comp, const qbl_adapter* const* list, const float* scales,
                           int32_t n);

/* Empty the list (deactivation: drop the adapter references, the base is
 * untouched; [design] section 6 "Exact Deactivation Flow").  Like an attach,
 * it keeps the replaced list as the previous list; clearing an empty list
 * changes nothing. */
qbl_status qbl_comp_clear(qbl_comp* comp);

/* Exchange the current and the previous list in one atomic step: the list that
 * the last successful attach, clear or rollback replaced becomes current again
 * ([overlay] state machine: the old state may be kept, and rollback restores
 * it).  A second rollback returns to the list the first one left.  QBL_E_STATE
 * when there is no previous list. */
qbl_status qbl_comp_rollback(qbl_comp* comp);

/* Release the previous list, and with it any adapter memory that only it still
 * holds.  Rollback is then unavailable until the next change. */
qbl_status qbl_comp_drop_previous(qbl_comp* comp);

/* Number of effective (non-zero-scale) entries in the current list. */
qbl_status qbl_comp_count(const qbl_comp* comp, int32_t* n);

/* Identity of the current composition: qbl_identity_digest of the base digest
 * and the current list.  Equal compositions (same base bytes, same effective
 * adapters, order and scales) have equal digests; a change of any of them
 * changes it. */
qbl_status qbl_comp_digest(const qbl_comp* comp, uint8_t sha256_out[32]);

/* The composition identity digest, defined on its own so that a caller can
 * compute it for a manifest before attaching ([overlay] "Composition Identity
 * and Manifest Schema": base hash, ordered adapter hashes, mixing weights and
 * the runtime version; [lora] "Runtime Identity and Cache Safety": adapter
 * order, digests and scales).  SHA-256 over, little-endian:
 *   [int32 QBL_ABI_VERSION][base_digest: 32 B][int32 m]
 *   then for each of the m entries i with scales[i] != 0, in list order:
 *   [adapter_digests[32*i .. 32*i+32)][float32 scales[i]]
 * Zero-scale entries (either sign of zero) are skipped, as attach drops them.
 * adapter_digests holds n digests of 32 B (host).  QBL_E_NONFINITE for a NaN or
 * infinite scale; 0 <= n <= QBL_MAX_ADAPTERS. */
qbl_status qbl_identity_digest(const uint8_t base_digest[32], const uint8_t* adapter_digests,
                               const float* scales, int32_t n, uint8_t sha256_out[32]);

qbl_status qbl_comp_free(qbl_comp* comp);

/* ------------------------------------------------------ fault injection --- */

/* For tests only: production code never calls this ([overlay] "TDD and
 * Fault-Injection Matrix": force a failure in each phase of an activation and
 * check that the previous state is intact).  Arms `point` to fire once, on its
 * `after`-th hit from now (1 = the next hit); after = 0 disarms it.  Points are
 * process-wide and thread-safe.
 *   QBL_FAULT_DEVICE_ALLOC: a device allocation by qbl_base_load (one per
 *     linear) or qbl_adapter_load (one per adapter) fails: QBL_E_NOMEM.
 *   QBL_FAULT_CORRUPT: after one upload (a base linear, or one adapter entry's
 *     A and B) the library changes one byte of the device copy before reading
 *     it back: QBL_E_CHECKSUM.
 *   QBL_FAULT_SWAP: an attach, clear or rollback fails after its new list is
 *     built and just before the exchange: QBL_E_INJECTED. */
#define QBL_FAULT_DEVICE_ALLOC 1
#define QBL_FAULT_CORRUPT 2
#define QBL_FAULT_SWAP 3
/*   QBL_FAULT_HANDOFF: the next batch-1 launch that hands adapter values over
 *     inside itself (see qbl_workspace_bytes) has its readers wait, with a zero
 *     time budget, for a launch number no writer stores: every wait gives up,
 *     the kernel still ends normally, and the failure is recorded for
 *     qbl_device_status (the run call itself returns QBL_OK: it only enqueues). */
#define QBL_FAULT_HANDOFF 4
qbl_status qbl_fault_inject(int32_t point, int32_t after);

/* Device-side failures that a run call cannot see when it enqueues
 * ([overlay] "Explicit Correctness and Atomicity Invariants": a hard,
 * deterministic error rather than a silent wrong result).  Batch-1 launches
 * hand values over between their workgroups (the adapter shrink, sparse row
 * sums), and a reader waits for each value under a time budget (50 ms per
 * thread and launch).  A wait that runs out records the failure in a
 * process-wide word of host memory, and that run's outputs are wrong.  While a
 * failure is recorded, every run call (qbl_linear, qbl_linear_jit, qbl_block,
 * qbl_decode) returns QBL_E_DEVICE without enqueueing anything.  This call
 * returns QBL_E_DEVICE once per recorded failure and clears the record, else
 * QBL_OK.  It does not synchronise: synchronise the streams first to include
 * every finished launch. */
qbl_status qbl_device_status(void);

/* ------------------------------------------------------------------ runs --- */

/* Workspace bytes (device, caller-owned, 256-byte aligned) that a run needs:
 *   op 0: qbl_linear on `index` = linear at batch m;
 *   op 1: qbl_linear_jit on linear `index` with m rows;
 *   op 2: qbl_block / qbl_decode (index ignored; m ignored).
 * The size depends on the current list; query after attach.  Op 0 above batch
 * 1 always needs a workspace (the inputs are staged there as f16 operands of
 * the matrix-core GEMV, with the partial sums of workgroups that split K),
 * with or without adapters.
 * At batch 1 (ops 0 and 2) one launch both computes the adapter shrink and
 * consumes it: each shrink value is stored with the launch's number beside it,
 * and readers wait until they see that number.  Zero the buffer once before its
 * first use (e.g. hipMemset) so that it holds no stale number; the library
 * keeps it valid afterwards.  Launch numbers are process-wide and repeat after
 * 2^32 launches: a stale word could only be taken for a fresh one if no launch
 * had rewritten it in the last 2^32 launches of the process.  Runs sharing one
 * workspace must be ordered on one stream: concurrent runs on one workspace race
 * on its contents.  A launch's number is fixed when the run is enqueued, so a
 * replayed graph would accept the values its previous replay left: batch-1 runs
 * with adapters return QBL_E_STATE on a stream that is capturing a graph (checked
 * before anything is enqueued).  A reader's wait is bounded; see
 * qbl_device_status. */
qbl_status qbl_workspace_bytes(const qbl_comp* comp, int32_t op, int32_t index, int32_t m,
                               int64_t* bytes_out);

/* Dual path, decode ([overlay] "Native/WASM Kernel Implications": y = xW + x(BA)
 * as a shrink t = A x then an expand B t; [design] section 8: dual path for
 * batch-one GEMV, kernels fused so adapter rows are used as the base block is
 * consumed; section 9: weighted adapters added at the final accumulation).
 *   y[b][n] = sum_k deq(W)[n][k] x[b][k] + sum_i s_i sum_j B_i[n][j] t_i[b][j],
 *   t_i[b] = A_i x[b]   (a sparse adapter i adds s_i sum_p val_i[p] x[b][col_i[p]]
 *   over row n's entries instead),
 * base sum first, adapters in list order, float32 accumulation.  Above batch 1
 * the base sum runs on the matrix cores: each input, scaled by a power of two
 * per batch row, enters as two f16 parts whose sum is within 2^-22 of it
 * (relative), multiplied by the exact integer codes, float32 sums per block.
 * x: device float32 batch x k_in; y: device float32 batch x n_out (must not
 * alias x); 1 <= batch <= QBL_MAX_BATCH.  Results are deterministic: the same
 * inputs and list give the same bits. */
qbl_status qbl_linear(qbl_comp* comp, int32_t linear, const float* x, float* y, int32_t batch,
                      void* ws, int64_t ws_bytes, void* stream);

/* qbl_linear for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments, kernels and results (bit for bit) as qbl_linear, but no workspace
 * argument.  The workspace is a library-owned array of 32 MiB per GPU, a
 * file-scope device array that each GPU the library runs on holds until the
 * process ends; a run needing more (qbl_workspace_bytes op 0) returns
 * QBL_E_LIMIT before enqueueing anything.  The call allocates no device or host
 * memory (the first run of an attached list on a stream creates that list's
 * completion event, as every run entry point does).  The first call on a device
 * sets the array up: it looks up the array's device address and enqueues a
 * clear on `stream`; that first call returns QBL_E_STATE on a capturing stream.
 * Every call on a GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (concurrent streams or threads) race
 * on it and must be ordered by the caller.  Capture rules as qbl_linear (batch-1
 * runs with adapters refuse a capturing stream). */
qbl_status qbl_linear_static(qbl_comp* comp, int32_t linear, const float* x, float* y, int32_t batch,
                             void* stream);

/* Per-layer just-in-time path for prefill ([design] sections 1 and 8: for
 * multi-token GEMM, materialise one layer in scratch, use it, discard it):
 *   W_eff = bf16( float32(deq(W)) + sum_i bf16(s_i B_i) bf16(A_i) )    (tile by tile, on chip)
 *   Y = X W_eff^T with float32 accumulation.
 * X: device bfloat16 bit patterns, m x k_in; Y: device float32 m x n_out;
 * q8_0, q4_sm and q4_K bases, low-rank adapters (QBL_E_FORMAT for a list with a
 * sparse delta); m >= 1. */
qbl_status qbl_linear_jit(qbl_comp* comp, int32_t linear, const uint16_t* x_bf16, float* y,
                          int32_t m, void* ws, int64_t ws_bytes, void* stream);

/* One block of linears at batch 1 (linears 7*block .. 7*block+6 = q, k, v, o,
 * gate, up, down), with linear glue between them:
 *   q,k,v = L(x); a = L_o(rms(q+k+v)); g,u = L_gate/up(rms(a));
 *   d = L_down(rms(g+u)); y = rms(d),      rms(v) = v / sqrt(mean(v^2) + 1e-6).
 * x, y: device float32 of the block's width. */
qbl_status qbl_block(qbl_comp* comp, int32_t block, const float* x, float* y, void* ws,
                     int64_t ws_bytes, void* stream);

/* Decode n_tokens tokens through blocks first_block .. first_block+n_blocks-1:
 * token 0 enters with x0, token t+1 with the output of token t.  y_tokens is
 * device float32 n_tokens x width (row t = token t's output).  The list is read
 * once at entry: a concurrent attach does not switch adapters inside one call
 * ([overlay] "Concurrent Safety"). */
qbl_status qbl_decode(qbl_comp* comp, int32_t first_block, int32_t n_blocks, const float* x0,
                      float* y_tokens, int32_t n_tokens, void* ws, int64_t ws_bytes,
                      void* stream);

/* ---------------------------------------------------------- measurement --- */

/* Dequantize-add-requantize of one linear under the composition's current list:
 * the destructive merge that the overlay never performs, offered only to
 * measure its drift ([overlay] "Quantized-Base Numerical Analysis"; [design]
 * "The Pathology of Dequantize-Add-Requantize (DAR) Error").  Writes the
 * canonical blocks of Q(W') to blocks_out (device, at least
 * n_out*k_in/qbl_block_weights*qbl_block_bytes bytes, 2-byte aligned; else
 * QBL_E_BUDGET / QBL_E_ARG), where Q is the base format's quantiser
 * (qbl_quantize) and W' the float32 merged weight
 *   w = f32(deq(W)[n][k]); then for each entry in list order
 *   low-rank: w = fma(s, u, w), u = fma chain over j = 0..rank-1 of B[n][j]*A[j][k]
 *   sparse:   w = fma(s, f32(val), w) at the delta's entries.
 * The base itself is never written.  Asynchronous on stream.  A block whose
 * scale overflows fp16 is written with an infinite scale. */
qbl_status qbl_requantize(qbl_comp* comp, int32_t linear, void* blocks_out, int64_t out_bytes,
                          void* stream);

/* Read-only HBM streaming probe, the achievable read bandwidth as context for
 * the fraction of the nameplate peak: reads the `bytes` bytes at buf (device,
 * 16-byte aligned, bytes a positive multiple of 16) once, with the access of the
 * batch-1 kernels (16-byte non-temporal loads from every lane; workgroup g,
 * thread t reads 16-byte words g*256 + t + i*stride, stride = 256 * workgroups).
 * Workgroup g writes the XOR of the 32-bit words it read to sink[g] (device,
 * sink_words >= 1 words); *workgroups (host) receives the workgroup count,
 * min(sink_words, 8 per compute unit).  Reading every word exactly once makes
 * the XOR of sink[0 .. *workgroups) equal the XOR of the whole buffer (a check
 * for callers: a word read twice would cancel).  Asynchronous on stream;
 * QBL_E_ARG for a null or misaligned pointer or a bad size. */
qbl_status qbl_hbm_probe(const void* buf, int64_t bytes, uint32_t* sink, int32_t sink_words,
                         int32_t* workgroups, void* stream);

/* ------------------------------------------------------------- timing --- */

/* Kernel timing for measurement tools.  While enabled (on != 0), every launch
 * of the library's kernels is bracketed by a pair of HIP events recorded on the
 * launch stream.  Enabling clears earlier records.  qbl_profile_read waits for
 * the recorded events and returns, per kernel kind (0 = batch-1 / batched
 * dequant-GEMV, 1 = glue/shrink prep, 2 = JIT prefill GEMM, 3 = qbl_requantize,
 * 4 = qbl_hbm_probe), the number of launches and their summed duration in
 * milliseconds.  Timing adds host work per launch: leave it off in production. */
qbl_status qbl_profile_enable(int32_t on);
qbl_status qbl_profile_read(int32_t kind, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif
#endif /* QBL_H */
