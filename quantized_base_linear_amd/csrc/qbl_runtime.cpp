// The C ABI of include/qbl.h: immutable bases, refcounted adapters, compositions
// with an atomically replaced adapter list, and the launch planning of the
// decode and prefill paths.
//
// Lifecycle follows "Deep Technical Design: Exact, Atomic, Reversible
// Specialist Overlays", section 6: validate everything first, stage the
// adapter in its own device arena, then commit with one atomic pointer swap;
// deactivation only drops references, the base bytes are never written
// (section 2).  Adapters are bound to the base they were loaded against, as
// the "LoRA adapters" blueprint reports for llama.cpp.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <memory>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/qbl.h"
#include "qbl_host.h"
#include "qbl_kernels.h"

namespace {

thread_local std::string g_err;

qbl_status fail(qbl_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

qbl_status hip_fail(hipError_t e, const char* what) {
  return fail(QBL_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

#define QBL_TRY(...)                                                     \
  try {                                                                  \
    __VA_ARGS__                                                          \
  } catch (const std::bad_alloc&) {                                      \
    return fail(QBL_E_NOMEM, "host allocation failed");                  \
  } catch (...) {                                                        \
    return fail(QBL_E_ARG, "unexpected internal exception");             \
  }

constexpr int64_t kAlign = 256;
int64_t align_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool all_finite(const float* p, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!std::isfinite(p[i])) return false;
  return true;
}

}  // namespace

// ----------------------------------------------------------------- objects ---

struct DevLinear {
  int qtype;
  int64_t n, k;
  uint8_t* qs;
  uint8_t* sc;
  int64_t qs_bytes, sc_bytes;
  void* mem;
  int64_t mem_bytes;
};

struct qbl_base {
  int device = 0;
  std::vector<DevLinear> lin;
  std::atomic<int> refs{0};
  uint8_t digest[32] = {};  // recorded at load from the canonical blocks
  mutable std::mutex mem_mu;  // guards held and budget
  int64_t held = 0;         // device bytes: base arrays + live adapter arenas
  int64_t budget = 0;       // 0 = no cap
};

// One linear of an adapter: a LoRA pair (rank >= 1) or a sparse delta (rank 0).
struct AdEntry {
  int linear;
  int rank;
  float* A;  // device rank x k
  float* B;  // device n x rank
  uint32_t* rp = nullptr;  // sparse: device row_ptr [n+1], col [nnz], fp16 val [nnz]
  uint32_t* ci = nullptr;
  uint16_t* sv = nullptr;
  int64_t nnz = 0;
};

struct AdapterImpl {
  qbl_base* base = nullptr;
  std::vector<AdEntry> ent;
  std::vector<int> slot;  // per base linear: index into ent, or -1
  uint8_t digest[32] = {};
  void* mem = nullptr;
  int64_t reserved = 0;  // bytes counted in base->held
  ~AdapterImpl() {
    if (mem) {
      int cur = 0;
      hipGetDevice(&cur);
      hipSetDevice(base->device);
      hipFree(mem);
      hipSetDevice(cur);
    }
    if (reserved) {
      std::lock_guard<std::mutex> g(base->mem_mu);
      base->held -= reserved;
    }
    if (base) base->refs.fetch_sub(1);
  }
};

struct qbl_adapter {
  std::shared_ptr<AdapterImpl> impl;
};

struct LoraRef {
  const float* A;
  const float* B;
  int rank;  // 0: sparse delta (rp, ci, sv)
  float scale;
  const uint32_t* rp;
  const uint32_t* ci;
  const uint16_t* sv;
  int64_t nnz;
};

// One attached list.  Immutable once published; freed when no composition or
// run holds it, after the work enqueued on every stream that used it is done.
struct ListImpl {
  std::vector<std::shared_ptr<AdapterImpl>> ads;  // effective entries (scale != 0), in order
  std::vector<float> scales;
  std::vector<const AdapterImpl*> in_ads;         // as attached, for the idempotency check
  std::vector<float> in_scales;
  std::vector<std::vector<LoraRef>> plan;         // per linear, in list order
  std::vector<int> total_rank;                    // per linear
  uint8_t digest[32] = {};                        // composition identity
  int device = 0;
  std::mutex ev_mu;
  std::vector<std::pair<hipStream_t, hipEvent_t>> uses;

  void mark_use(hipStream_t st) {
    std::lock_guard<std::mutex> g(ev_mu);
    for (auto& u : uses)
      if (u.first == st) {
        hipEventRecord(u.second, st);
        return;
      }
    // The event only has to tell when the work is done (to free the list's
    // memory), not make device memory visible to the host: without the
    // system-scope fence its record costs no cache writeback on the GPU (with
    // it, ~3 us of every run).
    hipEvent_t ev;
    if (hipEventCreateWithFlags(&ev, hipEventDisableTiming | hipEventDisableSystemFence) == hipSuccess) {
      hipEventRecord(ev, st);
      uses.emplace_back(st, ev);
    } else {
      hipStreamSynchronize(st);  // cannot track: make the use complete now
    }
  }
  // the event that tracks this list's work on st (created on first use)
  hipEvent_t event_for(hipStream_t st) {
    std::lock_guard<std::mutex> g(ev_mu);
    for (auto& u : uses)
      if (u.first == st) return u.second;
    hipEvent_t ev;
    if (hipEventCreateWithFlags(&ev, hipEventDisableTiming | hipEventDisableSystemFence) != hipSuccess) return nullptr;
    uses.emplace_back(st, ev);
    return ev;
  }
  ~ListImpl() {
    for (auto& u : uses) {
      hipEventSynchronize(u.second);
      hipEventDestroy(u.second);
    }
  }
};

// Records, at scope exit, that work enqueued on `st` may read list L, so that
// L (and the adapter memory it holds) outlives that work even when a run
// returns an error after enqueuing part of it.  A run's last launch can carry
// the list's event instead (the launch's stop event, completed with the kernel:
// no separate record between this run's work and the next one's, ~0.8 us of
// every block step); the record at scope exit is then skipped.
struct ListUse {
  ListImpl* L;
  hipStream_t st;
  bool on;
  bool attached = false;
  // Puts the list's event on lc as the stop event of the run's last launch when
  // lc carries no timing event; returns it (nullptr: record at scope exit).
  hipEvent_t attach(qbl::LaunchCtx& lc) {
    if (!on || lc.start || lc.stop) return nullptr;
    lc.stop = L->event_for(st);
    return lc.stop;
  }
  ~ListUse() {
    if (on && !attached) L->mark_use(st);
  }
};

struct qbl_comp {
  qbl_base* base = nullptr;
  std::mutex mu;                   // serialises list changes
  std::shared_ptr<ListImpl> list;  // read and replaced with std::atomic_load / atomic_exchange
  std::shared_ptr<ListImpl> prev;  // the list the last change replaced (under mu)
};

namespace {

void put_le32(uint8_t* p, uint32_t v) {
  for (int i = 0; i < 4; ++i) p[i] = (uint8_t)(v >> (8 * i));
}
void put_le64(uint8_t* p, uint64_t v) {
  for (int i = 0; i < 8; ++i) p[i] = (uint8_t)(v >> (8 * i));
}

// SHA-256 of one linear as a file: 24-byte header, then its canonical blocks.
void linear_digest(int qtype, int64_t n, int64_t k, const void* blocks, int64_t nbytes,
                   uint8_t out[32]) {
  uint8_t hdr[24];
  put_le32(hdr, (uint32_t)qtype);
  put_le32(hdr + 4, 0);
  put_le64(hdr + 8, (uint64_t)n);
  put_le64(hdr + 16, (uint64_t)k);
  qbl::Sha256 h;
  h.update(hdr, sizeof hdr);
  h.update(blocks, (size_t)nbytes);
  h.final(out);
}

// The composition identity over the effective entries (scale != 0).
void identity(const uint8_t base_digest[32], const std::vector<const uint8_t*>& ads,
              const std::vector<float>& scales, uint8_t out[32]) {
  uint8_t w[4];
  qbl::Sha256 h;
  put_le32(w, (uint32_t)QBL_ABI_VERSION);
  h.update(w, 4);
  h.update(base_digest, 32);
  put_le32(w, (uint32_t)ads.size());
  h.update(w, 4);
  for (size_t i = 0; i < ads.size(); ++i) {
    h.update(ads[i], 32);
    uint32_t bits;
    std::memcpy(&bits, &scales[i], 4);
    put_le32(w, bits);
    h.update(w, 4);
  }
  h.final(out);
}

std::shared_ptr<ListImpl> empty_list(const qbl_base* b) {
  auto L = std::make_shared<ListImpl>();
  L->device = b->device;
  L->plan.assign(b->lin.size(), {});
  L->total_rank.assign(b->lin.size(), 0);
  identity(b->digest, {}, {}, L->digest);
  return L;
}

qbl_status check_device(const qbl_base* b) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return fail(QBL_E_DEVICE, "no HIP device");
  if (cur != b->device)
    return fail(QBL_E_ARG, "current HIP device %d is not the base's device %d", cur, b->device);
  return QBL_OK;
}

// -- test-only fault points (qbl_fault_inject) --
constexpr int kFaultPoints = QBL_FAULT_HANDOFF + 1;
std::atomic<int> g_fault[kFaultPoints];

// True once: on the hit that `point` was armed for.
bool fault_fires(int point) {
  int v = g_fault[point].load();
  while (v > 0)
    if (g_fault[point].compare_exchange_weak(v, v - 1)) return v == 1;
  return false;
}

// -- the status word of in-launch hand-offs --
// One word of coherent pinned host memory for the process: a bounded device
// wait that gives up stores 1 into it (see HandoffWait in qbl_device.h).  Host
// code reads it with plain loads, so a run call can refuse while it is set
// without synchronising anything.
struct StatusWord {
  uint32_t* host = nullptr;
  uint32_t* dev = nullptr;
  hipError_t err = hipSuccess;
};

const StatusWord& status_word() {
  static StatusWord w = [] {
    StatusWord s;
    void* h = nullptr;
    s.err = hipHostMalloc(&h, 256, hipHostMallocCoherent | hipHostMallocMapped);
    if (s.err != hipSuccess) return s;
    std::memset(h, 0, 256);
    void* d = nullptr;
    s.err = hipHostGetDevicePointer(&d, h, 0);
    if (s.err != hipSuccess) return s;
    s.host = static_cast<uint32_t*>(h);
    s.dev = static_cast<uint32_t*>(d);
    return s;
  }();
  return w;
}

// QBL_E_DEVICE while a failed hand-off is recorded and not yet read by
// qbl_device_status; QBL_E_NOMEM if the word could not be allocated.
qbl_status check_handoffs() {
  const StatusWord& w = status_word();
  if (!w.host) return fail(QBL_E_NOMEM, "status word: %s", hipGetErrorString(w.err));
  if (__atomic_load_n(w.host, __ATOMIC_ACQUIRE))
    return fail(QBL_E_DEVICE,
                "a device-side wait for a value handed over inside a launch gave up; an earlier run's "
                "outputs are wrong (qbl_device_status reads and clears this)");
  return QBL_OK;
}

// Batch-1 runs with adapters hand values over inside a launch under a number
// fixed when the run is enqueued; a replayed graph would accept the words its
// previous replay left.  Such runs refuse a capturing stream.
qbl_status refuse_capture(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(st, &cs);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  if (cs != hipStreamCaptureStatusNone)
    return fail(QBL_E_STATE,
                "batch-1 runs with adapters hand values over inside a launch under a number fixed at "
                "enqueue and cannot be captured into a HIP graph");
  return QBL_OK;
}

hipError_t dev_alloc(void** p, int64_t bytes) {
  *p = nullptr;
  if (fault_fires(QBL_FAULT_DEVICE_ALLOC)) return hipErrorOutOfMemory;
  return hipMalloc(p, (size_t)bytes);
}

// One host-to-device copy of a staged upload.
struct Part {
  void* dst;
  const void* src;
  int64_t n;
};

// Copies every part to the device, then reads each device copy back and
// compares it byte for byte with its source.  Runs on worker threads, so the
// message goes to *msg instead of the thread's error text.
qbl_status upload_verified(const Part* parts, int np, std::string* msg) {
  for (int i = 0; i < np; ++i) {
    const hipError_t e = hipMemcpy(parts[i].dst, parts[i].src, (size_t)parts[i].n, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      *msg = std::string("upload: ") + hipGetErrorString(e);
      return QBL_E_DEVICE;
    }
  }
  if (np > 0 && parts[0].n > 0 && fault_fires(QBL_FAULT_CORRUPT)) {
    uint8_t* at = static_cast<uint8_t*>(parts[0].dst) + parts[0].n / 2;
    uint8_t byte = 0;
    if (hipMemcpy(&byte, at, 1, hipMemcpyDeviceToHost) == hipSuccess) {
      byte ^= 0x01;
      hipMemcpy(at, &byte, 1, hipMemcpyHostToDevice);
    }
  }
  std::vector<uint8_t> back;
  for (int i = 0; i < np; ++i) {
    back.resize((size_t)parts[i].n);
    const hipError_t e = hipMemcpy(back.data(), parts[i].dst, (size_t)parts[i].n, hipMemcpyDeviceToHost);
    if (e != hipSuccess) {
      *msg = std::string("read-back: ") + hipGetErrorString(e);
      return QBL_E_DEVICE;
    }
    if (std::memcmp(back.data(), parts[i].src, (size_t)parts[i].n) != 0) {
      *msg = "the device copy read back differs from the bytes sent";
      return QBL_E_CHECKSUM;
    }
  }
  return QBL_OK;
}

int loader_threads() { return std::min(qbl::default_threads(), 16); }

}  // namespace

// ------------------------------------------------------------- utilities ---

extern "C" const char* qbl_last_error(void) { return g_err.c_str(); }
extern "C" int32_t qbl_abi_version(void) { return QBL_ABI_VERSION; }
extern "C" int64_t qbl_block_bytes(int32_t qtype) {
  return qtype == QBL_Q8_0 ? 34 : qtype == QBL_Q4_SM ? 20 : qtype == QBL_Q4_K ? 144 : 0;
}
extern "C" int64_t qbl_block_weights(int32_t qtype) {
  return qtype == QBL_Q8_0 || qtype == QBL_Q4_SM ? 32 : qtype == QBL_Q4_K ? 256 : 0;
}

extern "C" qbl_status qbl_sha256(const void* data, int64_t n, uint8_t sha256_out[32]) {
  if ((!data && n) || n < 0 || !sha256_out) return fail(QBL_E_ARG, "bad arguments");
  qbl::Sha256 h;
  h.update(data, (size_t)n);
  h.final(sha256_out);
  return QBL_OK;
}

static qbl_status check_qshape(int32_t qtype, int64_t n, int64_t k) {
  if (!qbl_block_bytes(qtype)) return fail(QBL_E_FORMAT, "unknown quantisation type %d", qtype);
  if (n <= 0 || k <= 0) return fail(QBL_E_SHAPE, "non-positive shape %lld x %lld", (long long)n, (long long)k);
  const int64_t bw = qbl_block_weights(qtype);
  if (k % bw) return fail(QBL_E_FORMAT, "k_in=%lld is not a multiple of %lld", (long long)k, (long long)bw);
  if (k > QBL_MAX_K) return fail(QBL_E_LIMIT, "k_in=%lld above %d", (long long)k, QBL_MAX_K);
  if (n > (int64_t)1 << 30) return fail(QBL_E_LIMIT, "n_out=%lld too large", (long long)n);
  return QBL_OK;
}

extern "C" qbl_status qbl_quantize(int32_t qtype, const float* w, int64_t n, int64_t k,
                                   void* blocks_out, int32_t nthreads) {
  QBL_TRY({
    if (qbl_status s = check_qshape(qtype, n, k)) return s;
    if (!w || !blocks_out) return fail(QBL_E_ARG, "null pointer");
    const int s = qbl::quantize_rows(qtype, w, n, k, static_cast<uint8_t*>(blocks_out), nthreads);
    if (s == QBL_E_NONFINITE) return fail(s, "non-finite weight");
    if (s == QBL_E_LIMIT) return fail(s, "block scale or minimum overflows fp16");
    return QBL_OK;
  })
}

extern "C" qbl_status qbl_dequantize(int32_t qtype, const void* blocks, int64_t n, int64_t k,
                                     float* w_out) {
  QBL_TRY({
    if (qbl_status s = check_qshape(qtype, n, k)) return s;
    if (!blocks || !w_out) return fail(QBL_E_ARG, "null pointer");
    return qbl::dequantize_rows(qtype, static_cast<const uint8_t*>(blocks), n, k, w_out);
  })
}

// ------------------------------------------------------------------ base ---

extern "C" qbl_status qbl_base_load(const qbl_linear_desc* descs, int32_t n_linears,
                                    qbl_base** out) {
  QBL_TRY({
    if (!descs || !out || n_linears <= 0) return fail(QBL_E_ARG, "need descs, out and n_linears >= 1");
    // -- validation
    for (int i = 0; i < n_linears; ++i) {
      const qbl_linear_desc& d = descs[i];
      if (qbl_status s = check_qshape(d.qtype, d.n_out, d.k_in))
        return fail(s, "linear %d: %s", i, qbl_last_error());
      if (d.reserved != 0) return fail(QBL_E_ARG, "linear %d: reserved field must be 0", i);
      if (!d.blocks) return fail(QBL_E_ARG, "linear %d: null blocks", i);
      const int64_t want = d.n_out * (d.k_in / qbl_block_weights(d.qtype)) * qbl_block_bytes(d.qtype);
      if (d.nbytes != want)
        return fail(QBL_E_FORMAT, "linear %d: nbytes %lld, expected %lld", i, (long long)d.nbytes,
                    (long long)want);
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::unique_ptr<qbl_base> b(new qbl_base);
    b->device = dev;
    b->lin.reserve(n_linears);
    auto release = [&]() {
      for (auto& L : b->lin) hipFree(L.mem);
      b->lin.clear();
    };
    // -- allocation: one device arena per linear
    int64_t held = 0;
    for (int i = 0; i < n_linears; ++i) {
      const qbl_linear_desc& d = descs[i];
      DevLinear L{};
      L.qtype = d.qtype;
      L.n = d.n_out;
      L.k = d.k_in;
      L.qs_bytes = qbl::qs_bytes(d.qtype, d.n_out, d.k_in);
      L.sc_bytes = qbl::sc_bytes(d.qtype, d.n_out, d.k_in);
      L.mem_bytes = align_up(L.qs_bytes) + align_up(L.sc_bytes);
      e = dev_alloc(&L.mem, L.mem_bytes);
      if (e != hipSuccess) {
        release();
        return fail(QBL_E_NOMEM, "linear %d: device allocation of %lld bytes: %s", i,
                    (long long)L.mem_bytes, hipGetErrorString(e));
      }
      L.qs = static_cast<uint8_t*>(L.mem);
      L.sc = L.qs + align_up(L.qs_bytes);
      b->lin.push_back(L);
      held += L.mem_bytes;
    }
    // -- staging (repack), upload, verification and digest, linears in parallel
    std::vector<uint8_t> digests((size_t)n_linears * 32);
    std::vector<qbl_status> st((size_t)n_linears, QBL_OK);
    std::vector<std::string> msg((size_t)n_linears);
    qbl::parallel_for(n_linears, loader_threads(), [&](int64_t i) {
      hipSetDevice(dev);
      const qbl_linear_desc& d = descs[i];
      const DevLinear& L = b->lin[(size_t)i];
      linear_digest(d.qtype, d.n_out, d.k_in, d.blocks, d.nbytes, &digests[(size_t)i * 32]);
      std::vector<uint8_t> stage((size_t)L.mem_bytes, 0);
      qbl::repack_rows(d.qtype, static_cast<const uint8_t*>(d.blocks), d.n_out, d.k_in, stage.data(),
                       stage.data() + align_up(L.qs_bytes), 1);
      const Part p{L.mem, stage.data(), L.mem_bytes};
      st[(size_t)i] = upload_verified(&p, 1, &msg[(size_t)i]);
    });
    for (int i = 0; i < n_linears; ++i)
      if (st[(size_t)i] != QBL_OK) {
        release();
        return fail(st[(size_t)i], "linear %d: %s", i, msg[(size_t)i].c_str());
      }
    qbl::Sha256 h;
    h.update(digests.data(), digests.size());
    h.final(b->digest);
    b->held = held;
    *out = b.release();
    return QBL_OK;
  })
}

extern "C" qbl_status qbl_base_count(const qbl_base* base, int32_t* n_linears) {
  if (!base || !n_linears) return fail(QBL_E_ARG, "null pointer");
  *n_linears = (int32_t)base->lin.size();
  return QBL_OK;
}

extern "C" qbl_status qbl_base_info(const qbl_base* base, int32_t linear, int32_t* qtype,
                                    int64_t* n_out, int64_t* k_in) {
  if (!base) return fail(QBL_E_ARG, "null base");
  if (linear < 0 || linear >= (int32_t)base->lin.size()) return fail(QBL_E_ARG, "linear %d out of range", linear);
  const DevLinear& L = base->lin[linear];
  if (qtype) *qtype = L.qtype;
  if (n_out) *n_out = L.n;
  if (k_in) *k_in = L.k;
  return QBL_OK;
}

extern "C" qbl_status qbl_base_digest(const qbl_base* base, uint8_t sha256_out[32]) {
  if (!base || !sha256_out) return fail(QBL_E_ARG, "null pointer");
  std::memcpy(sha256_out, base->digest, 32);
  return QBL_OK;
}

extern "C" qbl_status qbl_base_hash(qbl_base* base, uint8_t sha256_out[32]) {
  QBL_TRY({
    if (!base || !sha256_out) return fail(QBL_E_ARG, "null pointer");
    if (qbl_status s = check_device(base)) return s;
    const int64_t n = (int64_t)base->lin.size();
    std::vector<uint8_t> digests((size_t)n * 32);
    std::vector<int> err((size_t)n, 0);
    qbl::parallel_for(n, loader_threads(), [&](int64_t i) {
      hipSetDevice(base->device);
      const DevLinear& L = base->lin[(size_t)i];
      std::vector<uint8_t> buf((size_t)(L.qs_bytes + L.sc_bytes));
      if (hipMemcpy(buf.data(), L.qs, (size_t)L.qs_bytes, hipMemcpyDeviceToHost) != hipSuccess ||
          hipMemcpy(buf.data() + L.qs_bytes, L.sc, (size_t)L.sc_bytes, hipMemcpyDeviceToHost) !=
              hipSuccess) {
        err[(size_t)i] = 1;
        return;
      }
      const int64_t nbytes = L.n * (L.k / qbl_block_weights(L.qtype)) * qbl_block_bytes(L.qtype);
      std::vector<uint8_t> blocks((size_t)nbytes);
      qbl::unpack_rows(L.qtype, buf.data(), buf.data() + L.qs_bytes, L.n, L.k, blocks.data());
      linear_digest(L.qtype, L.n, L.k, blocks.data(), nbytes, &digests[(size_t)i * 32]);
    });
    for (int x : err)
      if (x) return fail(QBL_E_DEVICE, "reading base bytes back failed");
    qbl::Sha256 h;
    h.update(digests.data(), digests.size());
    h.final(sha256_out);
    return QBL_OK;
  })
}

extern "C" qbl_status qbl_base_set_budget(qbl_base* base, int64_t budget_bytes) {
  if (!base) return fail(QBL_E_ARG, "null base");
  if (budget_bytes < 0) return fail(QBL_E_ARG, "negative budget");
  std::lock_guard<std::mutex> g(base->mem_mu);
  if (budget_bytes > 0 && budget_bytes < base->held)
    return fail(QBL_E_BUDGET, "budget %lld below the %lld bytes already held", (long long)budget_bytes,
                (long long)base->held);
  base->budget = budget_bytes;
  return QBL_OK;
}

extern "C" qbl_status qbl_base_memory(const qbl_base* base, int64_t* held_bytes, int64_t* budget_bytes) {
  if (!base) return fail(QBL_E_ARG, "null base");
  std::lock_guard<std::mutex> g(base->mem_mu);
  if (held_bytes) *held_bytes = base->held;
  if (budget_bytes) *budget_bytes = base->budget;
  return QBL_OK;
}

extern "C" qbl_status qbl_base_free(qbl_base* base) {
  if (!base) return fail(QBL_E_ARG, "null base");
  if (base->refs.load() != 0)
    return fail(QBL_E_BUSY, "base still referenced by %d adapter(s)/composition(s)", base->refs.load());
  int cur = 0;
  hipGetDevice(&cur);
  hipSetDevice(base->device);
  for (auto& L : base->lin) hipFree(L.mem);
  hipSetDevice(cur);
  delete base;
  return QBL_OK;
}

// -------------------------------------------------------------- adapters ---

extern "C" qbl_status qbl_adapter_load(qbl_base* base, const qbl_lora_desc* descs, int32_t n,
                                       qbl_adapter** out) {
  QBL_TRY({
    if (!base || !descs || !out) return fail(QBL_E_ARG, "null pointer");
    if (n <= 0) return fail(QBL_E_ARG, "an adapter must target at least one linear");
    if (qbl_status s = check_device(base)) return s;
    // -- validation: targets, ranks and shapes first, then the values
    const int nl = (int)base->lin.size();
    std::vector<char> seen((size_t)nl, 0);
    int64_t total = 0;
    for (int i = 0; i < n; ++i) {
      const qbl_lora_desc& d = descs[i];
      if (d.linear < 0 || d.linear >= nl)
        return fail(QBL_E_SHAPE, "entry %d targets linear %d; the base has %d", i, d.linear, nl);
      if (seen[(size_t)d.linear]) return fail(QBL_E_DUPLICATE, "linear %d appears twice", d.linear);
      seen[(size_t)d.linear] = 1;
      if (d.rank < 1 || d.rank > QBL_MAX_RANK)
        return fail(QBL_E_LIMIT, "entry %d: rank %d outside 1..%d", i, d.rank, QBL_MAX_RANK);
      if (!d.A || !d.B) return fail(QBL_E_ARG, "entry %d: null factor", i);
      const DevLinear& L = base->lin[(size_t)d.linear];
      total += align_up((int64_t)d.rank * L.k * 4) + align_up(L.n * d.rank * 4);
    }
    std::vector<char> bad((size_t)n, 0);
    qbl::parallel_for(n, loader_threads(), [&](int64_t i) {
      const qbl_lora_desc& d = descs[i];
      const DevLinear& L = base->lin[(size_t)d.linear];
      bad[(size_t)i] = !all_finite(d.A, (int64_t)d.rank * L.k) || !all_finite(d.B, L.n * d.rank);
    });
    for (int i = 0; i < n; ++i)
      if (bad[(size_t)i]) return fail(QBL_E_NONFINITE, "entry %d: non-finite value in A or B", i);
    // -- allocation: reserve the arena within the base's budget, then allocate
    auto impl = std::make_shared<AdapterImpl>();
    impl->base = base;
    base->refs.fetch_add(1);
    {
      std::lock_guard<std::mutex> g(base->mem_mu);
      if (base->budget > 0 && base->held + total > base->budget)
        return fail(QBL_E_BUDGET, "adapter needs %lld bytes; %lld of the budget of %lld are held",
                    (long long)total, (long long)base->held, (long long)base->budget);
      base->held += total;
      impl->reserved = total;
    }
    hipError_t e = dev_alloc(&impl->mem, total);
    if (e != hipSuccess)
      return fail(QBL_E_NOMEM, "device allocation of %lld bytes: %s", (long long)total, hipGetErrorString(e));
    impl->slot.assign((size_t)nl, -1);
    uint8_t* p = static_cast<uint8_t*>(impl->mem);
    for (int i = 0; i < n; ++i) {
      const qbl_lora_desc& d = descs[i];
      const DevLinear& L = base->lin[(size_t)d.linear];
      AdEntry en{d.linear, d.rank, reinterpret_cast<float*>(p), nullptr};
      p += align_up((int64_t)d.rank * L.k * 4);
      en.B = reinterpret_cast<float*>(p);
      p += align_up(L.n * d.rank * 4);
      impl->slot[(size_t)d.linear] = (int)impl->ent.size();
      impl->ent.push_back(en);
    }
    // -- staging, verification and digests, entries in parallel
    std::vector<uint8_t> digests((size_t)n * 32);
    std::vector<qbl_status> st((size_t)n, QBL_OK);
    std::vector<std::string> msg((size_t)n);
    qbl::parallel_for(n, loader_threads(), [&](int64_t i) {
      hipSetDevice(base->device);
      const qbl_lora_desc& d = descs[i];
      const DevLinear& L = base->lin[(size_t)d.linear];
      const AdEntry& en = impl->ent[(size_t)i];
      const int64_t abytes = (int64_t)d.rank * L.k * 4, bbytes = L.n * d.rank * 4;
      uint8_t hdr[8];
      put_le32(hdr, (uint32_t)d.linear);
      put_le32(hdr + 4, (uint32_t)d.rank);
      qbl::Sha256 h;
      h.update(hdr, sizeof hdr);
      h.update(d.A, (size_t)abytes);
      h.update(d.B, (size_t)bbytes);
      h.final(&digests[(size_t)i * 32]);
      const Part parts[2] = {{en.A, d.A, abytes}, {en.B, d.B, bbytes}};
      st[(size_t)i] = upload_verified(parts, 2, &msg[(size_t)i]);
    });
    for (int i = 0; i < n; ++i)
      if (st[(size_t)i] != QBL_OK)  // impl frees its arena and its reservation
        return fail(st[(size_t)i], "entry %d: %s", i, msg[(size_t)i].c_str());
    qbl::Sha256 h;
    h.update(digests.data(), digests.size());
    h.final(impl->digest);
    auto* a = new qbl_adapter;
    a->impl = std::move(impl);
    *out = a;
    return QBL_OK;
  })
}

namespace {

// The deep checks of one sparse entry ([design] section 11: strictly monotonic
// indices, finite f16 payloads, dimensions that match).
qbl_status check_sparse(const qbl_sparse_desc& d, int64_t n, int64_t k, int i) {
  if (!d.row_ptr) return fail(QBL_E_ARG, "entry %d: null row_ptr", i);
  if (d.nnz < 0 || d.nnz > n * k || d.nnz > (int64_t)UINT32_MAX)
    return fail(QBL_E_SHAPE, "entry %d: %lld entries for a %lld x %lld linear", i, (long long)d.nnz,
                (long long)n, (long long)k);
  if (d.nnz > 0 && (!d.col || !d.val)) return fail(QBL_E_ARG, "entry %d: null col or val", i);
  if (d.reserved != 0) return fail(QBL_E_ARG, "entry %d: reserved field must be 0", i);
  if (d.row_ptr[0] != 0 || (int64_t)d.row_ptr[n] != d.nnz)
    return fail(QBL_E_SHAPE, "entry %d: row_ptr must run from 0 to nnz", i);
  // row_ptr first, so that the column pass below never reads past nnz
  for (int64_t r = 0; r < n; ++r)
    if (d.row_ptr[r + 1] < d.row_ptr[r])
      return fail(QBL_E_SHAPE, "entry %d: row_ptr decreases at row %lld", i, (long long)r);
  for (int64_t r = 0; r < n; ++r) {
    const uint32_t p0 = d.row_ptr[r], p1 = d.row_ptr[r + 1];
    for (uint32_t p = p0; p < p1; ++p) {
      if ((int64_t)d.col[p] >= k)
        return fail(QBL_E_SHAPE, "entry %d: column %u of row %lld outside 0..%lld", i, d.col[p],
                    (long long)r, (long long)k - 1);
      if (p > p0 && d.col[p] <= d.col[p - 1])
        return fail(QBL_E_FORMAT, "entry %d: columns of row %lld not strictly increasing", i, (long long)r);
    }
  }
  for (int64_t p = 0; p < d.nnz; ++p)
    if ((d.val[p] & 0x7C00u) == 0x7C00u) return fail(QBL_E_NONFINITE, "entry %d: value %lld is not finite", i, (long long)p);
  return QBL_OK;
}

}  // namespace

extern "C" qbl_status qbl_adapter_load_sparse(qbl_base* base, const qbl_sparse_desc* descs, int32_t n,
                                              qbl_adapter** out) {
  QBL_TRY({
    if (!base || !descs || !out) return fail(QBL_E_ARG, "null pointer");
    if (n <= 0) return fail(QBL_E_ARG, "an adapter must target at least one linear");
    if (qbl_status s = check_device(base)) return s;
    // -- validation
    const int nl = (int)base->lin.size();
    std::vector<char> seen((size_t)nl, 0);
    int64_t total = 0;
    for (int i = 0; i < n; ++i) {
      const qbl_sparse_desc& d = descs[i];
      if (d.linear < 0 || d.linear >= nl)
        return fail(QBL_E_SHAPE, "entry %d targets linear %d; the base has %d", i, d.linear, nl);
      if (seen[(size_t)d.linear]) return fail(QBL_E_DUPLICATE, "linear %d appears twice", d.linear);
      seen[(size_t)d.linear] = 1;
      const DevLinear& L = base->lin[(size_t)d.linear];
      if (qbl_status s = check_sparse(d, L.n, L.k, i)) return s;
      total += align_up(4 * (L.n + 1)) + align_up(4 * d.nnz) + align_up(2 * d.nnz);
    }
    // -- allocation within the budget
    auto impl = std::make_shared<AdapterImpl>();
    impl->base = base;
    base->refs.fetch_add(1);
    {
      std::lock_guard<std::mutex> g(base->mem_mu);
      if (base->budget > 0 && base->held + total > base->budget)
        return fail(QBL_E_BUDGET, "adapter needs %lld bytes; %lld of the budget of %lld are held",
                    (long long)total, (long long)base->held, (long long)base->budget);
      base->held += total;
      impl->reserved = total;
    }
    hipError_t e = dev_alloc(&impl->mem, total);
    if (e != hipSuccess)
      return fail(QBL_E_NOMEM, "device allocation of %lld bytes: %s", (long long)total, hipGetErrorString(e));
    impl->slot.assign((size_t)nl, -1);
    uint8_t* p = static_cast<uint8_t*>(impl->mem);
    for (int i = 0; i < n; ++i) {
      const qbl_sparse_desc& d = descs[i];
      const DevLinear& L = base->lin[(size_t)d.linear];
      AdEntry en{d.linear, 0, nullptr, nullptr};
      en.nnz = d.nnz;
      en.rp = reinterpret_cast<uint32_t*>(p);
      p += align_up(4 * (L.n + 1));
      en.ci = reinterpret_cast<uint32_t*>(p);
      p += align_up(4 * d.nnz);
      en.sv = reinterpret_cast<uint16_t*>(p);
      p += align_up(2 * d.nnz);
      impl->slot[(size_t)d.linear] = (int)impl->ent.size();
      impl->ent.push_back(en);
    }
    // -- staging, verification and digests
    std::vector<uint8_t> digests((size_t)n * 32);
    std::vector<qbl_status> st((size_t)n, QBL_OK);
    std::vector<std::string> msg((size_t)n);
    qbl::parallel_for(n, loader_threads(), [&](int64_t i) {
      hipSetDevice(base->device);
      const qbl_sparse_desc& d = descs[i];
      const DevLinear& L = base->lin[(size_t)d.linear];
      const AdEntry& en = impl->ent[(size_t)i];
      uint8_t hdr[16];
      put_le32(hdr, (uint32_t)d.linear);
      put_le32(hdr + 4, 0xFFFFFFFFu);
      put_le64(hdr + 8, (uint64_t)d.nnz);
      qbl::Sha256 h;
      h.update(hdr, sizeof hdr);
      h.update(d.row_ptr, (size_t)(4 * (L.n + 1)));
      if (d.nnz) {
        h.update(d.col, (size_t)(4 * d.nnz));
        h.update(d.val, (size_t)(2 * d.nnz));
      }
      h.final(&digests[(size_t)i * 32]);
      const Part parts[3] = {{en.rp, d.row_ptr, 4 * (L.n + 1)}, {en.ci, d.col, 4 * d.nnz}, {en.sv, d.val, 2 * d.nnz}};
      st[(size_t)i] = upload_verified(parts, d.nnz ? 3 : 1, &msg[(size_t)i]);
    });
    for (int i = 0; i < n; ++i)
      if (st[(size_t)i] != QBL_OK) return fail(st[(size_t)i], "entry %d: %s", i, msg[(size_t)i].c_str());
    qbl::Sha256 h;
    h.update(digests.data(), digests.size());
    h.final(impl->digest);
    auto* a = new qbl_adapter;
    a->impl = std::move(impl);
    *out = a;
    return QBL_OK;
  })
}

extern "C" qbl_status qbl_adapter_digest(const qbl_adapter* adapter, uint8_t sha256_out[32]) {
  if (!adapter || !sha256_out) return fail(QBL_E_ARG, "null pointer");
  std::memcpy(sha256_out, adapter->impl->digest, 32);
  return QBL_OK;
}

extern "C" qbl_status qbl_adapter_free(qbl_adapter* adapter) {
  if (!adapter) return fail(QBL_E_ARG, "null adapter");
  delete adapter;  // the attached lists keep their own references
  return QBL_OK;
}

// ---------------------------------------------------------- compositions ---

namespace {

// The exchange of a list change (comp->mu held): the new list becomes current
// in one atomic step and the replaced one is kept as the previous list.
qbl_status swap_in(qbl_comp* comp, std::shared_ptr<ListImpl> L) {
  if (fault_fires(QBL_FAULT_SWAP)) return fail(QBL_E_INJECTED, "injected failure before the exchange");
  comp->prev = std::atomic_exchange(&comp->list, std::move(L));
  return QBL_OK;
}

}  // namespace

extern "C" qbl_status qbl_comp_create(qbl_base* base, qbl_comp** out) {
  QBL_TRY({
    if (!base || !out) return fail(QBL_E_ARG, "null pointer");
    auto* c = new qbl_comp;
    c->base = base;
    std::atomic_store(&c->list, empty_list(base));
    base->refs.fetch_add(1);
    *out = c;
    return QBL_OK;
  })
}

extern "C" qbl_status qbl_comp_attach(qbl_comp* comp, const qbl_adapter* const* list,
                                      const float* scales, int32_t n) {
  QBL_TRY({
    if (!comp) return fail(QBL_E_ARG, "null composition");
    if (n < 0 || n > QBL_MAX_ADAPTERS) return fail(QBL_E_LIMIT, "list of %d adapters; at most %d", n, QBL_MAX_ADAPTERS);
    if (n > 0 && (!list || !scales)) return fail(QBL_E_ARG, "null list or scales");
    const qbl_base* base = comp->base;
    const size_t nl = base->lin.size();
    // -- validation: nothing changes unless every check passes
    for (int i = 0; i < n; ++i) {
      if (!list[i]) return fail(QBL_E_ARG, "entry %d is null", i);
      if (list[i]->impl->base != base) return fail(QBL_E_FOREIGN, "entry %d belongs to another base", i);
      if (!std::isfinite(scales[i])) return fail(QBL_E_NONFINITE, "scale %d is not finite", i);
      for (int j = 0; j < i; ++j)
        if (list[j] == list[i] || list[j]->impl == list[i]->impl)
          return fail(QBL_E_DUPLICATE, "entries %d and %d are the same adapter", j, i);
    }
    std::vector<int> rank_sum(nl, 0);
    for (int i = 0; i < n; ++i) {
      if (scales[i] == 0.0f) continue;
      for (const AdEntry& e : list[i]->impl->ent) rank_sum[(size_t)e.linear] += e.rank;
    }
    for (size_t l = 0; l < nl; ++l)
      if (rank_sum[l] > QBL_MAX_TOTAL_RANK)
        return fail(QBL_E_LIMIT, "linear %zu: summed rank %d above %d", l, rank_sum[l], QBL_MAX_TOTAL_RANK);

    std::lock_guard<std::mutex> g(comp->mu);
    // -- idempotency: the same list and scales already in place
    {
      auto cur = std::atomic_load(&comp->list);
      bool same = (int)cur->in_ads.size() == n;
      for (int i = 0; same && i < n; ++i)
        same = cur->in_ads[(size_t)i] == list[i]->impl.get() && cur->in_scales[(size_t)i] == scales[i];
      if (same) return QBL_OK;
    }
    // -- staging: build the new immutable list and its identity
    auto L = empty_list(base);
    std::vector<const uint8_t*> eff_digests;
    for (int i = 0; i < n; ++i) {
      L->in_ads.push_back(list[i]->impl.get());
      L->in_scales.push_back(scales[i]);
      if (scales[i] == 0.0f) continue;  // a zero-scale entry contributes nothing
      L->ads.push_back(list[i]->impl);
      L->scales.push_back(scales[i]);
      eff_digests.push_back(list[i]->impl->digest);
      for (const AdEntry& e : list[i]->impl->ent) {
        L->plan[(size_t)e.linear].push_back(LoraRef{e.A, e.B, e.rank, scales[i], e.rp, e.ci, e.sv, e.nnz});
        L->total_rank[(size_t)e.linear] += e.rank;
      }
    }
    identity(base->digest, eff_digests, L->scales, L->digest);
    // zero-scale entries are compared by address in the idempotency check, so
    // hold them as well
    for (int i = 0; i < n; ++i)
      if (scales[i] == 0.0f) L->ads.push_back(list[i]->impl);
    // -- commit: one atomic exchange; the old list retires when its last user drops it
    return swap_in(comp, std::move(L));
  })
}

extern "C" qbl_status qbl_comp_clear(qbl_comp* comp) {
  QBL_TRY({
    if (!comp) return fail(QBL_E_ARG, "null composition");
    std::lock_guard<std::mutex> g(comp->mu);
    if (std::atomic_load(&comp->list)->in_ads.empty()) return QBL_OK;
    return swap_in(comp, empty_list(comp->base));
  })
}

extern "C" qbl_status qbl_comp_rollback(qbl_comp* comp) {
  QBL_TRY({
    if (!comp) return fail(QBL_E_ARG, "null composition");
    std::lock_guard<std::mutex> g(comp->mu);
    if (!comp->prev) return fail(QBL_E_STATE, "no previous list to return to");
    std::shared_ptr<ListImpl> back = comp->prev;
    return swap_in(comp, std::move(back));
  })
}

extern "C" qbl_status qbl_comp_drop_previous(qbl_comp* comp) {
  QBL_TRY({
    if (!comp) return fail(QBL_E_ARG, "null composition");
    std::shared_ptr<ListImpl> old;
    {
      std::lock_guard<std::mutex> g(comp->mu);
      old.swap(comp->prev);
    }
    return QBL_OK;  // `old` retires here, after the work that used it
  })
}

extern "C" qbl_status qbl_comp_count(const qbl_comp* comp, int32_t* n) {
  if (!comp || !n) return fail(QBL_E_ARG, "null pointer");
  *n = (int32_t)std::atomic_load(&comp->list)->scales.size();
  return QBL_OK;
}

extern "C" qbl_status qbl_comp_digest(const qbl_comp* comp, uint8_t sha256_out[32]) {
  if (!comp || !sha256_out) return fail(QBL_E_ARG, "null pointer");
  std::memcpy(sha256_out, std::atomic_load(&comp->list)->digest, 32);
  return QBL_OK;
}

extern "C" qbl_status qbl_identity_digest(const uint8_t base_digest[32], const uint8_t* adapter_digests,
                                          const float* scales, int32_t n, uint8_t sha256_out[32]) {
  QBL_TRY({
    if (!base_digest || !sha256_out) return fail(QBL_E_ARG, "null pointer");
    if (n < 0 || n > QBL_MAX_ADAPTERS) return fail(QBL_E_LIMIT, "list of %d adapters; at most %d", n, QBL_MAX_ADAPTERS);
    if (n > 0 && (!adapter_digests || !scales)) return fail(QBL_E_ARG, "null digests or scales");
    std::vector<const uint8_t*> ads;
    std::vector<float> sc;
    for (int i = 0; i < n; ++i) {
      if (!std::isfinite(scales[i])) return fail(QBL_E_NONFINITE, "scale %d is not finite", i);
      if (scales[i] == 0.0f) continue;
      ads.push_back(adapter_digests + 32 * i);
      sc.push_back(scales[i]);
    }
    identity(base_digest, ads, sc, sha256_out);
    return QBL_OK;
  })
}

extern "C" qbl_status qbl_comp_free(qbl_comp* comp) {
  if (!comp) return fail(QBL_E_ARG, "null composition");
  {
    std::lock_guard<std::mutex> g(comp->mu);
    std::atomic_store(&comp->list, std::shared_ptr<ListImpl>());
    comp->prev.reset();
  }
  comp->base->refs.fetch_sub(1);
  delete comp;
  return QBL_OK;
}

extern "C" qbl_status qbl_device_status(void) {
  QBL_TRY({
    const StatusWord& w = status_word();
    if (!w.host) return fail(QBL_E_NOMEM, "status word: %s", hipGetErrorString(w.err));
    if (__atomic_exchange_n(w.host, 0u, __ATOMIC_ACQ_REL))
      return fail(QBL_E_DEVICE, "a device-side wait for a value handed over inside a launch gave up");
    return QBL_OK;
  })
}

extern "C" qbl_status qbl_fault_inject(int32_t point, int32_t after) {
  if (point < 1 || point >= kFaultPoints) return fail(QBL_E_ARG, "unknown fault point %d", point);
  if (after < 0) return fail(QBL_E_ARG, "negative count");
  g_fault[point].store(after);
  return QBL_OK;
}

// ---------------------------------------------------------------- timing ---

namespace {

struct Profiler {
  struct Rec {
    int kind;
    hipEvent_t a, b;
  };
  std::mutex mu;
  std::atomic<bool> on{false};
  std::vector<Rec> recs;
};

Profiler& profiler() {
  static Profiler p;
  return p;
}

// Timing events for one kernel launch while timing is enabled: they ride on the
// dispatch itself, so they measure the kernel, not the queue around it.
class KernelTimer {
 public:
  KernelTimer(int kind, hipStream_t st) : kind_(kind) {
    ctx_.stream = st;
    if (!profiler().on.load()) return;
    if (hipEventCreate(&a_) != hipSuccess || hipEventCreate(&b_) != hipSuccess) return;
    ctx_.start = a_;
    ctx_.stop = b_;
  }
  const qbl::LaunchCtx& ctx() const { return ctx_; }
  void stop() {
    if (!a_ || !b_) return;
    Profiler& p = profiler();
    std::lock_guard<std::mutex> g(p.mu);
    p.recs.push_back(Profiler::Rec{kind_, a_, b_});
    a_ = b_ = nullptr;
  }
  ~KernelTimer() {
    if (a_) hipEventDestroy(a_);
    if (b_) hipEventDestroy(b_);
  }

 private:
  int kind_;
  qbl::LaunchCtx ctx_;
  hipEvent_t a_ = nullptr, b_ = nullptr;
};

void clear_records(Profiler& p) {
  for (auto& r : p.recs) {
    hipEventSynchronize(r.b);
    hipEventDestroy(r.a);
    hipEventDestroy(r.b);
  }
  p.recs.clear();
}

}  // namespace

extern "C" qbl_status qbl_profile_enable(int32_t on) {
  QBL_TRY({
    Profiler& p = profiler();
    std::lock_guard<std::mutex> g(p.mu);
    clear_records(p);
    p.on.store(on != 0);
    return QBL_OK;
  })
}

extern "C" qbl_status qbl_profile_read(int32_t kind, int64_t* launches, double* total_ms) {
  QBL_TRY({
    if (!launches || !total_ms) return fail(QBL_E_ARG, "null pointer");
    Profiler& p = profiler();
    std::lock_guard<std::mutex> g(p.mu);
    int64_t n = 0;
    double ms = 0.0;
    for (auto& r : p.recs) {
      if (r.kind != kind) continue;
      hipError_t e = hipEventSynchronize(r.b);
      float t = 0.0f;
      if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
      if (e != hipSuccess) return hip_fail(e, "reading timing events");
      ++n;
      ms += t;
    }
    *launches = n;
    *total_ms = ms;
    return QBL_OK;
  })
}

// ------------------------------------------------------------------ runs ---

namespace {

struct Block {
  int first;  // linear index of q
  int64_t d, h;
};

qbl_status block_shape(const qbl_base* b, int blk, Block* out) {
  const int first = 7 * blk;
  if (blk < 0 || first + 7 > (int)b->lin.size())
    return fail(QBL_E_ARG, "block %d needs linears %d..%d; the base has %zu", blk, first, first + 6,
                b->lin.size());
  const DevLinear* L = &b->lin[(size_t)first];
  const int64_t d = L[0].k, h = L[4].n;
  for (int i = 0; i < 4; ++i)
    if (L[i].n != d || L[i].k != d) return fail(QBL_E_SHAPE, "block %d: q/k/v/o must be d x d", blk);
  if (L[4].k != d || L[5].n != h || L[5].k != d || L[6].n != d || L[6].k != h)
    return fail(QBL_E_SHAPE, "block %d: gate/up must be h x d and down d x h", blk);
  *out = Block{first, d, h};
  return QBL_OK;
}

// Layout of the block/decode workspace (floats, 256-byte aligned pieces).
struct BlockWs {
  float *xin, *t, *q, *k, *v, *a, *g, *u, *dd;
  uint64_t* sp;
  int64_t bytes;
};

BlockWs block_ws(void* ws, int64_t d, int64_t h, int64_t tmax, int64_t spmax) {
  BlockWs w{};
  int64_t off = 0;
  auto take = [&](int64_t floats) {
    float* p = ws ? reinterpret_cast<float*>(static_cast<char*>(ws) + off) : nullptr;
    off += align_up(floats * 4);
    return p;
  };
  const int64_t m = std::max(d, h);
  w.xin = take(m);
  w.t = take(std::max<int64_t>(2 * qbl::kTCopies * qbl::t_copy_stride(tmax), tmax));  // tagged 8-byte words
  w.sp = reinterpret_cast<uint64_t*>(take(2 * spmax));  // tagged 8-byte words
  w.q = take(d);
  w.k = take(d);
  w.v = take(d);
  w.a = take(d);
  w.g = take(h);
  w.u = take(h);
  w.dd = take(d);
  w.bytes = off;
  return w;
}

// Sparse (linear, adapter, row) items of a launch group: the rows of every
// sparse delta on its linears.
int64_t group_sp_items(const qbl_base* base, const ListImpl* L, const int* lin, int nlin) {
  int64_t n = 0;
  for (int i = 0; i < nlin; ++i)
    for (const LoraRef& r : L->plan[(size_t)lin[i]])
      if (r.rank == 0) n += base->lin[(size_t)lin[i]].n;
  return n;
}

// Max sparse items over the four launch groups of every block in range.
int64_t blocks_spmax(const qbl_base* base, const ListImpl* L, int first_block, int n_blocks) {
  int64_t m = 0;
  for (int b = first_block; b < first_block + n_blocks; ++b) {
    const int f = 7 * b;
    const int g0[3] = {f, f + 1, f + 2}, g1[1] = {f + 3}, g2[2] = {f + 4, f + 5}, g3[1] = {f + 6};
    m = std::max({m, group_sp_items(base, L, g0, 3), group_sp_items(base, L, g1, 1),
                  group_sp_items(base, L, g2, 2), group_sp_items(base, L, g3, 1)});
  }
  return m;
}

// True when some linear of the blocks in range has an adapter entry.
bool blocks_have_entries(const ListImpl* L, int first_block, int n_blocks) {
  for (int i = 7 * first_block; i < 7 * (first_block + n_blocks); ++i)
    if (!L->plan[(size_t)i].empty()) return true;
  return false;
}

int group_rank(const ListImpl* L, const int* lin, int nlin) {
  int t = 0;
  for (int i = 0; i < nlin; ++i) t += L->total_rank[(size_t)lin[i]];
  return t;
}

// Max shrink width over the four launch groups of every block in range.
int blocks_tmax(const ListImpl* L, int first_block, int n_blocks) {
  int tmax = 0;
  for (int b = first_block; b < first_block + n_blocks; ++b) {
    const int f = 7 * b;
    const int g0[3] = {f, f + 1, f + 2}, g1[1] = {f + 3}, g2[2] = {f + 4, f + 5}, g3[1] = {f + 6};
    tmax = std::max({tmax, group_rank(L, g0, 3), group_rank(L, g1, 1), group_rank(L, g2, 2),
                     group_rank(L, g3, 1)});
  }
  return tmax;
}

// One launch group: linears sharing one input.  Input = c * (v0 + v1 + v2) with
// c the RMS scale when rms != 0.  At batch 1 the glue, the shrink and the GEMV
// share one launch (the shrink results pass through t_buf as tagged words);
// otherwise the prep kernel (glue and/or shrink) runs first, then one GEMV per
// quantisation type present: at batch 2..8 the matrix-core GEMV, which stages
// its inputs in `stage` first.
// Wall-clock budget (100 MHz ticks) of one thread's waits for handed-over
// values within a launch: 50 ms, far above any legitimate wait (a few us).
constexpr int64_t kWaitTicks = 5000000;

// Numbers that tag the shrink results one workgroup hands to others within a
// launch: unique per launch (mod 2^32), never 0, so a zeroed workspace holds
// no valid value.
uint32_t next_tag() {
  static std::atomic<uint32_t> counter{0};
  uint32_t t = counter.fetch_add(1, std::memory_order_relaxed) + 1;
  while (t == 0) t = counter.fetch_add(1, std::memory_order_relaxed) + 1;
  return t;
}

qbl_status run_group(const qbl_base* base, const ListImpl* L, const int* lin, float* const* outs,
                     int nlin, const float* const* vin, int nv, int rms, int batch, int64_t v_stride,
                     float* xin_buf, float* t_buf, uint64_t* sp_buf, hipStream_t st, bool sum_ok = false,
                     bool* summed = nullptr, void* stage = nullptr, ListUse* last = nullptr) {
  if (summed) *summed = false;
  const int64_t K = base->lin[(size_t)lin[0]].k;
  int T = 0;
  qbl::PrepEntry ent[qbl::kMaxPrepEntries];
  int n_ent = 0;
  for (int i = 0; i < nlin; ++i) {
    for (const LoraRef& r : L->plan[(size_t)lin[i]]) {
      if (r.rank == 0) continue;  // a sparse delta has no shrink
      ent[n_ent++] = qbl::PrepEntry{r.A, r.rank, T};
      T += r.rank;
    }
  }
  bool same_type = true;
  for (int i = 1; i < nlin; ++i) same_type &= base->lin[(size_t)lin[i]].qtype == base->lin[(size_t)lin[0]].qtype;

  int has_sparse = 0;
  auto fill_segments = [&](qbl::GemvArgs& a, int qt) {
    int toff = 0;
    for (int i = 0; i < nlin; ++i) {
      const DevLinear& D = base->lin[(size_t)lin[i]];
      const int this_rank = L->total_rank[(size_t)lin[i]];
      if (D.qtype != qt) {
        toff += this_rank;
        continue;
      }
      qbl::GemvSeg& s = a.seg[a.nseg++];
      s.qs = D.qs;
      s.sc = D.sc;
      s.y = outs[i];
      s.y_stride = D.n;
      s.n = (int)D.n;
      int o = toff;
      for (const LoraRef& r : L->plan[(size_t)lin[i]]) {
        const int j = s.lora.n_ad++;
        s.lora.toff[j] = o;
        s.lora.rank[j] = r.rank;
        s.lora.scale[j] = r.scale;
        s.lora.B[j] = r.B;
        s.lora.rp[j] = r.rp;
        s.lora.ci[j] = r.ci;
        s.lora.sv[j] = r.sv;
        has_sparse |= r.rank == 0;
        o += r.rank;
      }
      toff += this_rank;
    }
  };

  const int qt0 = base->lin[(size_t)lin[0]].qtype;
  // the fused batch-1 launch takes a single input vector; the sum of several
  // (q, k and v written apart) goes through the prep + GEMV path
  if (batch == 1 && nv == 1 && same_type && qbl::fused_supported(qt0, (int)K) &&
      (T == 0 || t_buf) && v_stride == K) {
    qbl::FusedArgs f{};
    fill_segments(f.g, qt0);
    f.g.qtype = qt0;
    f.g.k = (int)K;
    f.g.batch = 1;
    for (int i = 0; i < nv; ++i) f.v[i] = vin[i];
    f.nv = nv;
    f.rms = rms;
    f.sum = sum_ok && nlin > 1;
    f.n_ent = n_ent;
    for (int i = 0; i < n_ent; ++i) f.ent[i] = ent[i];
    f.rows_total = T;
    f.has_sparse = has_sparse;
    // sparse items: the rows of each (linear, sparse adapter), in segment and list order
    for (int i = 0; i < f.g.nseg; ++i) {
      int j = 0;
      for (const LoraRef& r : L->plan[(size_t)lin[i]]) {
        f.sp_base[i][j] = -1;
        if (r.rank == 0) {
          f.sp_base[i][j] = f.sp_items;
          f.sp_items += f.g.seg[i].n;
          f.sp_bytes += r.nnz * 6 + ((int64_t)f.g.seg[i].n + 1) * 4;
        }
        ++j;
      }
    }
    if (f.sp_items > 0 && !sp_buf) return fail(QBL_E_ARG, "the workspace has no room for the sparse values");
    f.sp = sp_buf;
    f.tag = next_tag();
    f.read_tag = f.tag;
    f.wait_ticks = kWaitTicks;
    f.fail = status_word().dev;
    if ((T > 0 || f.sp_items > 0) && fault_fires(QBL_FAULT_HANDOFF)) {
      // readers wait for a number no writer stores, with no budget: every wait
      // gives up at once and records the failure
      f.read_tag = f.tag ^ 0x5A5A5A5Au;
      f.wait_ticks = 0;
    }
    f.t = reinterpret_cast<uint64_t*>(t_buf);
    f.t_copy_stride = qbl::t_copy_stride(T);
    KernelTimer tm(0, st);
    qbl::LaunchCtx lc = tm.ctx();
    const hipEvent_t done = last ? last->attach(lc) : nullptr;
    hipError_t e = qbl::launch_fused(f, lc);
    if (e != hipSuccess) return hip_fail(e, "fused gemv launch");
    if (done) last->attached = true;
    tm.stop();
    if (summed) *summed = f.sum != 0;
    return QBL_OK;
  }

  qbl::PrepArgs p{};
  for (int i = 0; i < n_ent; ++i) p.ent[i] = ent[i];
  p.n_ent = n_ent;
  const bool glue = rms || nv > 1;
  const float* x = vin[0];
  if (batch > 1 && glue) return fail(QBL_E_ARG, "input glue runs at batch 1 only");
  if (batch == 1 && (glue || T > 0)) {
    for (int i = 0; i < nv; ++i) p.v[i] = vin[i];
    p.nv = nv;
    p.rms = rms;
    p.batch = batch;
    p.k = (int)K;
    p.v_stride = v_stride;
    p.xin = glue ? xin_buf : nullptr;
    p.t = T > 0 ? t_buf : nullptr;
    p.T = T;
    p.rows_total = T;
    KernelTimer tm(1, st);
    hipError_t e = qbl::launch_prep(p, tm.ctx());
    if (e != hipSuccess) return hip_fail(e, "prep launch");
    tm.stop();
    if (glue) x = xin_buf;
  }
  int launched = 0;  // linears given to a GEMV launch: all of them, or an error
  for (int qt = QBL_Q8_0; qt <= QBL_Q4_K; ++qt) {
    qbl::GemvArgs a{};
    fill_segments(a, qt);
    if (!a.nseg) continue;
    launched += a.nseg;
    a.qtype = qt;
    a.k = (int)K;
    a.batch = batch;
    a.x = x;
    a.x_stride = glue ? K : v_stride;
    a.t = T > 0 ? t_buf : nullptr;
    a.t_stride = T;
    if (batch > 1) {
      if (!stage) return fail(QBL_E_ARG, "the batched GEMV needs a staging buffer");
      KernelTimer ts(1, st);
      KernelTimer tm(0, st);
      qbl::LaunchCtx lc = tm.ctx();
      // the list's event rides on this group's last kernel when it is the run's last
      const hipEvent_t done = last && launched == nlin ? last->attach(lc) : nullptr;
      hipError_t e = qbl::launch_gemv_mfma(a, ent, n_ent, T, stage, 0, ts.ctx(), lc);
      if (e != hipSuccess) return hip_fail(e, "batched gemv launch");
      if (done) last->attached = true;
      ts.stop();
      tm.stop();
      continue;
    }
    KernelTimer tm(0, st);
    hipError_t e = qbl::launch_gemv(a, tm.ctx());
    if (e != hipSuccess) return hip_fail(e, "gemv launch");
    tm.stop();
  }
  if (launched != nlin) return fail(QBL_E_FORMAT, "a linear of an unsupported type got no GEMV launch");
  return QBL_OK;
}

// rms of one vector into y (a prep launch with no adapter rows)
qbl_status run_rms(const float* v, int64_t n, float* y, hipStream_t st, ListUse* last = nullptr) {
  KernelTimer tm(1, st);
  qbl::LaunchCtx lc = tm.ctx();
  const hipEvent_t done = last ? last->attach(lc) : nullptr;
  hipError_t e = qbl::launch_rms(v, (int)n, y, lc);
  if (e != hipSuccess) return hip_fail(e, "rms launch");
  if (done) last->attached = true;
  tm.stop();
  return QBL_OK;
}

// One block; `in` is either a plain input (rms_in = 0) or the previous block's
// down output that still needs its RMS scale (rms_in = 1).  Leaves d in w.dd.
qbl_status run_block(const qbl_base* base, const ListImpl* L, const Block& B, const float* in,
                     int rms_in, const BlockWs& w, hipStream_t st) {
  const int f = B.first;
  // At batch 1 the parallel projections can be written as their sum (all the
  // glue needs); then the next group reads one vector instead of three or two.
  bool summed = false;
  {
    const int lin[3] = {f, f + 1, f + 2};
    float* outs[3] = {w.q, w.k, w.v};
    const float* v[1] = {in};
    if (qbl_status s = run_group(base, L, lin, outs, 3, v, 1, rms_in, 1, B.d, w.xin, w.t, w.sp, st, true, &summed))
      return s;
  }
  {
    const int lin[1] = {f + 3};
    float* outs[1] = {w.a};
    const float* v[3] = {w.q, w.k, w.v};
    if (qbl_status s = run_group(base, L, lin, outs, 1, v, summed ? 1 : 3, 1, 1, B.d, w.xin, w.t, w.sp, st)) return s;
  }
  {
    const int lin[2] = {f + 4, f + 5};
    float* outs[2] = {w.g, w.u};
    const float* v[1] = {w.a};
    if (qbl_status s = run_group(base, L, lin, outs, 2, v, 1, 1, 1, B.d, w.xin, w.t, w.sp, st, true, &summed))
      return s;
  }
  {
    const int lin[1] = {f + 6};
    float* outs[1] = {w.dd};
    const float* v[2] = {w.g, w.u};
    if (qbl_status s = run_group(base, L, lin, outs, 1, v, summed ? 1 : 2, 1, 1, B.h, w.xin, w.t, w.sp, st)) return s;
  }
  return QBL_OK;
}

qbl_status check_ws(void* ws, int64_t ws_bytes, int64_t need) {
  if (need == 0) return QBL_OK;
  if (!ws) return fail(QBL_E_BUDGET, "workspace of %lld bytes required", (long long)need);
  if (ws_bytes < need)
    return fail(QBL_E_BUDGET, "workspace of %lld bytes given, %lld required", (long long)ws_bytes,
                (long long)need);
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return fail(QBL_E_ARG, "workspace not 256-byte aligned");
  return QBL_OK;
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// qbl_linear: the shrink results t, float per batch row, or at batch 1 (the
// fused launch) kTCopies copies of one tagged 8-byte word each; above batch 1
// the matrix-core GEMV's staged inputs follow t.
int64_t linear_t_bytes(int64_t batch, int64_t T) {
  if (T == 0) return 0;
  return align_up(batch == 1 ? qbl::kTCopies * qbl::t_copy_stride(T) * 8 : batch * T * 4);
}
int64_t linear_ws_bytes(int64_t batch, int64_t T, int64_t n, int64_t k, int64_t sp_items) {
  return linear_t_bytes(batch, T) +
         (batch > 1 ? align_up(qbl::mfma_stage_bytes(n, (int)k, (int)T)) : align_up(sp_items * 8));
}

}  // namespace

extern "C" qbl_status qbl_workspace_bytes(const qbl_comp* comp, int32_t op, int32_t index,
                                          int32_t m, int64_t* bytes_out) {
  QBL_TRY({
    if (!comp || !bytes_out) return fail(QBL_E_ARG, "null pointer");
    auto L = std::atomic_load(&comp->list);
    const qbl_base* b = comp->base;
    if (op == 0) {
      if (index < 0 || index >= (int)b->lin.size()) return fail(QBL_E_ARG, "linear %d out of range", index);
      if (m < 1 || m > QBL_MAX_BATCH) return fail(QBL_E_LIMIT, "batch %d outside 1..%d", m, QBL_MAX_BATCH);
      *bytes_out = linear_ws_bytes(m, L->total_rank[(size_t)index], b->lin[(size_t)index].n, b->lin[(size_t)index].k,
                                   group_sp_items(b, L.get(), &index, 1));
      return QBL_OK;
    }
    if (op == 1) {
      if (index < 0 || index >= (int)b->lin.size()) return fail(QBL_E_ARG, "linear %d out of range", index);
      const DevLinear& D = b->lin[(size_t)index];
      *bytes_out = align_up(qbl::jit_workspace_bytes((int)D.n, (int)D.k, L->total_rank[(size_t)index]));
      return QBL_OK;
    }
    if (op == 2) {
      const int nb = (int)b->lin.size() / 7;
      if (nb < 1) return fail(QBL_E_SHAPE, "the base holds no block of 7 linears");
      int64_t d = 0, h = 0;
      for (int i = 0; i < nb; ++i) {
        Block B;
        if (qbl_status s = block_shape(b, i, &B)) return s;
        d = std::max(d, B.d);
        h = std::max(h, B.h);
      }
      *bytes_out = block_ws(nullptr, d, h, blocks_tmax(L.get(), 0, nb), blocks_spmax(b, L.get(), 0, nb)).bytes;
      return QBL_OK;
    }
    return fail(QBL_E_ARG, "unknown op %d", op);
  })
}

namespace {

// qbl_linear with the workspace either the caller's (ws, ws_bytes) or, when
// `use_static`, the library's per-device scratch array.
qbl_status linear_run(qbl_comp* comp, int32_t linear, const float* x, float* y, int32_t batch, void* ws,
                      int64_t ws_bytes, void* stream, bool use_static) {
  if (!comp || !x || !y) return fail(QBL_E_ARG, "null pointer");
  const qbl_base* b = comp->base;
  if (linear < 0 || linear >= (int)b->lin.size()) return fail(QBL_E_ARG, "linear %d out of range", linear);
  if (batch < 1 || batch > QBL_MAX_BATCH) return fail(QBL_E_LIMIT, "batch %d outside 1..%d", batch, QBL_MAX_BATCH);
  if (!aligned16(x) || !aligned16(y)) return fail(QBL_E_ARG, "x and y must be 16-byte aligned");
  if (x == y) return fail(QBL_E_ARG, "y must not alias x");
  if (qbl_status s = check_device(b)) return s;
  std::lock_guard<std::mutex> g(comp->mu);
  auto L = std::atomic_load(&comp->list);
  const int T = L->total_rank[(size_t)linear];
  const DevLinear& D = b->lin[(size_t)linear];
  const int64_t sp_items = group_sp_items(b, L.get(), &linear, 1);
  const int64_t need = linear_ws_bytes(batch, T, D.n, D.k, sp_items);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (use_static) {
    if (need > qbl::kStaticScratchBytes)
      return fail(QBL_E_LIMIT, "this run needs %lld bytes of scratch; the static array holds %lld", (long long)need,
                  (long long)qbl::kStaticScratchBytes);
  } else if (qbl_status s = check_ws(ws, ws_bytes, need)) {
    return s;
  }
  if (qbl_status s = check_handoffs()) return s;
  if (batch == 1 && (T > 0 || sp_items > 0))
    if (qbl_status s = refuse_capture(st)) return s;
  if (use_static && need > 0) {
    hipError_t e = qbl::static_scratch(st, &ws);
    if (e == hipErrorStreamCaptureUnsupported)
      return fail(QBL_E_STATE, "the first static-scratch run on a device sets the array up and cannot be captured");
    if (e != hipSuccess) return hip_fail(e, "static scratch");
  }
  const int lin[1] = {linear};
  float* outs[1] = {y};
  const float* v[1] = {x};
  ListUse use{L.get(), st, !L->plan[(size_t)linear].empty()};
  void* stage = batch > 1 ? static_cast<char*>(ws) + linear_t_bytes(batch, T) : nullptr;
  uint64_t* sp = batch == 1 && sp_items > 0
                     ? reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + linear_t_bytes(batch, T))
                     : nullptr;
  return run_group(b, L.get(), lin, outs, 1, v, 1, 0, batch, D.k, nullptr, static_cast<float*>(ws), sp, st, false,
                   nullptr, stage, &use);
}

}  // namespace

extern "C" qbl_status qbl_linear(qbl_comp* comp, int32_t linear, const float* x, float* y,
                                 int32_t batch, void* ws, int64_t ws_bytes, void* stream) {
  QBL_TRY({ return linear_run(comp, linear, x, y, batch, ws, ws_bytes, stream, false); })
}

extern "C" qbl_status qbl_linear_static(qbl_comp* comp, int32_t linear, const float* x, float* y,
                                        int32_t batch, void* stream) {
  QBL_TRY({ return linear_run(comp, linear, x, y, batch, nullptr, 0, stream, true); })
}

extern "C" qbl_status qbl_linear_jit(qbl_comp* comp, int32_t linear, const uint16_t* x_bf16,
                                     float* y, int32_t m, void* ws, int64_t ws_bytes, void* stream) {
  QBL_TRY({
    if (!comp || !x_bf16 || !y) return fail(QBL_E_ARG, "null pointer");
    const qbl_base* b = comp->base;
    if (linear < 0 || linear >= (int)b->lin.size()) return fail(QBL_E_ARG, "linear %d out of range", linear);
    if (m < 1) return fail(QBL_E_ARG, "m must be >= 1");
    if (!aligned16(x_bf16) || !aligned16(y)) return fail(QBL_E_ARG, "x and y must be 16-byte aligned");
    if (qbl_status s = check_device(b)) return s;
    std::lock_guard<std::mutex> g(comp->mu);
    auto L = std::atomic_load(&comp->list);
    const DevLinear& D = b->lin[(size_t)linear];
    for (const LoraRef& r : L->plan[(size_t)linear])
      if (r.rank == 0) return fail(QBL_E_FORMAT, "the prefill path takes low-rank adapters only");
    const int T = L->total_rank[(size_t)linear];
    if (qbl_status s = check_ws(ws, ws_bytes, align_up(qbl::jit_workspace_bytes((int)D.n, (int)D.k, T))))
      return s;
    qbl::JitArgs a{};
    a.qtype = D.qtype;
    a.qs = D.qs;
    a.sc = D.sc;
    a.n = (int)D.n;
    a.k = (int)D.k;
    a.m = m;
    a.X = x_bf16;
    a.Y = y;
    for (const LoraRef& r : L->plan[(size_t)linear]) {
      const int j = a.n_ad++;
      a.A[j] = r.A;
      a.B[j] = r.B;
      a.rank[j] = r.rank;
      a.scale[j] = r.scale;
    }
    a.total_rank = T;
    a.ws = static_cast<uint16_t*>(ws);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (qbl_status s = check_handoffs()) return s;
    ListUse use{L.get(), st, T > 0};
    KernelTimer tm(2, st);
    qbl::LaunchCtx lc = tm.ctx();
    const hipEvent_t done = use.attach(lc);  // on the GEMM launch, the last one
    hipError_t e = qbl::launch_jit(a, lc);
    if (e != hipSuccess) return hip_fail(e, "jit launch");
    if (done) use.attached = true;
    tm.stop();
    return QBL_OK;
  })
}

extern "C" qbl_status qbl_hbm_probe(const void* buf, int64_t bytes, uint32_t* sink, int32_t sink_words,
                                    int32_t* workgroups, void* stream) {
  QBL_TRY({
    if (!buf || !sink || !workgroups) return fail(QBL_E_ARG, "null pointer");
    if (bytes < 16 || bytes % 16) return fail(QBL_E_ARG, "bytes must be a positive multiple of 16");
    if (reinterpret_cast<uintptr_t>(buf) % 16) return fail(QBL_E_ARG, "buf must be 16-byte aligned");
    if (sink_words < 1) return fail(QBL_E_ARG, "sink_words must be >= 1");
    hipStream_t st = static_cast<hipStream_t>(stream);
    KernelTimer tm(4, st);
    hipError_t e = qbl::launch_hbm_probe(buf, bytes, sink, sink_words, tm.ctx());
    if (e != hipSuccess) return hip_fail(e, "probe launch");
    tm.stop();
    *workgroups = qbl::probe_workgroups(sink_words);
    return QBL_OK;
  })
}

extern "C" qbl_status qbl_requantize(qbl_comp* comp, int32_t linear, void* blocks_out, int64_t out_bytes,
                                     void* stream) {
  QBL_TRY({
    if (!comp || !blocks_out) return fail(QBL_E_ARG, "null pointer");
    const qbl_base* b = comp->base;
    if (linear < 0 || linear >= (int)b->lin.size()) return fail(QBL_E_ARG, "linear %d out of range", linear);
    if (qbl_status s = check_device(b)) return s;
    const DevLinear& D = b->lin[(size_t)linear];
    const int64_t need = D.n * (D.k / qbl_block_weights(D.qtype)) * qbl_block_bytes(D.qtype);
    if (out_bytes < need)
      return fail(QBL_E_BUDGET, "output holds %lld bytes; the linear needs %lld", (long long)out_bytes, (long long)need);
    if (reinterpret_cast<uintptr_t>(blocks_out) % 2) return fail(QBL_E_ARG, "output must be 2-byte aligned");
    std::lock_guard<std::mutex> g(comp->mu);
    auto L = std::atomic_load(&comp->list);
    qbl::DarArgs a{};
    a.qtype = D.qtype;
    a.qs = D.qs;
    a.sc = D.sc;
    a.n = (int)D.n;
    a.k = (int)D.k;
    for (const LoraRef& r : L->plan[(size_t)linear]) {
      const int j = a.n_ad++;
      a.rank[j] = r.rank;
      a.scale[j] = r.scale;
      a.A[j] = r.A;
      a.B[j] = r.B;
      a.rp[j] = r.rp;
      a.ci[j] = r.ci;
      a.sv[j] = r.sv;
    }
    a.out = static_cast<uint8_t*>(blocks_out);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const ListUse use{L.get(), st, a.n_ad > 0};
    KernelTimer tm(3, st);
    hipError_t e = qbl::launch_dar(a, tm.ctx());
    if (e != hipSuccess) return hip_fail(e, "requantize launch");
    tm.stop();
    return QBL_OK;
  })
}

extern "C" qbl_status qbl_block(qbl_comp* comp, int32_t block, const float* x, float* y, void* ws,
                                int64_t ws_bytes, void* stream) {
  QBL_TRY({
    if (!comp || !x || !y) return fail(QBL_E_ARG, "null pointer");
    const qbl_base* b = comp->base;
    Block B;
    if (qbl_status s = block_shape(b, block, &B)) return s;
    if (!aligned16(x) || !aligned16(y)) return fail(QBL_E_ARG, "x and y must be 16-byte aligned");
    if (qbl_status s = check_device(b)) return s;
    std::lock_guard<std::mutex> g(comp->mu);
    auto L = std::atomic_load(&comp->list);
    const BlockWs need = block_ws(nullptr, B.d, B.h, blocks_tmax(L.get(), block, 1), blocks_spmax(b, L.get(), block, 1));
    if (qbl_status s = check_ws(ws, ws_bytes, need.bytes)) return s;
    const BlockWs w = block_ws(ws, B.d, B.h, blocks_tmax(L.get(), block, 1), blocks_spmax(b, L.get(), block, 1));
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (qbl_status s = check_handoffs()) return s;
    if (blocks_have_entries(L.get(), block, 1))
      if (qbl_status s = refuse_capture(st)) return s;
    ListUse use{L.get(), st, true};
    if (qbl_status s = run_block(b, L.get(), B, x, 0, w, st)) return s;
    return run_rms(w.dd, B.d, y, st, &use);
  })
}

extern "C" qbl_status qbl_decode(qbl_comp* comp, int32_t first_block, int32_t n_blocks,
                                 const float* x0, float* y_tokens, int32_t n_tokens, void* ws,
                                 int64_t ws_bytes, void* stream) {
  QBL_TRY({
    if (!comp || !x0 || !y_tokens) return fail(QBL_E_ARG, "null pointer");
    if (n_blocks < 1 || n_tokens < 1) return fail(QBL_E_ARG, "n_blocks and n_tokens must be >= 1");
    const qbl_base* b = comp->base;
    std::vector<Block> blocks((size_t)n_blocks);
    for (int i = 0; i < n_blocks; ++i)
      if (qbl_status s = block_shape(b, first_block + i, &blocks[(size_t)i])) return s;
    const int64_t d = blocks[0].d;
    int64_t h = 0;
    for (auto& B : blocks) {
      if (B.d != d) return fail(QBL_E_SHAPE, "blocks of different widths in one stack");
      h = std::max(h, B.h);
    }
    if (!aligned16(x0) || !aligned16(y_tokens)) return fail(QBL_E_ARG, "x0 and y must be 16-byte aligned");
    if (qbl_status s = check_device(b)) return s;
    std::lock_guard<std::mutex> g(comp->mu);
    auto L = std::atomic_load(&comp->list);  // one list for the whole call
    const int tmax = blocks_tmax(L.get(), first_block, n_blocks);
    const int64_t spmax = blocks_spmax(b, L.get(), first_block, n_blocks);
    if (qbl_status s = check_ws(ws, ws_bytes, block_ws(nullptr, d, h, tmax, spmax).bytes)) return s;
    const BlockWs w = block_ws(ws, d, h, tmax, spmax);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (qbl_status s = check_handoffs()) return s;
    if (blocks_have_entries(L.get(), first_block, n_blocks))
      if (qbl_status s = refuse_capture(st)) return s;
    ListUse use{L.get(), st, true};
    for (int t = 0; t < n_tokens; ++t) {
      const float* in = t == 0 ? x0 : y_tokens + (int64_t)(t - 1) * d;
      for (int i = 0; i < n_blocks; ++i) {
        if (qbl_status s = run_block(b, L.get(), blocks[(size_t)i], i == 0 ? in : w.dd, i == 0 ? 0 : 1, w, st))
          return s;
      }
      if (qbl_status s = run_rms(w.dd, d, y_tokens + (int64_t)t * d, st, t + 1 == n_tokens ? &use : nullptr))
        return s;
    }
    return QBL_OK;
  })
}
