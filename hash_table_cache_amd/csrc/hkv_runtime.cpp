// Host runtime of the C ABI declared in include/hkv.h: argument validation,
// table storage, workspace management and reader/updater/inserter ordering.
//
// Group ordering follows the compatibility matrix of §3.5 (Table 4) of
// "HierarchicalKV: A GPU Hash Table with Cache Semantics for Continuous Online
// Embedding Storage": readers may overlap readers, updaters may overlap
// updaters, inserters overlap nothing. The paper enforces it with host
// counters mirrored to the device by a propagation kernel (§4.4); here every
// call instead makes its own stream wait (hipStreamWaitEvent) on the last
// event recorded by each incompatible group on every other stream, then
// records its own event. The host never blocks, and calls issued on a single
// stream need no waits at all because stream order already serializes them.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "hkv.h"
#include "hkv_internal.h"

#define HKV_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr uint64_t kSlots = HKV_BUCKET_SLOTS;
constexpr uint64_t kMaxBatch = 0xFFFFFFFCull;  // indices 0xFFFFFFFC..F are chain markers
constexpr uint32_t kMaxDim = 1u << 20;
constexpr size_t kProfileEvents = 512;  // timing events made ready by hkv_profile_start

enum Group { kReader = 0, kUpdater = 1, kInserter = 2 };

// Table 4: readers overlap readers, updaters overlap updaters. Under the
// reader/writer baseline only readers overlap.
bool groups_conflict(int a, int b, bool rw_lock) {
  if (rw_lock) return !(a == kReader && b == kReader);
  return !(a == b && a != kInserter);
}

thread_local std::string g_error;

hkv_status fail(hkv_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

hkv_status fail_hip(hipError_t e, const char* what) {
  return fail(HKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

struct StreamEvent {
  hipStream_t stream;
  hipEvent_t event;
};

// Makes `device` current for the lifetime of the guard.
class DeviceGuard {
 public:
  explicit DeviceGuard(int device) : target_(device) {
    err_ = hipGetDevice(&prev_);
    if (err_ == hipSuccess && prev_ != target_) err_ = hipSetDevice(target_);
  }
  ~DeviceGuard() {
    if (err_ == hipSuccess && prev_ != target_) (void)hipSetDevice(prev_);
  }
  hipError_t error() const { return err_; }

 private:
  int prev_ = -1;
  int target_;
  hipError_t err_;
};

// Per-kernel timing (hkv_profile_start/stop): while profiling is on, every
// kernel is launched with a start/stop event pair that its dispatch records.
class Profiler final : public hkv::KernelTimer {
 public:
  struct Rec {
    const char* name;
    hipEvent_t start;
    hipEvent_t stop;
  };
  bool take(hipEvent_t* start, hipEvent_t* stop) override {
    *start = next_event();
    *stop = *start ? next_event() : nullptr;
    if (*start && !*stop) {
      pool_.push_back(*start);
      *start = nullptr;
    }
    return *start != nullptr;
  }
  void launched(const char* kernel, hipEvent_t start, hipEvent_t stop) override {
    recs_.push_back({kernel, start, stop});
  }
  std::vector<Rec>& records() { return recs_; }
  void give_back(hipEvent_t e) { pool_.push_back(e); }
  // Creates events until the pool holds `count`, and records each new one
  // once (on a private stream, waited for), so that no event is created or
  // used for the first time while launches are being timed. The stream
  // lives as long as the events: an event keeps a reference to the stream
  // it was last recorded on, which later synchronization on it consults.
  void prewarm(size_t count) {
    if (pool_.size() >= count) return;
    if (!warm_ && hipStreamCreateWithFlags(&warm_, hipStreamNonBlocking) != hipSuccess) {
      (void)hipGetLastError();
      warm_ = nullptr;
      return;
    }
    while (pool_.size() < count) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) {
        (void)hipGetLastError();
        break;
      }
      (void)hipEventRecord(e, warm_);
      pool_.push_back(e);
    }
    (void)hipStreamSynchronize(warm_);
  }
  void destroy_all() {
    for (auto& r : recs_) {
      (void)hipEventDestroy(r.start);
      (void)hipEventDestroy(r.stop);
    }
    for (auto e : pool_) (void)hipEventDestroy(e);
    recs_.clear();
    pool_.clear();
    if (warm_) (void)hipStreamDestroy(warm_);
    warm_ = nullptr;
  }

 private:
  hipEvent_t next_event() {
    if (!pool_.empty()) {
      hipEvent_t e = pool_.back();
      pool_.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  std::vector<Rec> recs_;
  std::vector<hipEvent_t> pool_;
  hipStream_t warm_ = nullptr;  // the prewarm records' stream (kept with the pool)
};

}  // namespace

struct hkv_table {
  hkv_options opt{};
  uint32_t* scratch = nullptr;  // the device's fixed no-alloc scratch (not owned)
  hkv::TableView view{};
  void* values_host = nullptr;  // hipHostMalloc base of the host-resident rows
  float* values_dev = nullptr;  // hipMalloc base of the HBM-resident rows
  uint32_t* ws_next = nullptr;  // inserter workspace
  uint32_t* ws_target = nullptr;
  uint64_t ws_cap = 0;
  uint8_t* ev_kind = nullptr;  // insert_and_evict staging (parallel inserter)
  uint64_t* ev_keys = nullptr;
  uint64_t* ev_scores = nullptr;
  float* ev_rows = nullptr;
  uint32_t* ev_chunks = nullptr;
  uint64_t ev_cap = 0;
  unsigned long long* size_dev = nullptr;
  unsigned long long* size_host = nullptr;  // pinned
  unsigned long long* stat_slots = nullptr;  // outcome counting words (4 * kStatSlots)
  unsigned long long* outcomes = nullptr;    // the caller's 4 counters, or nullptr
  std::mutex mu;
  std::vector<StreamEvent> last[3];  // per group: last event recorded on each stream
  bool any_call = false;             // a call has been issued
  bool multi_stream = false;         // calls have come from more than one stream
  hipStream_t first_stream = nullptr;
  Profiler prof;
  bool profiling = false;
  hkv::KernelTimer* timer() { return profiling ? &prof : nullptr; }
};

namespace {

void free_storage(hkv_table* t) {
  hkv::TableView& v = t->view;
  if (v.digests) (void)hipFree(v.digests);
  if (v.keys) (void)hipFree(v.keys);
  if (v.scores) (void)hipFree(v.scores);
  if (v.occ) (void)hipFree(v.occ);
  if (v.head) (void)hipFree(v.head);
  if (v.bmin) (void)hipFree(v.bmin);
  if (v.claim) (void)hipFree(v.claim);
  if (t->values_host) (void)hipHostFree(t->values_host);
  if (t->values_dev) (void)hipFree(t->values_dev);
  if (t->ws_next) (void)hipFree(t->ws_next);
  if (t->ws_target) (void)hipFree(t->ws_target);
  if (t->ev_kind) (void)hipFree(t->ev_kind);
  if (t->ev_keys) (void)hipFree(t->ev_keys);
  if (t->ev_scores) (void)hipFree(t->ev_scores);
  if (t->ev_rows) (void)hipFree(t->ev_rows);
  if (t->ev_chunks) (void)hipFree(t->ev_chunks);
  if (t->stat_slots) (void)hipFree(t->stat_slots);
  if (t->size_dev) (void)hipFree(t->size_dev);
  if (t->size_host) (void)hipHostFree(t->size_host);
  for (auto& list : t->last)
    for (auto& r : list) (void)hipEventDestroy(r.event);
  t->prof.destroy_all();
}

// Checks that [p, p + bytes) is memory the table's GPU can access: device
// memory of that GPU, or pinned/mapped host memory, inside one allocation.
hkv_status check_buffer(const hkv_table* t, const void* p, uint64_t bytes, const char* what) {
  if (!p) return fail(HKV_EINVAL, "%s is NULL", what);
  hipPointerAttribute_t a;
  std::memset(&a, 0, sizeof(a));
  hipError_t e = hipPointerGetAttributes(&a, p);
  if (e != hipSuccess || a.type == hipMemoryTypeUnregistered) {
    (void)hipGetLastError();
    return fail(HKV_EINVAL, "%s (%p) is not device-accessible memory (pageable host memory?)", what, p);
  }
  if (a.type == hipMemoryTypeDevice && a.device != t->opt.device)
    return fail(HKV_EINVAL, "%s lives on device %d, table on device %d", what, a.device, t->opt.device);
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  e = hipMemGetAddressRange(&base, &size, const_cast<void*>(p));
  if (e == hipSuccess && base && size) {
    const uint64_t off = reinterpret_cast<uintptr_t>(p) - reinterpret_cast<uintptr_t>(base);
    if (off > size || bytes > size - off)
      return fail(HKV_EINVAL, "%s holds %llu bytes past %p, call needs %llu", what,
                  static_cast<unsigned long long>(size - off), p, static_cast<unsigned long long>(bytes));
  } else {
    (void)hipGetLastError();
  }
  return HKV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// While every call of a table comes from one stream, stream order alone
// orders them and no events are recorded (an event record costs about as
// much host time as the launch it follows). The first call from a second
// stream finds earlier calls without events, so it waits once for the device
// to finish its work; from then on every call records its event. Caller
// holds t->mu.
hkv_status enter_stream(hkv_table* t, hipStream_t s) {
  if (t->multi_stream) return HKV_OK;
  if (!t->any_call) {
    t->any_call = true;
    t->first_stream = s;
    return HKV_OK;
  }
  if (s == t->first_stream) return HKV_OK;
  const hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return fail_hip(e, "hipDeviceSynchronize");
  t->multi_stream = true;
  return HKV_OK;
}

// Makes stream s wait for every outstanding call of a group incompatible with g
// that was issued on another stream. Caller holds t->mu.
hkv_status order_before(hkv_table* t, int g, hipStream_t s) {
  hkv_status st = enter_stream(t, s);
  if (st != HKV_OK || !t->multi_stream) return st;
  for (int h = 0; h < 3; ++h) {
    if (!groups_conflict(g, h, (t->opt.flags & HKV_FLAG_RW_LOCK) != 0)) continue;
    for (auto& r : t->last[h]) {
      if (r.stream == s) continue;
      const hipError_t q = hipEventQuery(r.event);
      if (q == hipSuccess) continue;
      if (q != hipErrorNotReady) (void)hipGetLastError();
      const hipError_t e = hipStreamWaitEvent(s, r.event, 0);
      if (e != hipSuccess) return fail_hip(e, "hipStreamWaitEvent");
    }
  }
  return HKV_OK;
}

// Records group g's completion event on stream s (once the table is used
// from more than one stream). Caller holds t->mu.
hkv_status record_after(hkv_table* t, int g, hipStream_t s) {
  if (!t->multi_stream) return HKV_OK;
  hipEvent_t ev = nullptr;
  for (auto& r : t->last[g])
    if (r.stream == s) ev = r.event;
  if (!ev) {
    const hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return fail_hip(e, "hipEventCreateWithFlags");
    t->last[g].push_back({s, ev});
  }
  const hipError_t e = hipEventRecord(ev, s);
  if (e != hipSuccess) return fail_hip(e, "hipEventRecord");
  return HKV_OK;
}

// Waits for every outstanding call of group g (used before replacing a
// workspace and on destroy). Single-stream calls have no events: the device
// is synchronized instead.
hkv_status drain_group(hkv_table* t, int g) {
  if (!t->multi_stream) {
    if (!t->any_call) return HKV_OK;
    const hipError_t e = hipDeviceSynchronize();
    return e == hipSuccess ? HKV_OK : fail_hip(e, "hipDeviceSynchronize");
  }
  for (auto& r : t->last[g]) {
    const hipError_t e = hipEventSynchronize(r.event);
    if (e != hipSuccess) return fail_hip(e, "hipEventSynchronize");
  }
  return HKV_OK;
}

hkv_status ensure_workspace(hkv_table* t, uint64_t n) {
  if (n <= t->ws_cap) return HKV_OK;
  hkv_status st = drain_group(t, kInserter);
  if (st != HKV_OK) return st;
  uint64_t cap = t->ws_cap ? t->ws_cap : 1024;
  while (cap < n) cap *= 2;
  if (cap > kMaxBatch) cap = kMaxBatch;
  auto release = [t]() {
    if (t->ws_next) (void)hipFree(t->ws_next);
    if (t->ws_target) (void)hipFree(t->ws_target);
    t->ws_next = t->ws_target = nullptr;
    t->ws_cap = 0;
  };
  release();
  if (hipMalloc(&t->ws_next, cap * sizeof(uint32_t)) != hipSuccess ||
      hipMalloc(&t->ws_target, cap * sizeof(uint32_t)) != hipSuccess) {
    (void)hipGetLastError();
    release();
    return fail(HKV_ENOMEM, "inserter workspace of %llu entries", static_cast<unsigned long long>(cap));
  }
  t->ws_cap = cap;
  return HKV_OK;
}

// Staging for insert_and_evict's hand-back: 17 + 4*dim bytes per batch key
// plus 4 bytes per 1024 keys, grown on demand like the inserter workspace.
hkv_status ensure_evict_stage(hkv_table* t, uint64_t n) {
  if (n <= t->ev_cap) return HKV_OK;
  hkv_status st = drain_group(t, kInserter);
  if (st != HKV_OK) return st;
  uint64_t cap = t->ev_cap ? t->ev_cap : 1024;
  while (cap < n) cap *= 2;
  if (cap > kMaxBatch) cap = kMaxBatch;
  auto release = [t]() {
    void* p[5] = {t->ev_kind, t->ev_keys, t->ev_scores, t->ev_rows, t->ev_chunks};
    for (void* q : p)
      if (q) (void)hipFree(q);
    t->ev_kind = nullptr;
    t->ev_keys = t->ev_scores = nullptr;
    t->ev_rows = nullptr;
    t->ev_chunks = nullptr;
    t->ev_cap = 0;
  };
  release();
  const uint64_t dim = t->opt.dim;
  const uint64_t chunks = (cap + 1023) / 1024;
  if (hipMalloc(&t->ev_kind, cap) != hipSuccess || hipMalloc(&t->ev_keys, cap * 8) != hipSuccess ||
      hipMalloc(&t->ev_scores, cap * 8) != hipSuccess || hipMalloc(&t->ev_rows, cap * dim * 4) != hipSuccess ||
      hipMalloc(&t->ev_chunks, chunks * 4) != hipSuccess) {
    (void)hipGetLastError();
    release();
    return fail(HKV_ENOMEM, "insert_and_evict staging of %llu entries", static_cast<unsigned long long>(cap));
  }
  t->ev_cap = cap;
  return HKV_OK;
}

// Address of the fixed no-alloc scratch array on each device, looked up once
// per device (with that device current) and kept for the process.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint32_t* g_scratch[kMaxDevices] = {};

hkv_status device_scratch(int device, uint32_t** out) {
  if (device < 0 || device >= kMaxDevices) return fail(HKV_EUNSUPPORTED, "device %d beyond %d", device, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[device]) {
    uint32_t* p = nullptr;
    const hipError_t e = hkv::scratch_address(&p);
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail_hip(e, "hipGetSymbolAddress(scratch)");
    }
    g_scratch[device] = p;
  }
  *out = g_scratch[device];
  return HKV_OK;
}

// True when a call on stream s would have to create an ordering event (the
// table is, or by this call becomes, used from several streams, and s has no
// inserter event yet). Caller holds t->mu.
bool would_create_event(const hkv_table* t, hipStream_t s) {
  const bool multi = t->multi_stream || (t->any_call && s != t->first_stream);
  if (!multi) return false;
  for (const auto& r : t->last[kInserter])
    if (r.stream == s) return false;
  return true;
}

}  // namespace

// Shared tail of the inserter calls (arguments already validated): workspace,
// ordering after incompatible groups, launch, completion event. `fixed`: the
// no-alloc variant: the chain and target words come from the device's fixed
// scratch array and nothing is allocated.
static hkv_status run_inserter(hkv_table* t, uint64_t n, hkv::InsertCall c, bool vec4, const char* what,
                               hipStream_t stream, bool fixed = false) {
  const bool serial = (t->opt.flags & HKV_FLAG_SERIAL_INSERT) != 0;
  const bool needs_ws = !serial || c.fetch || c.ev_keys;
  std::lock_guard<std::mutex> lk(t->mu);
  DeviceGuard dg(t->opt.device);
  if (dg.error() != hipSuccess) return fail_hip(dg.error(), "hipSetDevice");
  hkv_status st;
  uint32_t* ws_next = t->ws_next;
  uint32_t* ws_target = t->ws_target;
  if (fixed) {
    if (would_create_event(t, stream))
      return fail(HKV_EINVAL, "%s: the table is used from several streams and this stream has no inserter event "
                  "yet; issue one hkv_insert_or_assign on it first", what);
    ws_next = t->scratch;
    ws_target = t->scratch + hkv::noalloc_max_keys();
  } else if (needs_ws && (st = ensure_workspace(t, n)) != HKV_OK) {
    return st;
  } else {
    ws_next = t->ws_next;
    ws_target = t->ws_target;
  }
  if (c.ev_keys && !serial && n > 0) {
    if ((st = ensure_evict_stage(t, n)) != HKV_OK) return st;
    c.st_kind = t->ev_kind;
    c.st_keys = t->ev_keys;
    c.st_scores = t->ev_scores;
    c.st_rows = t->ev_rows;
    c.chunk_count = t->ev_chunks;
  }
  if (!serial && t->outcomes) {
    c.stat_slots = t->stat_slots;
    c.outcomes = t->outcomes;
  }
  if ((st = order_before(t, kInserter, stream)) != HKV_OK) return st;
  // A new epoch per call: chain heads of earlier calls then read as empty.
  // After 2^32 - 1 calls the counter wraps and every head is reset first.
  // A call captured into a graph is replayed with the arguments it was
  // captured with, so it runs at epoch 0, whose owners reset their heads.
  hkv::TableView v = t->view;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
    (void)hipGetLastError();
    cs = hipStreamCaptureStatusNone;
  }
  if (cs == hipStreamCaptureStatusActive) {
    v.epoch = 0;
  } else {
    if (++t->view.epoch == 0) {
      const hipError_t er = hkv::launch_reset_heads(t->view, stream);
      if (er != hipSuccess) return fail_hip(er, what);
      t->view.epoch = 1;
    }
    v.epoch = t->view.epoch;
  }
  const hipError_t e = hkv::launch_upsert(v, n, c, ws_next, ws_target, vec4, serial, stream, t->timer());
  if (e != hipSuccess) return fail_hip(e, what);
  return record_after(t, kInserter, stream);
}

// Shared tail of find_ptr and contains.
static hkv_status run_locate(hkv_table* t, uint64_t n, const uint64_t* keys, uint64_t* ptrs, uint8_t* found,
                             uint64_t* scores, hipStream_t stream) {
  std::lock_guard<std::mutex> lk(t->mu);
  DeviceGuard dg(t->opt.device);
  if (dg.error() != hipSuccess) return fail_hip(dg.error(), "hipSetDevice");
  hkv_status st;
  if ((st = order_before(t, kReader, stream)) != HKV_OK) return st;
  const hipError_t e = hkv::launch_locate(t->view, n, keys, ptrs, found, scores, stream, t->timer());
  if (e != hipSuccess) return fail_hip(e, ptrs ? "find_ptr launch" : "contains launch");
  return record_after(t, kReader, stream);
}

HKV_API const char* hkv_last_error(void) { return g_error.c_str(); }

HKV_API hkv_status hkv_create(const hkv_options* o, hkv_table** out) {
  if (!out) return fail(HKV_EINVAL, "out is NULL");
  *out = nullptr;
  if (!o) return fail(HKV_EINVAL, "options is NULL");
  if (o->capacity == 0 || o->capacity % kSlots != 0)
    return fail(HKV_EINVAL, "capacity %llu is not a positive multiple of 128",
                static_cast<unsigned long long>(o->capacity));
  if (o->capacity / kSlots > 0x7FFFFFFFull)
    return fail(HKV_EINVAL, "capacity %llu exceeds 2^31 - 1 buckets", static_cast<unsigned long long>(o->capacity));
  if (o->dim == 0 || o->dim > kMaxDim) return fail(HKV_EINVAL, "dim %u outside [1, %u]", o->dim, kMaxDim);
  if (o->bucket_slots != 0 && o->bucket_slots != kSlots)
    return fail(HKV_EINVAL, "bucket_slots %u: only 128-slot buckets exist", o->bucket_slots);
  if (o->dual_bucket > 1 || o->values_on_host > 1) return fail(HKV_EINVAL, "dual_bucket/values_on_host must be 0 or 1");
  if (o->flags & ~(HKV_FLAG_SERIAL_INSERT | HKV_FLAG_RW_LOCK | HKV_FLAG_UNIQUE_KEYS))
    return fail(HKV_EINVAL, "unknown flags 0x%x", o->flags);
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess || ndev == 0) {
    (void)hipGetLastError();
    return fail(HKV_EHIP, "no HIP device available");
  }
  if (o->device < 0 || o->device >= ndev) return fail(HKV_EINVAL, "device %d outside [0, %d)", o->device, ndev);

  hkv_table* t = new (std::nothrow) hkv_table();
  if (!t) return fail(HKV_ENOMEM, "host allocation");
  t->opt = *o;
  t->opt.bucket_slots = kSlots;
  DeviceGuard dg(o->device);
  if (dg.error() != hipSuccess) {
    delete t;
    return fail_hip(dg.error(), "hipSetDevice");
  }
  const uint64_t cap = o->capacity, nb = cap / kSlots;
  hkv::TableView& v = t->view;
  v.nb = nb;
  v.pow2 = (nb & (nb - 1)) == 0;
  v.nb_mask = v.pow2 ? nb - 1 : 0;
  v.dim = o->dim;
  v.dual = o->dual_bucket;
  v.claims = (o->flags & HKV_FLAG_UNIQUE_KEYS) ? 0u : 1u;
  // Tuning overrides: lanes serving one key (4, 8 or 16; anything else keeps
  // the default chosen from dim) and keys per group of the key-side probes of
  // find* and contains (1, 2 or 4; default 2).
  if (const char* g = std::getenv("HKV_GROUP_LANES")) v.lanes = static_cast<uint32_t>(std::atoi(g));
  v.keys_per_group = 2;
  if (const char* g = std::getenv("HKV_KEYS_PER_GROUP")) v.keys_per_group = static_cast<uint32_t>(std::atoi(g));
  // Inserter-call counter (the first eager call takes epoch 1; 0 is kept for
  // captured calls); a start value lets tests reach its wrap.
  v.epoch = 0;
  if (const char* g = std::getenv("HKV_EPOCH_START")) v.epoch = static_cast<uint32_t>(std::strtoul(g, nullptr, 0));
  bool ok = hipMalloc(&v.digests, cap) == hipSuccess && hipMalloc(&v.keys, cap * 8) == hipSuccess &&
            hipMalloc(&v.scores, cap * 8) == hipSuccess && hipMalloc(&v.occ, nb * 4) == hipSuccess &&
            hipMalloc(&v.head, nb * 8) == hipSuccess && hipMalloc(&v.claim, nb * 16) == hipSuccess &&
            hipMalloc(&t->size_dev, 8) == hipSuccess &&
            (!o->dual_bucket || hipMalloc(&v.bmin, nb * 16) == hipSuccess) &&
            hipHostMalloc(&t->size_host, 8, hipHostMallocDefault) == hipSuccess;
  // Value rows: the first `split` positions in HBM, the rest in pinned host
  // memory mapped into the GPU (§3.6, §4.2 watermark); split is whole buckets.
  const uint64_t row_bytes = static_cast<uint64_t>(o->dim) * sizeof(float);
  uint64_t split = cap;
  if (o->values_on_host) {
    const uint64_t hbm_buckets = o->hbm_value_bytes / (kSlots * row_bytes);
    split = hbm_buckets >= nb ? cap : hbm_buckets * kSlots;
  }
  v.split = split;
  if (ok && split > 0) ok = hipMalloc(&t->values_dev, split * row_bytes) == hipSuccess;
  float* host_dev = nullptr;
  if (ok && split < cap)
    ok = hipHostMalloc(&t->values_host, (cap - split) * row_bytes, hipHostMallocMapped) == hipSuccess &&
         hipHostGetDevicePointer(reinterpret_cast<void**>(&host_dev), t->values_host, 0) == hipSuccess;
  if (ok) {
    v.values = split > 0 ? t->values_dev : host_dev;
    // second-region base, offset so that row p sits at values_hi + p * dim
    v.values_hi = split < cap ? reinterpret_cast<float*>(reinterpret_cast<uintptr_t>(host_dev) -
                                                         split * row_bytes)
                              : v.values;
  }
  if (!ok) {
    (void)hipGetLastError();
    free_storage(t);
    delete t;
    return fail(HKV_ENOMEM, "table storage for capacity %llu, dim %u (%llu rows in HBM, %llu on the host)",
                static_cast<unsigned long long>(cap), o->dim, static_cast<unsigned long long>(split),
                static_cast<unsigned long long>(cap - split));
  }
  // Initialise on a private non-blocking stream: the legacy null stream
  // would also synchronize with (and be checked against) every other stream
  // of the process. A stale error of an earlier, unrelated call on this
  // thread is cleared first so that it is not reported as the launch's.
  (void)hipGetLastError();
  hipStream_t init_stream = nullptr;
  e = hipStreamCreateWithFlags(&init_stream, hipStreamNonBlocking);
  if (e == hipSuccess) {
    e = hkv::launch_init(v, init_stream);
    const hipError_t e2 = hipStreamSynchronize(init_stream);
    if (e == hipSuccess) e = e2;
    (void)hipStreamDestroy(init_stream);
  }
  if (e != hipSuccess) {
    free_storage(t);
    delete t;
    return fail_hip(e, "table initialisation");
  }
  const hkv_status sst = device_scratch(o->device, &t->scratch);
  if (sst != HKV_OK) {
    free_storage(t);
    delete t;
    return sst;
  }
  *out = t;
  return HKV_OK;
}

HKV_API hkv_status hkv_destroy(hkv_table* t) {
  if (!t) return HKV_OK;
  {
    std::lock_guard<std::mutex> lk(t->mu);
    DeviceGuard dg(t->opt.device);
    for (int g = 0; g < 3; ++g) (void)drain_group(t, g);
    free_storage(t);
  }
  delete t;
  return HKV_OK;
}

HKV_API hkv_status hkv_get_options(const hkv_table* t, hkv_options* out) {
  if (!t || !out) return fail(HKV_EINVAL, "NULL argument");
  *out = t->opt;
  return HKV_OK;
}

HKV_API hkv_status hkv_find(hkv_table* t, uint64_t n, const uint64_t* keys, float* values_out,
                            uint8_t* found_out, uint64_t* scores_out, hipStream_t stream) {
  if (!t) return fail(HKV_EINVAL, "table is NULL");
  if (n == 0) return HKV_OK;
  if (n > kMaxBatch) return fail(HKV_EINVAL, "batch of %llu keys exceeds the limit", static_cast<unsigned long long>(n));
  const uint64_t dim = t->opt.dim;
  hkv_status st;
  if ((st = check_buffer(t, keys, n * 8, "keys")) != HKV_OK) return st;
  if ((st = check_buffer(t, values_out, n * dim * 4, "values_out")) != HKV_OK) return st;
  if ((st = check_buffer(t, found_out, n, "found_out")) != HKV_OK) return st;
  if (scores_out && (st = check_buffer(t, scores_out, n * 8, "scores_out")) != HKV_OK) return st;
  const bool vec4 = dim % 4 == 0 && aligned16(values_out);
  std::lock_guard<std::mutex> lk(t->mu);
  DeviceGuard dg(t->opt.device);
  if (dg.error() != hipSuccess) return fail_hip(dg.error(), "hipSetDevice");
  if ((st = order_before(t, kReader, stream)) != HKV_OK) return st;
  const hipError_t e = hkv::launch_find(t->view, n, keys, values_out, found_out, scores_out, vec4, stream, t->timer());
  if (e != hipSuccess) return fail_hip(e, "find launch");
  return record_after(t, kReader, stream);
}

HKV_API hkv_status hkv_find_ptr(hkv_table* t, uint64_t n, const uint64_t* keys, float** values_ptr_out,
                                uint8_t* found_out, uint64_t* scores_out, hipStream_t stream) {
  if (!t) return fail(HKV_EINVAL, "table is NULL");
  if (n == 0) return HKV_OK;
  if (n > kMaxBatch) return fail(HKV_EINVAL, "batch of %llu keys exceeds the limit", static_cast<unsigned long long>(n));
  hkv_status st;
  if ((st = check_buffer(t, keys, n * 8, "keys")) != HKV_OK) return st;
  if ((st = check_buffer(t, values_ptr_out, n * sizeof(float*), "values_ptr_out")) != HKV_OK) return st;
  if (found_out && (st = check_buffer(t, found_out, n, "found_out")) != HKV_OK) return st;
  if (scores_out && (st = check_buffer(t, scores_out, n * 8, "scores_out")) != HKV_OK) return st;
  static_assert(sizeof(float*) == sizeof(uint64_t), "64-bit addresses");
  return run_locate(t, n, keys, reinterpret_cast<uint64_t*>(values_ptr_out), found_out, scores_out, stream);
}

HKV_API hkv_status hkv_contains(hkv_table* t, uint64_t n, const uint64_t* keys, uint8_t* found_out,
                                hipStream_t stream) {
  if (!t) return fail(HKV_EINVAL, "table is NULL");
  if (n == 0) return HKV_OK;
  if (n > kMaxBatch) return fail(HKV_EINVAL, "batch of %llu keys exceeds the limit", static_cast<unsigned long long>(n));
  hkv_status st;
  if ((st = check_buffer(t, keys, n * 8, "keys")) != HKV_OK) return st;
  if ((st = check_buffer(t, found_out, n, "found_out")) != HKV_OK) return st;
  return run_locate(t, n, keys, nullptr, found_out, nullptr, stream);
}

HKV_API hkv_status hkv_insert_or_assign(hkv_table* t, uint64_t n, const uint64_t* keys,
                                        const float* values, const uint64_t* scores,
                                        hipStream_t stream) {
  if (!t) return fail(HKV_EINVAL, "table is NULL");
  if (n == 0) return HKV_OK;
  if (n > kMaxBatch) return fail(HKV_EINVAL, "batch of %llu keys exceeds the limit", static_cast<unsigned long long>(n));
  const uint64_t dim = t->opt.dim;
  hkv_status st;
  if ((st = check_buffer(t, keys, n * 8, "keys")) != HKV_OK) return st;
  if ((st = check_buffer(t, values, n * dim * 4, "values")) != HKV_OK) return st;
  if ((st = check_buffer(t, scores, n * 8, "scores")) != HKV_OK) return st;
  const bool vec4 = dim % 4 == 0 && aligned16(values);
  hkv::InsertCall c{};
  c.keys = keys;
  c.values = const_cast<float*>(values);  // read only: fetch and eviction output are off
  c.scores = scores;
  return run_inserter(t, n, c, vec4, "insert_or_assign", stream);
}

HKV_API hkv_status hkv_insert_or_assign_noalloc(hkv_table* t, uint64_t n, const uint64_t* keys,
                                                const float* values, const uint64_t* scores,
                                                hipStream_t stream) {
  if (!t) return fail(HKV_EINVAL, "table is NULL");
  if (n == 0) return HKV_OK;
  if (n > hkv::noalloc_max_keys())
    return fail(HKV_EINVAL, "insert_or_assign_noalloc: batch of %llu keys exceeds its limit of %llu",
                static_cast<unsigned long long>(n), static_cast<unsigned long long>(hkv::noalloc_max_keys()));
  const uint64_t dim = t->opt.dim;
  hkv_status st;
  if ((st = check_buffer(t, keys, n * 8, "keys")) != HKV_OK) return st;
  if ((st = check_buffer(t, values, n * dim * 4, "values")) != HKV_OK) return st;
  if ((st = check_buffer(t, scores, n * 8, "scores")) != HKV_OK) return st;
  const bool vec4 = dim % 4 == 0 && aligned16(values);
  hkv::InsertCall c{};
  c.keys = keys;
  c.values = const_cast<float*>(values);  // read only
  c.scores = scores;
  return run_inserter(t, n, c, vec4, "insert_or_assign_noalloc", stream, true);
}

HKV_API hkv_status hkv_insert_and_evict(hkv_table* t, uint64_t n, const uint64_t* keys, const float* values,
                                        const uint64_t* scores, uint64_t* evicted_keys, float* evicted_values,
                                        uint64_t* evicted_scores, uint64_t* evicted_count,
                                        hipStream_t stream) {
  if (!t) return fail(HKV_EINVAL, "table is NULL");
  if (n > kMaxBatch) return fail(HKV_EINVAL, "batch of %llu keys exceeds the limit", static_cast<unsigned long long>(n));
  const uint64_t dim = t->opt.dim;
  hkv_status st;
  if ((st = check_buffer(t, evicted_count, 8, "evicted_count")) != HKV_OK) return st;
  if (n == 0) {
    // only the count is written (zero), in inserter order like any other call
    hkv::InsertCall c{};
    c.ev_keys = evicted_keys;
    c.ev_count = reinterpret_cast<unsigned long long*>(evicted_count);
    return run_inserter(t, 0, c, false, "insert_and_evict", stream);
  }
  if ((st = check_buffer(t, keys, n * 8, "keys")) != HKV_OK) return st;
  if ((st = check_buffer(t, values, n * dim * 4, "values")) != HKV_OK) return st;
  if ((st = check_buffer(t, scores, n * 8, "scores")) != HKV_OK) return st;
  if ((st = check_buffer(t, evicted_keys, n * 8, "evicted_keys")) != HKV_OK) return st;
  if (evicted_values && (st = check_buffer(t, evicted_values, n * dim * 4, "evicted_values")) != HKV_OK) return st;
  if (evicted_scores && (st = check_buffer(t, evicted_scores, n * 8, "evicted_scores")) != HKV_OK) return st;
  const bool vec4 = dim % 4 == 0 && aligned16(values) && (!evicted_values || aligned16(evicted_values));
  hkv::InsertCall c{};
  c.keys = keys;
  c.values = const_cast<float*>(values);  // read only: fetch is off
  c.scores = scores;
  c.ev_keys = evicted_keys;
  c.ev_values = evicted_values;
  c.ev_scores = evicted_scores;
  c.ev_count = reinterpret_cast<unsigned long long*>(evicted_count);
  return run_inserter(t, n, c, vec4, "insert_and_evict", stream);
}

HKV_API hkv_status hkv_find_or_insert(hkv_table* t, uint64_t n, const uint64_t* keys, float* values,
                                      const uint64_t* scores, uint8_t* found_out, hipStream_t stream) {
  if (!t) return fail(HKV_EINVAL, "table is NULL");
  if (n == 0) return HKV_OK;
  if (n > kMaxBatch) return fail(HKV_EINVAL, "batch of %llu keys exceeds the limit", static_cast<unsigned long long>(n));
  const uint64_t dim = t->opt.dim;
  hkv_status st;
  if ((st = check_buffer(t, keys, n * 8, "keys")) != HKV_OK) return st;
  if ((st = check_buffer(t, values, n * dim * 4, "values")) != HKV_OK) return st;
  if ((st = check_buffer(t, scores, n * 8, "scores")) != HKV_OK) return st;
  if (found_out && (st = check_buffer(t, found_out, n, "found_out")) != HKV_OK) return st;
  const bool vec4 = dim % 4 == 0 && aligned16(values);
  hkv::InsertCall c{};
  c.keys = keys;
  c.values = values;
  c.scores = scores;
  c.fetch = true;
  c.found = found_out;
  return run_inserter(t, n, c, vec4, "find_or_insert", stream);
}

HKV_API hkv_status hkv_assign(hkv_table* t, uint64_t n, const uint64_t* keys, const float* values,
                              const uint64_t* scores, hipStream_t stream) {
  if (!t) return fail(HKV_EINVAL, "table is NULL");
  if (n == 0) return HKV_OK;
  if (!values && !scores) return fail(HKV_EINVAL, "assign needs values or scores");
  if (n > kMaxBatch) return fail(HKV_EINVAL, "batch of %llu keys exceeds the limit", static_cast<unsigned long long>(n));
  const uint64_t dim = t->opt.dim;
  hkv_status st;
  if ((st = check_buffer(t, keys, n * 8, "keys")) != HKV_OK) return st;
  if (values && (st = check_buffer(t, values, n * dim * 4, "values")) != HKV_OK) return st;
  if (scores && (st = check_buffer(t, scores, n * 8, "scores")) != HKV_OK) return st;
  const bool vec4 = dim % 4 == 0 && (!values || aligned16(values));
  std::lock_guard<std::mutex> lk(t->mu);
  DeviceGuard dg(t->opt.device);
  if (dg.error() != hipSuccess) return fail_hip(dg.error(), "hipSetDevice");
  if ((st = order_before(t, kUpdater, stream)) != HKV_OK) return st;
  const hipError_t e = hkv::launch_assign(t->view, n, keys, values, scores, vec4, stream, t->timer());
  if (e != hipSuccess) return fail_hip(e, "assign launch");
  return record_after(t, kUpdater, stream);
}

HKV_API hkv_status hkv_size(hkv_table* t, uint64_t* out_host, hipStream_t stream) {
  if (!t || !out_host) return fail(HKV_EINVAL, "NULL argument");
  std::lock_guard<std::mutex> lk(t->mu);
  DeviceGuard dg(t->opt.device);
  if (dg.error() != hipSuccess) return fail_hip(dg.error(), "hipSetDevice");
  hkv_status st = order_before(t, kReader, stream);
  if (st != HKV_OK) return st;
  hipError_t e = hkv::launch_size(t->view, t->size_dev, stream, t->timer());
  if (e == hipSuccess)
    e = hipMemcpyAsync(t->size_host, t->size_dev, sizeof(unsigned long long), hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return fail_hip(e, "size launch");
  if ((st = record_after(t, kReader, stream)) != HKV_OK) return st;
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail_hip(e, "hipStreamSynchronize");
  *out_host = *t->size_host;
  return HKV_OK;
}

HKV_API hkv_status hkv_export_batch(hkv_table* t, uint64_t offset, uint64_t n_slots, uint64_t* keys_out,
                                    float* values_out, uint64_t* scores_out, uint64_t* pos_out,
                                    uint64_t* count_out, hipStream_t stream) {
  if (!t) return fail(HKV_EINVAL, "table is NULL");
  const uint64_t cap = t->opt.capacity;
  const uint64_t begin = offset < cap ? offset : cap;
  const uint64_t end = (n_slots > cap - begin) ? cap : begin + n_slots;
  const uint64_t m = end - begin;
  const uint64_t dim = t->opt.dim;
  hkv_status st;
  if ((st = check_buffer(t, count_out, 8, "count_out")) != HKV_OK) return st;
  if (m > 0) {
    if ((st = check_buffer(t, keys_out, m * 8, "keys_out")) != HKV_OK) return st;
    if (values_out && (st = check_buffer(t, values_out, m * dim * 4, "values_out")) != HKV_OK) return st;
    if (scores_out && (st = check_buffer(t, scores_out, m * 8, "scores_out")) != HKV_OK) return st;
    if (pos_out && (st = check_buffer(t, pos_out, m * 8, "pos_out")) != HKV_OK) return st;
  }
  const bool vec4 = dim % 4 == 0 && (!values_out || aligned16(values_out));
  std::lock_guard<std::mutex> lk(t->mu);
  DeviceGuard dg(t->opt.device);
  if (dg.error() != hipSuccess) return fail_hip(dg.error(), "hipSetDevice");
  if ((st = order_before(t, kReader, stream)) != HKV_OK) return st;
  const hipError_t e = hkv::launch_export(t->view, begin, end, keys_out, values_out, scores_out, pos_out,
                                          reinterpret_cast<unsigned long long*>(count_out), vec4, stream,
                                          t->timer());
  if (e != hipSuccess) return fail_hip(e, "export launch");
  return record_after(t, kReader, stream);
}

HKV_API hkv_status hkv_set_outcome_counters(hkv_table* t, uint64_t* counts) {
  if (!t) return fail(HKV_EINVAL, "table is NULL");
  if (counts && (t->opt.flags & HKV_FLAG_SERIAL_INSERT))
    return fail(HKV_EINVAL, "outcome counters: the table inserts serially (HKV_FLAG_SERIAL_INSERT); "
                "they are kept by the parallel inserter only");
  hkv_status st;
  if (counts) {
    if ((st = check_buffer(t, counts, 4 * sizeof(uint64_t), "counts")) != HKV_OK) return st;
    hipPointerAttribute_t a;
    std::memset(&a, 0, sizeof(a));
    if (hipPointerGetAttributes(&a, counts) != hipSuccess || a.type != hipMemoryTypeDevice) {
      (void)hipGetLastError();
      return fail(HKV_EINVAL, "counts (%p) must be device memory of the table's GPU", static_cast<void*>(counts));
    }
    if (reinterpret_cast<uintptr_t>(counts) & 7) return fail(HKV_EINVAL, "counts is not 8-byte aligned");
  }
  std::lock_guard<std::mutex> lk(t->mu);
  DeviceGuard dg(t->opt.device);
  if (dg.error() != hipSuccess) return fail_hip(dg.error(), "hipSetDevice");
  if (counts && !t->stat_slots) {
    // the counting words start at zero; every counted call leaves them so
    const size_t bytes = 4 * hkv::kStatSlots * sizeof(unsigned long long);
    hipError_t e = hipMalloc(&t->stat_slots, bytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      t->stat_slots = nullptr;
      return fail(HKV_ENOMEM, "outcome counters (%zu bytes)", bytes);
    }
    hipStream_t s = nullptr;
    e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
    if (e == hipSuccess) {
      e = hipMemsetAsync(t->stat_slots, 0, bytes, s);
      const hipError_t e2 = hipStreamSynchronize(s);
      if (e == hipSuccess) e = e2;
      (void)hipStreamDestroy(s);
    }
    if (e != hipSuccess) {
      (void)hipFree(t->stat_slots);
      t->stat_slots = nullptr;
      return fail_hip(e, "outcome counters");
    }
  }
  t->outcomes = reinterpret_cast<unsigned long long*>(counts);
  return HKV_OK;
}

HKV_API hkv_status hkv_profile_start(hkv_table* t) {
  if (!t) return fail(HKV_EINVAL, "table is NULL");
  std::lock_guard<std::mutex> lk(t->mu);
  DeviceGuard dg(t->opt.device);
  for (auto& r : t->prof.records()) {
    (void)hipEventSynchronize(r.stop);
    t->prof.give_back(r.start);
    t->prof.give_back(r.stop);
  }
  t->prof.records().clear();
  t->prof.prewarm(kProfileEvents);
  t->profiling = true;
  return HKV_OK;
}

HKV_API hkv_status hkv_profile_stop(hkv_table* t, hkv_kernel_stat* out, uint32_t cap, uint32_t* count) {
  if (!t || !count || (cap && !out)) return fail(HKV_EINVAL, "NULL argument");
  std::lock_guard<std::mutex> lk(t->mu);
  DeviceGuard dg(t->opt.device);
  t->profiling = false;
  std::vector<hkv_kernel_stat> agg;
  std::vector<std::vector<float>> times;  // per entry of agg: every launch's time
  hkv_status st = HKV_OK;
  for (auto& r : t->prof.records()) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess && st == HKV_OK) st = fail_hip(e, "timing event");
    hkv_kernel_stat* a = nullptr;
    size_t ai = 0;
    for (size_t x = 0; x < agg.size(); ++x)
      if (std::strncmp(agg[x].name, r.name, sizeof(agg[x].name)) == 0) {
        a = &agg[x];
        ai = x;
      }
    if (!a) {
      agg.push_back(hkv_kernel_stat{});
      times.emplace_back();
      ai = agg.size() - 1;
      a = &agg.back();
      std::snprintf(a->name, sizeof(a->name), "%s", r.name);
      a->min_ms = ms;
    }
    times[ai].push_back(ms);
    a->launches += 1;
    a->total_ms += ms;
    a->sumsq_ms2 += static_cast<double>(ms) * ms;
    if (ms > a->max_ms) a->max_ms = ms;
    if (ms < a->min_ms) a->min_ms = ms;
    t->prof.give_back(r.start);
    t->prof.give_back(r.stop);
  }
  t->prof.records().clear();
  for (size_t x = 0; x < agg.size(); ++x) {
    std::vector<float>& v = times[x];
    std::nth_element(v.begin(), v.begin() + v.size() / 2, v.end());
    agg[x].median_ms = v[v.size() / 2];
  }
  *count = static_cast<uint32_t>(agg.size());
  for (uint32_t j = 0; j < cap && j < agg.size(); ++j) out[j] = agg[j];
  return st;
}
