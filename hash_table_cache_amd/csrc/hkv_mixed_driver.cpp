// Multi-threaded driver of the mixed reader / updater / inserter workload of
// the concurrency ablation in §5.4 of "HierarchicalKV: A GPU Hash Table with
// Cache Semantics for Continuous Online Embedding Storage": several host
// threads share one table, each issuing back-to-back batches of one role on
// a stream of its own, with the table's group ordering (§3.5, Table 4, or
// the reader/writer baseline when the table was created with
// HKV_FLAG_RW_LOCK) deciding which calls may overlap on the GPU.
//
// A benchmark harness, built as its own library (libhkv_mixed.so) on top of
// the C ABI; it adds nothing to the table itself.
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cstdint>
#include <map>
#include <mutex>
#include <thread>
#include <vector>

#include "hkv.h"

#define HKV_MIXED_API extern "C" __attribute__((visibility("default")))

namespace {

enum Role { kFind = 0, kAssign = 1, kInsert = 2 };

struct ThreadArgs {
  int32_t role;
  const uint64_t* keys;    // pool * batch
  const float* values;     // pool * batch * dim (assign, insert)
  const uint64_t* scores;  // pool * batch (assign, insert)
  float* out;              // batch * dim (find)
  uint8_t* found;          // batch (find)
};

// The worker streams, per device, created on first use and kept for the
// process: a table keeps the last event it recorded on each stream and
// queries or waits on it in later calls, so the streams its calls ran on
// stay alive (and their handles stable from one run to the next).
std::mutex g_streams_mu;
std::map<int, std::vector<hipStream_t>> g_streams;

hipError_t worker_streams(int device, uint32_t count, std::vector<hipStream_t>* out) {
  std::lock_guard<std::mutex> lk(g_streams_mu);
  std::vector<hipStream_t>& v = g_streams[device];
  int prev = -1;
  hipError_t e = hipGetDevice(&prev);
  if (e == hipSuccess) e = hipSetDevice(device);
  while (e == hipSuccess && v.size() < count) {
    hipStream_t s = nullptr;
    e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
    if (e == hipSuccess) v.push_back(s);
  }
  if (prev >= 0) (void)hipSetDevice(prev);
  if (e != hipSuccess) return e;
  out->assign(v.begin(), v.begin() + count);
  return hipSuccess;
}

}  // namespace

// Runs `threads` host threads. Thread j issues `batches` calls of role
// roles[j] (0 find, 1 assign, 2 insert_or_assign) on stream j of the
// driver's worker streams (created once per device and kept), cycling
// through `pool` pre-made device batches of `batch` keys: batch b uses
// keys[j] + (b % pool) * batch, and likewise for values and scores. find
// writes its rows and flags to out[j] / found[j]. All threads start together;
// *seconds receives the wall time from the start until every thread's stream
// has drained. Returns HKV_OK or the first failing call's status.
HKV_MIXED_API hkv_status hkv_mixed_run(hkv_table* table, uint32_t threads, const int32_t* roles,
                                       uint32_t batches, uint64_t batch, uint32_t pool,
                                       const uint64_t* const* keys, const float* const* values,
                                       const uint64_t* const* scores, float* const* out,
                                       uint8_t* const* found, double* seconds) {
  if (!table || !roles || !keys || !seconds || threads == 0 || pool == 0) return HKV_EINVAL;
  hkv_options opt;
  hkv_status st = hkv_get_options(table, &opt);
  if (st != HKV_OK) return st;
  const uint64_t dim = opt.dim;
  std::vector<ThreadArgs> args(threads);
  for (uint32_t j = 0; j < threads; ++j) {
    args[j].role = roles[j];
    if (roles[j] < kFind || roles[j] > kInsert) return HKV_EINVAL;
    args[j].keys = keys[j];
    args[j].values = values ? values[j] : nullptr;
    args[j].scores = scores ? scores[j] : nullptr;
    args[j].out = out ? out[j] : nullptr;
    args[j].found = found ? found[j] : nullptr;
    // every role's own buffers must be given (the library itself checks
    // that they are device-accessible and large enough)
    if (!args[j].keys) return HKV_EINVAL;
    if (roles[j] == kFind && (!args[j].out || !args[j].found)) return HKV_EINVAL;
    if (roles[j] != kFind && (!args[j].values || !args[j].scores)) return HKV_EINVAL;
  }
  std::vector<hipStream_t> streams;
  if (worker_streams(opt.device, threads, &streams) != hipSuccess) return HKV_EHIP;
  std::atomic<uint32_t> ready{0};
  std::atomic<bool> go{false};
  std::vector<hkv_status> result(threads, HKV_OK);
  std::vector<std::thread> pool_threads;
  pool_threads.reserve(threads);
  for (uint32_t j = 0; j < threads; ++j) {
    pool_threads.emplace_back([&, j]() {
      const ThreadArgs& a = args[j];
      const hipStream_t s = streams[j];
      if (hipSetDevice(opt.device) != hipSuccess) {
        result[j] = HKV_EHIP;
        ready.fetch_add(1);
        return;
      }
      ready.fetch_add(1);
      while (!go.load(std::memory_order_acquire)) std::this_thread::yield();
      for (uint32_t b = 0; b < batches && result[j] == HKV_OK; ++b) {
        const uint64_t off = static_cast<uint64_t>(b % pool) * batch;
        const uint64_t* k = a.keys + off;
        switch (a.role) {
          case kFind:
            result[j] = hkv_find(table, batch, k, a.out, a.found, nullptr, s);
            break;
          case kAssign:
            result[j] = hkv_assign(table, batch, k, a.values + off * dim, a.scores + off, s);
            break;
          default:
            result[j] = hkv_insert_or_assign(table, batch, k, a.values + off * dim, a.scores + off, s);
        }
      }
      if (hipStreamSynchronize(s) != hipSuccess && result[j] == HKV_OK) result[j] = HKV_EHIP;
    });
  }
  while (ready.load() < threads) std::this_thread::yield();
  const auto t0 = std::chrono::steady_clock::now();
  go.store(true, std::memory_order_release);
  for (auto& th : pool_threads) th.join();
  *seconds = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
  for (hkv_status r : result)
    if (r != HKV_OK) return r;
  return HKV_OK;
}
