// Internal interface between the host runtime (hkv_runtime.cpp) and the
// gfx950 kernels (hkv_kernels.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace hkv {

// Device-side view of one table. Slot s of bucket b is position p = b*128 + s
// in digests/keys/scores and value row p (dim floats).
struct TableView {
  uint8_t* digests;   // [nb*128]  one-byte digest per slot; 0 marks an empty slot
  uint64_t* keys;     // [nb*128]
  uint64_t* scores;   // [nb*128]
  float* values;      // rows [0, split): HBM, or host-mapped pinned memory
  float* values_hi;   // rows [split, nb*128): host-mapped pinned memory, base
                      // offset by -split rows (row p at values_hi + p*dim)
  uint64_t split;     // first position whose row is in the second region
  uint32_t* occ;      // [nb]  occupied slots; slots [0, occ) are the occupied ones
  uint64_t* head;     // [nb]  inserter chain heads: low word the batch index last
                      // pushed, high word the epoch of the call that pushed it; a
                      // head of another epoch is an empty chain (reset only by
                      // calls captured into a graph, which run at epoch 0)
  uint64_t* bmin;     // [2*nb] dual mode: lowest (score, key) of each full bucket
                      // as its last owner left it; key ~0 = not known
  uint32_t* claim;    // [nb*4] one bit per slot (bit p%32 of word p/32): taken by the
                      // occurrence of a resident key that updates it in an inserter
                      // call, so one occurrence alone writes the row and score;
                      // all 0 between calls
  uint64_t nb;        // number of buckets
  uint64_t nb_mask;   // nb - 1 when nb is a power of two
  uint32_t dim;
  uint32_t pow2;      // nb is a power of two
  uint32_t dual;      // dual-bucket mode
  uint32_t lanes;     // lanes per key of find/assign/insert probes; 0 = by dim
  uint32_t keys_per_group;  // keys each group of the key-side probes serves (1, 2 or 4)
  uint32_t claims;    // inserters claim slots they update in place (0: the caller
                      // promised distinct keys per write batch)
  uint32_t epoch;     // this inserter call's epoch (1 .. 2^32-1; 0 for calls
                      // captured into a graph)
};

// Optional per-kernel timing: when a timer is passed, each kernel is launched
// with hipExtLaunchKernelGGL and a start/stop event pair taken from the timer,
// so the timestamps are written by the dispatch itself (no extra packets on
// the stream); launched() hands the pair back with the kernel's name.
struct KernelTimer {
  virtual bool take(hipEvent_t* start, hipEvent_t* stop) = 0;
  virtual void launched(const char* kernel, hipEvent_t start, hipEvent_t stop) = 0;

 protected:
  ~KernelTimer() = default;
};

// Row copies use 16-byte vectors when dim % 4 == 0 and every row pointer
// involved is 16-byte aligned; the host decides and passes `vec4`.

hipError_t launch_init(const TableView& t, hipStream_t s);

// Sets every chain head to the empty head (epoch 0, no index), when the
// epoch counter wraps.
hipError_t launch_reset_heads(const TableView& t, hipStream_t s);

// Device address, on the current device, of the library's fixed scratch array
// for calls that may not allocate, and its capacity in keys (the array holds
// 2 u32 words per key: next, then target).
hipError_t scratch_address(uint32_t** out);
uint64_t noalloc_max_keys();

hipError_t launch_find(const TableView& t, uint64_t n, const uint64_t* keys, float* values_out,
                       uint8_t* found_out, uint64_t* scores_out, bool vec4, hipStream_t s,
                       KernelTimer* timer);

hipError_t launch_assign(const TableView& t, uint64_t n, const uint64_t* keys,
                         const float* values, const uint64_t* scores, bool vec4, hipStream_t s,
                         KernelTimer* timer);

// find* / contains: every output optional (ptrs: one u64 address per key).
hipError_t launch_locate(const TableView& t, uint64_t n, const uint64_t* keys, uint64_t* ptrs_out,
                         uint8_t* found_out, uint64_t* scores_out, hipStream_t s, KernelTimer* timer);

// Arguments of the inserter calls. insert_or_assign: keys, values, scores.
// find_or_insert: fetch = true, values is in/out, found optional.
// insert_and_evict: ev_keys/ev_count set (ev_values, ev_scores optional);
// ev_count is zeroed by the launch.
// Outcome counters: each of the four counts (updated, inserted, evicted,
// rejected) is accumulated over kStatSlots device words (block b adds to word
// b mod kStatSlots) and summed into the caller's counters at the end of the
// call, which also clears the words.
constexpr int kStatSlots = 256;

struct InsertCall {
  const uint64_t* keys;
  float* values;
  const uint64_t* scores;
  bool fetch;
  uint8_t* found;
  uint64_t* ev_keys;
  float* ev_values;
  uint64_t* ev_scores;
  unsigned long long* ev_count;
  // insert_and_evict, parallel inserter: staging of n entries (kind [n] u8,
  // keys and scores [n] u64, rows [n*dim] f32)
  uint8_t* st_kind;
  uint64_t* st_keys;
  uint64_t* st_scores;
  float* st_rows;
  uint32_t* chunk_count;  // [ceil(n / 1024)]
  // outcome counters (parallel inserter): the table's 4 * kStatSlots words,
  // all zero between calls, and the caller's 4 counters; nullptr: not counted
  unsigned long long* stat_slots;
  unsigned long long* outcomes;
};

// next, target: [n] u32 workspaces (not used by insert_or_assign in serial mode).
hipError_t launch_upsert(const TableView& t, uint64_t n, const InsertCall& c, uint32_t* next,
                         uint32_t* target, bool vec4, bool serial, hipStream_t s, KernelTimer* timer);

// Writes the number of occupied slots to *dev_out (device memory).
hipError_t launch_size(const TableView& t, unsigned long long* dev_out, hipStream_t s,
                       KernelTimer* timer);

hipError_t launch_export(const TableView& t, uint64_t begin, uint64_t end, uint64_t* keys_out,
                         float* values_out, uint64_t* scores_out, uint64_t* pos_out,
                         unsigned long long* count_out, bool vec4, hipStream_t s,
                         KernelTimer* timer);

}  // namespace hkv
