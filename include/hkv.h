/*
 * hkv.h - C ABI of a cache-semantic bucketed GPU hash table for gfx950.
 *
 * The table follows "HierarchicalKV: A GPU Hash Table with Cache Semantics for
 * Continuous Online Embedding Storage" (arXiv 2603.17168):
 *   - §3.2 and Figure 4: buckets of 128 slots; each bucket has a contiguous
 *     128-byte line of one-byte digests, 64-bit keys, 64-bit scores and value
 *     rows addressed by (bucket, slot) position; no rehash, chain or stash.
 *   - §3.3, Algorithm 2: a full bucket resolves an upsert in place by evicting
 *     its lowest-score entry or by refusing admission to the incoming key.
 *   - §3.4, Algorithm 3: optional score-based dual-bucket selection.
 *   - §3.5, Table 4: readers (find, find*, contains, size, export), updaters
 *     (assign) and inserters (insert_or_assign, insert_and_evict,
 *     find_or_insert); readers may overlap readers and updaters may overlap
 *     updaters, every other pair is exclusive.
 *   - §4.1: the cache-specific calls find* (pointer-returning find),
 *     contains, insert_and_evict and find_or_insert.
 *   - §3.6 and §4.2: optional placement of value rows in pinned host memory
 *     mapped into the GPU address space, keys/digests/scores staying in HBM,
 *     with an HBM watermark: rows up to the budget stay in HBM, the rest
 *     spill to host memory; a row's address follows from its position.
 *
 * Types: keys and scores are uint64_t, values are float32 rows of `dim`
 * elements stored row-major (n x dim for batches). A full table is the normal
 * operating state, not an error (Definition 2.1, CS1/CS2).
 *
 * Conventions shared by every call below:
 *   - All array arguments are caller-owned, contiguous, and must be readable
 *     (inputs) or writable (outputs) by the table's GPU: device memory or
 *     pinned/mapped host memory. Pageable host pointers are rejected with
 *     HKV_EINVAL before anything is enqueued.
 *   - Calls are asynchronous on `stream` (0 = the null stream) except
 *     hkv_size. Inputs must stay valid and outputs unread until the stream has
 *     passed the call.
 *   - Group ordering (§3.5, Table 4) is enforced with stream/event ordering:
 *     a call waits, on its own stream, for every outstanding call of an
 *     incompatible group issued earlier on another stream. The host does not
 *     block for this, with one exception: while all calls on a table come
 *     from a single stream they record no events (stream order suffices), so
 *     the first call from a second stream waits once for the device
 *     (hipDeviceSynchronize). Several host threads may call concurrently.
 *     The table keeps the last event it recorded on each stream, and later
 *     calls from other streams query or wait on it; an event refers to the
 *     stream it was recorded on, so a stream that has carried calls on a
 *     table used from several streams must stay alive until the table is
 *     destroyed (likewise the streams of calls timed by hkv_profile_start,
 *     until hkv_profile_stop).
 *   - The calls may be captured into a HIP graph when every call on the table
 *     is issued on the capturing stream and, for each inserter call captured,
 *     a call of the same kind with at least as many keys ran before the
 *     capture (inserters grow their workspaces on demand, which a capture
 *     cannot do; hkv_insert_or_assign_noalloc needs no such call). A captured
 *     call keeps the outcome-counter setting it was captured with.
 *   - Arguments are validated synchronously; on any error nothing is enqueued,
 *     the call returns a negative status and hkv_last_error() describes it.
 *   - n == 0 is a valid no-op. Batches are limited to n <= 2^32 - 4 keys.
 *   - The reserved keys HKV_EMPTY_KEY and HKV_LOCKED_KEY always miss in the
 *     readers and are skipped by the updaters and inserters.
 *   - No C++ exception crosses this boundary.
 *   - Two environment variables, read by hkv_create, override launch shapes
 *     for tuning; results do not depend on them. HKV_GROUP_LANES: lanes that
 *     serve one key in the probing kernels (4, 8 or 16; any other value keeps
 *     the default chosen from dim). HKV_KEYS_PER_GROUP: keys each group serves
 *     in the key-side probes of hkv_find_ptr and hkv_contains (1, 2 or 4;
 *     default 2). A third, HKV_EPOCH_START, sets the table's inserter-call
 *     counter (it tags the chain heads and wraps after 2^32 - 1 calls; calls
 *     captured into a graph use epoch 0 instead) to a start value, so that
 *     tests can reach the wrap quickly.
 */
#ifndef HKV_H_
#define HKV_H_

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct hkv_table hkv_table;
typedef int32_t hkv_status;

#define HKV_OK 0
#define HKV_EINVAL (-1)       /* bad argument (null, size, alignment, pointer kind) */
#define HKV_ENOMEM (-2)       /* device or pinned host allocation failed */
#define HKV_EHIP (-3)         /* a HIP runtime call or kernel launch failed */
#define HKV_EUNSUPPORTED (-4) /* valid request the library does not implement */

#define HKV_BUCKET_SLOTS 128u
/* Reserved key values: an empty slot and the slot-lock sentinel (§4.4). */
#define HKV_EMPTY_KEY 0xFFFFFFFFFFFFFFFFull
#define HKV_LOCKED_KEY 0xFFFFFFFFFFFFFFFEull

/* Option flags. */
/* The inserter applies a batch one key at a time, in input order, in a single
 * group of lanes. Slow; gives run-to-run identical slot placement and, in
 * dual-bucket mode, exactly Algorithm 3's sequential decisions. */
#define HKV_FLAG_SERIAL_INSERT 0x1u
/* Conventional reader/writer ordering instead of the three groups (the
 * baseline of the paper's concurrency ablation, §5.4): readers may overlap
 * readers, every updater and inserter call is exclusive. */
#define HKV_FLAG_RW_LOCK 0x2u
/* The caller guarantees that the keys of every write batch (insert_or_assign,
 * insert_and_evict) are distinct, as the paper's benchmarks and the DynamicEmb
 * API's unique-key inputs have them. The inserter then takes no per-slot claim
 * when it updates a resident key in place (one device atomic per update
 * saved). A batch that breaks the promise still leaves every key resident at
 * most once, but a duplicated resident key's row may combine 16-byte pieces
 * of several occurrences. */
#define HKV_FLAG_UNIQUE_KEYS 0x4u

typedef struct hkv_options {
  uint64_t capacity;        /* slots; a positive multiple of 128 (§3.2). B = capacity / 128 buckets,
                               at most 2^31 - 1 */
  uint32_t dim;             /* float32 elements per value row, 1 .. 2^20 */
  uint32_t bucket_slots;    /* must be 128 (or 0, meaning 128) */
  uint32_t dual_bucket;     /* 0: single-bucket (§3.2); 1: score-based dual-bucket (§3.4) */
  uint32_t values_on_host;  /* 0: value rows in HBM; 1: in pinned, GPU-mapped host memory (§3.6),
                               except the first hbm_value_bytes' worth (§4.2 watermark) */
  int32_t device;           /* HIP device ordinal that owns the table */
  uint32_t flags;           /* HKV_FLAG_* */
  uint64_t hbm_value_bytes; /* values_on_host == 1 only: HBM budget for value rows (the §4.2
                               watermark). The rows of the first
                               floor(hbm_value_bytes / (128 * 4 * dim)) buckets live in HBM,
                               the rest in pinned host memory; 0 = all rows on the host,
                               >= 4 * dim * capacity = all in HBM. Ignored when values_on_host
                               == 0 (all rows in HBM). */
} hkv_options;

/*
 * hkv_create - allocate an empty table (§3.2 layout, §4.2 placement).
 * Storage per slot: key 8 B + score 8 B + digest 1 B in HBM (§5.1, memory
 * overhead), plus a value row of 4*dim bytes in HBM or in pinned host memory
 * (split at a bucket boundary by hbm_value_bytes, see hkv_options). Per
 * bucket, 28 bytes of bookkeeping in HBM (occupancy 4, inserter chain head 8,
 * one claim bit per slot) and, in dual-bucket mode, 16 more (its lowest entry).
 * Every slot starts empty. The table owns all of its storage.
 * Errors: HKV_EINVAL (null arguments, capacity not a positive multiple of 128
 * or above 2^31 - 1 buckets, dim outside 1 .. 2^20, bucket_slots not 128, bad
 * device), HKV_ENOMEM, HKV_EHIP.
 * On error *out is set to NULL.
 */
hkv_status hkv_create(const hkv_options* options, hkv_table** out);

/* hkv_destroy - end of the table's lifetime: waits for the table's
 * outstanding work on every stream, then frees all storage hkv_create
 * allocated (the §3.2 bucket arrays, the §3.6 host-memory value rows) and the
 * inserter workspaces. The paper's API (§4.1) is that of a container object
 * and names no explicit teardown call; releasing everything the table owns
 * at its end is the reading taken here. NULL is accepted and ignored; the
 * handle must not be used afterwards. Always returns HKV_OK. */
hkv_status hkv_destroy(hkv_table* table);

/* hkv_get_options - copy the options the table was created with. */
hkv_status hkv_get_options(const hkv_table* table, hkv_options* out);

/*
 * hkv_find - reader (§3.2, Algorithm 1; dual buckets per §3.4).
 * For each i < n: if keys[i] is resident, copies its value row to
 * values_out[i*dim .. i*dim+dim), sets found_out[i] = 1 and, when scores_out is
 * not NULL, scores_out[i] = its score. Otherwise sets found_out[i] = 0 and
 * leaves values_out's row and scores_out[i] untouched. Scores in the table are
 * never modified. Duplicate keys in the batch are allowed.
 *   keys       [n] uint64, input
 *   values_out [n*dim] float32, output (16-byte alignment enables wide copies)
 *   found_out  [n] uint8, output
 *   scores_out [n] uint64, output, nullable
 */
hkv_status hkv_find(hkv_table* table, uint64_t n, const uint64_t* keys, float* values_out,
                    uint8_t* found_out, uint64_t* scores_out, hipStream_t stream);

/*
 * hkv_insert_or_assign - inserter (§3.3, Algorithm 2; §3.4, Algorithm 3).
 * For each non-reserved key: if resident, its value row and score are
 * overwritten; else it is written to an empty slot of its bucket (dual mode:
 * of the less-occupied candidate bucket); else the lowest-ranked entry of the
 * full bucket (dual mode: of the two buckets, the lower one) is evicted if the
 * incoming key ranks higher, and the key is rejected otherwise. Rank is the
 * pair (score, key) ordered lexicographically, which fixes ties. None of these
 * outcomes is an error.
 * Keys within one batch must be distinct for a deterministic result. With
 * duplicates, the key ends up stored (or not) as if exactly one of its
 * occurrences had been applied, whole: its row and score come from that one
 * occurrence, which one is unspecified, and the key is resident at most once
 * (unless the table was created with HKV_FLAG_UNIQUE_KEYS, see there).
 * For single-bucket tables and batches of distinct keys whose
 * scores never decrease over time, the resulting bucket contents equal those
 * of applying the batch one key at a time, whatever the in-batch order.
 *   keys   [n] uint64, input
 *   values [n*dim] float32, input
 *   scores [n] uint64, input, required
 * The call uses a table-owned workspace of 8*n bytes, grown on demand.
 */
hkv_status hkv_insert_or_assign(hkv_table* table, uint64_t n, const uint64_t* keys,
                                const float* values, const uint64_t* scores,
                                hipStream_t stream);

/*
 * hkv_insert_or_assign_noalloc - hkv_insert_or_assign for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments, result and ordering as
 * hkv_insert_or_assign, but the per-key scratch of its kernels (8 bytes per
 * key) is a fixed array that the library holds in each GPU's memory for the
 * life of the process (HKV_NOALLOC_MAX_KEYS keys, 16 MiB), instead of the
 * table-owned workspace that hkv_insert_or_assign grows with hipMalloc; the
 * call allocates nothing.
 * Limits: n > HKV_NOALLOC_MAX_KEYS is HKV_EINVAL. Every no-alloc call on one
 * GPU, from any table, uses that GPU's one array: calls that overlap on a
 * GPU (different streams without ordering between them) race, so order them.
 * On a table used from several streams, the stream must already have issued
 * an inserter call (which creates its ordering event), else HKV_EINVAL.
 */
#define HKV_NOALLOC_MAX_KEYS (1ull << 21)
hkv_status hkv_insert_or_assign_noalloc(hkv_table* table, uint64_t n, const uint64_t* keys,
                                        const float* values, const uint64_t* scores, hipStream_t stream);

/*
 * hkv_assign - updater (§3.5): overwrites the value row (when values is not
 * NULL) and the score (when scores is not NULL) of keys already resident.
 * Absent and reserved keys are ignored; the bucket structure never changes.
 * values and scores may not both be NULL (HKV_EINVAL).
 * Keys within one batch should be distinct. Every occurrence of a duplicated
 * key writes in place, as concurrent updater calls on different streams do
 * (§3.5 lets updaters overlap and takes no lock for them): its score is one
 * occurrence's, and with dim > 4 its row may combine 16-byte pieces of
 * several occurrences.
 *   keys   [n] uint64, input
 *   values [n*dim] float32, input, nullable
 *   scores [n] uint64, input, nullable
 */
hkv_status hkv_assign(hkv_table* table, uint64_t n, const uint64_t* keys, const float* values,
                      const uint64_t* scores, hipStream_t stream);

/*
 * hkv_find_ptr - reader, the pointer-returning find* of §4.1 (measured in
 * §5.3). For each i < n: if keys[i] is resident, values_ptr_out[i] = the
 * address of its value row (device memory, or the GPU-mapped address of the
 * host row when values live in host memory; rows are addressed by position,
 * §3.6), found_out[i] = 1 and scores_out[i] = its score; otherwise
 * values_ptr_out[i] = NULL, found_out[i] = 0 and scores_out[i] is untouched.
 * A returned address stays the key's row until the next inserter call on the
 * table (which may evict the key and reuse the slot); updaters change the
 * row's contents in place.
 *   keys           [n] uint64, input
 *   values_ptr_out [n] float*, output
 *   found_out      [n] uint8, output, nullable
 *   scores_out     [n] uint64, output, nullable
 */
hkv_status hkv_find_ptr(hkv_table* table, uint64_t n, const uint64_t* keys, float** values_ptr_out,
                        uint8_t* found_out, uint64_t* scores_out, hipStream_t stream);

/*
 * hkv_contains - reader (§3.5, §4.1): found_out[i] = 1 iff keys[i] is
 * resident, else 0. Nothing else is read or written.
 *   keys      [n] uint64, input
 *   found_out [n] uint8, output
 */
hkv_status hkv_contains(hkv_table* table, uint64_t n, const uint64_t* keys, uint8_t* found_out,
                        hipStream_t stream);

/*
 * hkv_insert_and_evict - inserter (§4.1): insert_or_assign that also hands
 * back what leaves. Order inside the call: keys resident when the call starts
 * are updated first (row and score), then the other keys are inserted as by
 * insert_or_assign. Handed back, compacted in unspecified order: every
 * resident entry an insertion evicts (with the key, row and score it held) and
 * every offered entry that admission turns away (with the offered row and
 * score). So the output is exactly the entries that were resident before the
 * call or offered by it and are not resident after it. *evicted_count (a
 * device-accessible uint64, reset by the call itself) receives how many; it is
 * at most the number of keys not resident at the start, so outputs of n
 * entries always suffice. Same distinct-key and determinism rules as
 * insert_or_assign.
 *   keys             [n] uint64, input
 *   values           [n*dim] float32, input
 *   scores           [n] uint64, input, required
 *   evicted_keys     [n] uint64, output
 *   evicted_values   [n*dim] float32, output, nullable
 *   evicted_scores   [n] uint64, output, nullable
 *   evicted_count    [1] uint64, output
 * Uses the same table-owned workspace as insert_or_assign plus a staging area
 * of (17 + 4*dim)*n bytes, both grown on demand.
 */
hkv_status hkv_insert_and_evict(hkv_table* table, uint64_t n, const uint64_t* keys, const float* values,
                                const uint64_t* scores, uint64_t* evicted_keys, float* evicted_values,
                                uint64_t* evicted_scores, uint64_t* evicted_count, hipStream_t stream);

/*
 * hkv_find_or_insert - inserter (§3.5, §4.1): lookup combined with insertion
 * for cold starts. A key resident when the call starts is a hit: its stored
 * row is written to values[i*dim ..), its score is replaced by scores[i] and
 * found_out[i] = 1. Every other key is inserted with the caller's row and
 * score exactly as insert_or_assign inserts it (it may evict, or be turned
 * away); found_out[i] = 0 and its row in values is left as it was.
 *   keys      [n] uint64, input
 *   values    [n*dim] float32, input and output
 *   scores    [n] uint64, input, required
 *   found_out [n] uint8, output, nullable
 * Uses the same table-owned workspace as insert_or_assign.
 */
hkv_status hkv_find_or_insert(hkv_table* table, uint64_t n, const uint64_t* keys, float* values,
                              const uint64_t* scores, uint8_t* found_out, hipStream_t stream);

/*
 * hkv_size - reader (§3.5): number of resident entries. Enqueues the count on
 * `stream`, synchronizes that stream, and stores the result in *out_host.
 */
hkv_status hkv_size(hkv_table* table, uint64_t* out_host, hipStream_t stream);

/*
 * hkv_export_batch - reader (§4.1, export for checkpointing): scans slot
 * positions p in [offset, offset + n_slots) clipped to [0, capacity), where
 * p = bucket * 128 + slot, and writes every occupied one, compacted, to the
 * outputs: keys_out[j], values_out[j*dim ..), scores_out[j], pos_out[j] = p.
 * *count_out (a device-accessible uint64) receives the number written; it is
 * reset by the call itself. Output order is unspecified. Outputs must hold
 * n_slots entries (clipped). values_out, scores_out and pos_out are nullable.
 */
hkv_status hkv_export_batch(hkv_table* table, uint64_t offset, uint64_t n_slots,
                            uint64_t* keys_out, float* values_out, uint64_t* scores_out,
                            uint64_t* pos_out, uint64_t* count_out, hipStream_t stream);

/*
 * hkv_set_outcome_counters - optional outcome counts of the inserter calls
 * (a metrics aid the paper's API does not have; the DynamicEmb API page, in
 * its DynamicEmbCheckMode section, counts the keys a lookup could not
 * insert, which is `rejected` below).
 * After this call, every insert_or_assign (and its no-alloc variant),
 * insert_and_evict and find_or_insert on the table adds to counts[0..3]:
 *   counts[0] updated:  keys of the batch resident when the call started
 *                       (updated in place, or their stored row returned by
 *                       find_or_insert);
 *   counts[1] inserted: keys absent when the call started, resident at its end;
 *   counts[2] evicted:  keys resident when the call started, absent at its end;
 *   counts[3] rejected: keys of the batch absent when the call started and at
 *                       its end (turned away by admission, or admitted and
 *                       displaced by a later key of the same call).
 * So size after = size before + inserted - evicted. For batches of distinct
 * keys these are properties of the call's start and end states alone. With a
 * key repeated in a batch, updated counts it once in insert_or_assign and
 * insert_and_evict, once per occurrence in find_or_insert; rejected counts a
 * key again when an occurrence arrives after its earlier one was displaced.
 * The reserved keys, which every inserter skips, count in none of the four.
 * counts: 4 uint64 in device memory of the table's GPU, owned by the caller
 * and valid while set; the calls add to them (zero them to start) with
 * device atomics, after the call's other kernels, on the call's stream.
 * NULL turns counting off. Counting adds one small kernel per call.
 * Errors: HKV_EINVAL (NULL table, counts not device memory of that GPU or
 * shorter than 32 bytes, a table with HKV_FLAG_SERIAL_INSERT), HKV_ENOMEM
 * (the table's 8 KiB of counting words, allocated on the first call).
 */
hkv_status hkv_set_outcome_counters(hkv_table* table, uint64_t* counts);

/*
 * Kernel timing (tracing aid; not part of the paper's API).
 * While profiling is on, every kernel the table launches carries a start and
 * a stop event that its own dispatch records (hipExtLaunchKernelGGL), so no
 * extra work is queued on the stream; a record's time is the elapsed time
 * between them.
 */
typedef struct hkv_kernel_stat {
  char name[32];      /* find, find_ptr, contains, assign, upsert_probe, probe_fetch, upsert_owner,
                         owner_evict, evict_count, evict_write, outcomes, upsert_serial, size,
                         export, zero */
  uint64_t launches;  /* timed launches of that kernel */
  double total_ms;    /* sum of their times */
  double max_ms;      /* longest one */
  double min_ms;      /* shortest one */
  double sumsq_ms2;   /* sum of their squared times (spread across launches) */
  double median_ms;   /* median launch time (upper median for an even count): unlike the
                         average, not moved by a few launches whose start event was taken
                         before the kernel was dispatched */
} hkv_kernel_stat;

/* hkv_profile_start - discards earlier records and turns timing on. The
 * timing events are created (a pool of 512, grown if needed) and recorded
 * once here, so that none is created during the timed launches. */
hkv_status hkv_profile_start(hkv_table* table);

/* hkv_profile_stop - turns timing off, waits for every timed launch, writes
 * one record per kernel name to out[0 .. min(cap, *count)) and the number of
 * distinct kernels to *count. out may be NULL when cap == 0. */
hkv_status hkv_profile_stop(hkv_table* table, hkv_kernel_stat* out, uint32_t cap, uint32_t* count);

/* hkv_last_error - description of the last failure on the calling thread. */
const char* hkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HKV_H_ */
