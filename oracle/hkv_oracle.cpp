// CPU oracle for the cache-semantic bucketed hash table.
//
// TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or
// calls this file. Only the tests, the smoke check and the CPU-baseline leg
// of the benchmark use it. It shares no code, header, table or constant
// generator with the HIP implementation.
//
// What it computes follows the paper "HierarchicalKV: A GPU Hash Table with
// Cache Semantics for Continuous Online Embedding Storage" (arXiv 2603.17168):
//   - §3.2, Algorithm 1: digest-accelerated find over one 128-slot bucket.
//   - §3.3, Algorithm 2: upsert with bucket-local admission and eviction.
//   - §3.4, Algorithm 3: score-based dual-bucket upsert (phases D1 and D2).
//   - §3.5: updaters (assign) change values/scores of present keys only;
//     readers never write.
//   - §4.1: export of resident entries for checkpointing.
// Where the paper leaves a step open, the reading taken is written next to the
// code that implements it.
//
// It is deliberately plain: single-threaded loops over whole buckets, one key
// at a time, in input order. No blocking, no fusion, no reordering.
//
// Parity status of each function (what pins it) is stated in the test suite;
// the routing hash is pinned through MurmurHash3_x64_128's published SMHasher
// verification value, which exercises the same 64-bit finalizer.

#include <cstdint>
#include <new>
#include <vector>

namespace {

constexpr int kSlots = 128;  // bucket width (§3.2: 128 one-byte digests = one 128 B line)

// Reserved key values. The paper's key-level CAS (§4.4) swaps a key with a
// lock sentinel, and Algorithm 2 writes new keys into an empty slot, but it
// gives neither value. Reading: all-ones marks an empty slot and
// all-ones minus one is the lock sentinel; neither may be stored by a caller.
constexpr uint64_t kEmptyKey = ~0ull;
constexpr uint64_t kLockedKey = ~0ull - 1;

// Reading for the dual-bucket second hash (§3.4 only asks that the two hashes
// be independent): the same finalizer applied to the key xor floor(2^64 / phi).
constexpr uint64_t kSecondHashSalt = 0x9E3779B97F4A7C15ull;

enum Outcome : uint32_t {
  kSkipped = 0,   // reserved key, ignored
  kUpdated = 1,   // key was present: value and score overwritten
  kInserted = 2,  // written into an empty slot
  kEvicted = 3,   // replaced the lowest-ranked resident of a full bucket
  kRejected = 4,  // admission control refused it
};

bool is_reserved(uint64_t k) { return k == kEmptyKey || k == kLockedKey; }

// MurmurHash3's 64-bit finalizer (Appleby, SMHasher, public domain): three
// xor-shift-right-by-33 steps around two multiplications by odd constants.
// The paper calls its hash a GPU-optimized variant of Murmur3 (§3.1, §3.2)
// without giving it; this finalizer is the reading taken.
uint64_t fmix64(uint64_t k) {
  k ^= k >> 33;
  k *= 0xff51afd7ed558ccdull;
  k ^= k >> 33;
  k *= 0xc4ceb9fe1a85ec53ull;
  k ^= k >> 33;
  return k;
}

uint64_t rotl64(uint64_t x, int r) { return (x << r) | (x >> (64 - r)); }

uint64_t load_le64(const uint8_t* p) {
  uint64_t v = 0;
  for (int i = 7; i >= 0; --i) v = (v << 8) | p[i];
  return v;
}

// MurmurHash3_x64_128 (Appleby, SMHasher). Not used by the table; it exists so
// that a test can check fmix64 against SMHasher's published verification
// value for this hash, which runs every output through fmix64.
void murmur3_x64_128(const uint8_t* data, uint64_t len, uint32_t seed, uint64_t out[2]) {
  const uint64_t c1 = 0x87c37b91114253d5ull;
  const uint64_t c2 = 0x4cf5ad432745937full;
  uint64_t h1 = seed, h2 = seed;
  const uint64_t nblocks = len / 16;
  for (uint64_t i = 0; i < nblocks; ++i) {
    uint64_t k1 = load_le64(data + 16 * i);
    uint64_t k2 = load_le64(data + 16 * i + 8);
    k1 *= c1; k1 = rotl64(k1, 31); k1 *= c2; h1 ^= k1;
    h1 = rotl64(h1, 27); h1 += h2; h1 = h1 * 5 + 0x52dce729;
    k2 *= c2; k2 = rotl64(k2, 33); k2 *= c1; h2 ^= k2;
    h2 = rotl64(h2, 31); h2 += h1; h2 = h2 * 5 + 0x38495ab5;
  }
  const uint8_t* tail = data + 16 * nblocks;
  const uint64_t rem = len & 15;
  uint64_t k1 = 0, k2 = 0;
  for (uint64_t i = rem; i > 8; --i) k2 = (k2 << 8) | tail[i - 1];
  if (rem > 8) { k2 *= c2; k2 = rotl64(k2, 33); k2 *= c1; h2 ^= k2; }
  for (uint64_t i = (rem < 8 ? rem : 8); i > 0; --i) k1 = (k1 << 8) | tail[i - 1];
  if (rem > 0) { k1 *= c1; k1 = rotl64(k1, 31); k1 *= c2; h1 ^= k1; }
  h1 ^= len; h2 ^= len;
  h1 += h2; h2 += h1;
  h1 = fmix64(h1); h2 = fmix64(h2);
  h1 += h2; h2 += h1;
  out[0] = h1; out[1] = h2;
}

struct Route {
  uint64_t b1;  // primary bucket: Hash(k) mod B (Algorithm 1)
  uint64_t b2;  // second candidate (dual mode only, else == b1)
  uint8_t d;    // 8-bit digest
};

struct Table {
  uint64_t capacity = 0;
  uint64_t buckets = 0;
  uint32_t dim = 0;
  bool dual = false;
  bool tag_mode = false;  // store one u64 tag per slot instead of dim floats

  // Slot s of bucket b lives at position p = b * 128 + s in every array.
  std::vector<uint64_t> key;
  std::vector<uint64_t> score;
  std::vector<uint8_t> digest;
  std::vector<float> value;   // capacity * dim (value mode)
  std::vector<uint64_t> tag;  // capacity (tag mode)

  // Instrumentation for the false-positive statistic of Proposition 3.1.
  uint64_t probes = 0;           // bucket scans made by find
  uint64_t false_compares = 0;   // digest matched but key differed (find only)
};

// Digest reading: the prose of §3.2 says bits 32-39 of the hash; Algorithm 1
// writes bits 31:24. The two conflict; bits 32-39 are taken, which keeps the
// digest disjoint from the bucket bits for up to 2^32 buckets.
uint8_t digest_of(uint64_t h) { return static_cast<uint8_t>((h >> 32) & 0xFF); }

Route route(const Table& t, uint64_t k) {
  const uint64_t h1 = fmix64(k);
  Route r;
  r.b1 = h1 % t.buckets;
  r.d = digest_of(h1);
  r.b2 = t.dual ? fmix64(k ^ kSecondHashSalt) % t.buckets : r.b1;
  return r;
}

uint64_t pos_of(uint64_t b, int s) { return b * kSlots + static_cast<uint64_t>(s); }

// Algorithm 1 over one bucket: every slot whose digest equals d gets a full
// key comparison. Returns the slot or -1 (a definitive miss for this bucket).
int scan_bucket(Table& t, uint64_t b, uint64_t k, uint8_t d, bool count) {
  for (int s = 0; s < kSlots; ++s) {
    const uint64_t p = pos_of(b, s);
    if (t.digest[p] != d) continue;
    if (t.key[p] == k) return s;
    if (count) ++t.false_compares;
  }
  return -1;
}

// Looks for k in its candidate bucket(s): b1, then b2 in dual mode.
bool locate(Table& t, uint64_t k, const Route& r, uint64_t* b, int* s, bool count) {
  if (count) ++t.probes;
  int j = scan_bucket(t, r.b1, k, r.d, count);
  if (j >= 0) { *b = r.b1; *s = j; return true; }
  if (t.dual && r.b2 != r.b1) {
    if (count) ++t.probes;
    j = scan_bucket(t, r.b2, k, r.d, count);
    if (j >= 0) { *b = r.b2; *s = j; return true; }
  }
  return false;
}

// Number of occupied slots of a bucket (a slot is occupied iff it holds a key
// other than the empty sentinel).
int occupancy(const Table& t, uint64_t b) {
  int n = 0;
  for (int s = 0; s < kSlots; ++s) n += (t.key[pos_of(b, s)] != kEmptyKey);
  return n;
}

// The empty slot Algorithm 2 inserts into, read as the lowest-index empty slot.
int first_empty(const Table& t, uint64_t b) {
  for (int s = 0; s < kSlots; ++s)
    if (t.key[pos_of(b, s)] == kEmptyKey) return s;
  return -1;
}

// Rank order used for eviction and admission. The paper's Algorithm 2 rejects
// only when s < min (admitting ties) while Algorithm 3 admits only when
// s > min; neither says which of several minimum-score slots is the victim.
// Reading: entries are totally ordered by the pair (score, key); the victim is
// the lowest pair, and an incoming key is admitted iff its pair is higher.
bool rank_below(uint64_t s1, uint64_t k1, uint64_t s2, uint64_t k2) {
  return s1 < s2 || (s1 == s2 && k1 < k2);
}

// argmin over a full bucket by (score, key).
int lowest_ranked(const Table& t, uint64_t b) {
  int m = 0;
  for (int s = 1; s < kSlots; ++s) {
    const uint64_t p = pos_of(b, s), q = pos_of(b, m);
    if (rank_below(t.score[p], t.key[p], t.score[q], t.key[q])) m = s;
  }
  return m;
}

void write_payload(Table& t, uint64_t p, const float* v, uint64_t tag) {
  if (t.tag_mode) {
    t.tag[p] = tag;
  } else {
    for (uint32_t c = 0; c < t.dim; ++c) t.value[p * t.dim + c] = v[c];
  }
}

void write_slot(Table& t, uint64_t b, int s, uint64_t k, uint8_t d, const float* v,
                uint64_t tag, uint64_t sc) {
  const uint64_t p = pos_of(b, s);
  t.key[p] = k;
  t.digest[p] = d;
  t.score[p] = sc;
  write_payload(t, p, v, tag);
}

// An entry that leaves the table, or is turned away, during an upsert.
struct Departure {
  uint64_t key = 0, score = 0, tag = 0;
  std::vector<float> row;
};

void record_resident(const Table& t, uint64_t p, Departure* out) {
  out->key = t.key[p];
  out->score = t.score[p];
  if (t.tag_mode) {
    out->tag = t.tag[p];
  } else {
    out->row.assign(t.value.begin() + p * t.dim, t.value.begin() + (p + 1) * t.dim);
  }
}

void record_offered(const Table& t, uint64_t k, const float* v, uint64_t tag, uint64_t sc, Departure* out) {
  out->key = k;
  out->score = sc;
  if (t.tag_mode) {
    out->tag = tag;
  } else {
    out->row.assign(v, v + t.dim);
  }
}

// One key of insert_or_assign (Algorithm 2; Algorithm 3 in dual mode).
// When `gone` is given it receives the entry that an eviction pushes out, or
// the offered entry itself when admission turns it away.
Outcome upsert_one(Table& t, uint64_t k, const float* v, uint64_t tag, uint64_t sc,
                   Departure* gone = nullptr) {
  if (is_reserved(k)) return kSkipped;
  const Route r = route(t, k);
  uint64_t b;
  int s;
  // Present in a candidate bucket: overwrite value and score.
  if (locate(t, k, r, &b, &s, false)) {
    const uint64_t p = pos_of(b, s);
    t.score[p] = sc;
    write_payload(t, p, v, tag);
    return kUpdated;
  }
  if (!t.dual || r.b1 == r.b2) {
    // Single-bucket mode (a dual-mode key whose two hashes share a bucket has
    // only one candidate and is handled the same way).
    b = r.b1;
    s = first_empty(t, b);
    if (s >= 0) {
      write_slot(t, b, s, k, r.d, v, tag, sc);
      return kInserted;
    }
    s = lowest_ranked(t, b);
  } else {
    // Phase D1: some candidate has room -> the less-occupied bucket.
    // Reading for a tie in occupancy: b1.
    const int o1 = occupancy(t, r.b1), o2 = occupancy(t, r.b2);
    if (o1 < kSlots || o2 < kSlots) {
      b = (o1 <= o2) ? r.b1 : r.b2;
      s = first_empty(t, b);
      write_slot(t, b, s, k, r.d, v, tag, sc);
      return kInserted;
    }
    // Phase D2: both full -> the bucket whose lowest-ranked entry is lower.
    const int s1 = lowest_ranked(t, r.b1), s2 = lowest_ranked(t, r.b2);
    const uint64_t p1 = pos_of(r.b1, s1), p2 = pos_of(r.b2, s2);
    if (rank_below(t.score[p2], t.key[p2], t.score[p1], t.key[p1])) {
      b = r.b2;
      s = s2;
    } else {
      b = r.b1;
      s = s1;
    }
  }
  // Admission control against the chosen victim.
  const uint64_t p = pos_of(b, s);
  if (!rank_below(t.score[p], t.key[p], sc, k)) {
    if (gone) record_offered(t, k, v, tag, sc, gone);
    return kRejected;
  }
  if (gone) record_resident(t, p, gone);
  write_slot(t, b, s, k, r.d, v, tag, sc);
  return kEvicted;
}

// Which keys of a batch are resident when the call starts.
std::vector<char> resident_at_start(Table& t, uint64_t n, const uint64_t* keys) {
  std::vector<char> res(n, 0);
  for (uint64_t i = 0; i < n; ++i) {
    uint64_t b;
    int s;
    res[i] = !is_reserved(keys[i]) && locate(t, keys[i], route(t, keys[i]), &b, &s, false);
  }
  return res;
}

}  // namespace

extern "C" {

struct oracle_table;  // opaque to callers

oracle_table* oracle_create(uint64_t capacity, uint32_t dim, int dual, int tag_mode) {
  if (capacity == 0 || capacity % kSlots != 0 || dim == 0) return nullptr;
  Table* t = new (std::nothrow) Table();
  if (!t) return nullptr;
  try {
    t->capacity = capacity;
    t->buckets = capacity / kSlots;
    t->dim = dim;
    t->dual = dual != 0;
    t->tag_mode = tag_mode != 0;
    t->key.assign(capacity, kEmptyKey);
    t->score.assign(capacity, 0);
    // Every slot carries the digest of the key it holds, the empty sentinel
    // included (reading: the paper does not say what an empty slot's digest is).
    t->digest.assign(capacity, digest_of(fmix64(kEmptyKey)));
    if (t->tag_mode) {
      t->tag.assign(capacity, 0);
    } else {
      t->value.assign(capacity * dim, 0.0f);
    }
  } catch (...) {
    delete t;
    return nullptr;
  }
  return reinterpret_cast<oracle_table*>(t);
}

void oracle_destroy(oracle_table* h) { delete reinterpret_cast<Table*>(h); }

uint64_t oracle_fmix64(uint64_t k) { return fmix64(k); }

void oracle_murmur3_x64_128(const void* data, uint64_t len, uint32_t seed, uint64_t* out2) {
  murmur3_x64_128(static_cast<const uint8_t*>(data), len, seed, out2);
}

// Routing of n keys: primary bucket, second candidate, digest.
void oracle_route(const oracle_table* h, uint64_t n, const uint64_t* keys, uint64_t* b1,
                  uint64_t* b2, uint8_t* d) {
  const Table& t = *reinterpret_cast<const Table*>(h);
  for (uint64_t i = 0; i < n; ++i) {
    const Route r = route(t, keys[i]);
    if (b1) b1[i] = r.b1;
    if (b2) b2[i] = r.b2;
    if (d) d[i] = r.d;
  }
}

// Routing of n keys for a table of `buckets` buckets, without a table.
void oracle_route_buckets(uint64_t buckets, int dual, uint64_t n, const uint64_t* keys, uint64_t* b1,
                          uint64_t* b2, uint8_t* d) {
  Table t;
  t.buckets = buckets;
  t.dual = dual != 0;
  for (uint64_t i = 0; i < n; ++i) {
    const Route r = route(t, keys[i]);
    if (b1) b1[i] = r.b1;
    if (b2) b2[i] = r.b2;
    if (d) d[i] = r.d;
  }
}

// find (reader): on a hit writes the value row (or tag), found = 1 and the
// score; on a miss writes found = 0 and leaves the row, tag and score alone.
// Reserved keys always miss. Scores are never modified.
void oracle_find(oracle_table* h, uint64_t n, const uint64_t* keys, float* values_out,
                 uint8_t* found_out, uint64_t* scores_out, uint64_t* tags_out) {
  Table& t = *reinterpret_cast<Table*>(h);
  for (uint64_t i = 0; i < n; ++i) {
    const uint64_t k = keys[i];
    uint64_t b;
    int s;
    if (is_reserved(k) || !locate(t, k, route(t, k), &b, &s, true)) {
      found_out[i] = 0;
      continue;
    }
    const uint64_t p = pos_of(b, s);
    found_out[i] = 1;
    if (scores_out) scores_out[i] = t.score[p];
    if (t.tag_mode) {
      if (tags_out) tags_out[i] = t.tag[p];
    } else if (values_out) {
      for (uint32_t c = 0; c < t.dim; ++c) values_out[i * t.dim + c] = t.value[p * t.dim + c];
    }
  }
}

// insert_or_assign (inserter), keys applied one at a time in input order.
// values: n x dim floats (value mode); tags: n u64 (tag mode); scores required.
// outcomes (nullable): one Outcome code per key.
void oracle_insert_or_assign(oracle_table* h, uint64_t n, const uint64_t* keys,
                             const float* values, const uint64_t* tags,
                             const uint64_t* scores, uint32_t* outcomes) {
  Table& t = *reinterpret_cast<Table*>(h);
  for (uint64_t i = 0; i < n; ++i) {
    const float* v = t.tag_mode ? nullptr : values + i * t.dim;
    const uint64_t tg = t.tag_mode ? tags[i] : 0;
    const Outcome o = upsert_one(t, keys[i], v, tg, scores[i]);
    if (outcomes) outcomes[i] = o;
  }
}

// assign (updater): overwrites the value (if given) and score (if given) of
// keys already present; absent and reserved keys are left alone.
void oracle_assign(oracle_table* h, uint64_t n, const uint64_t* keys, const float* values,
                   const uint64_t* tags, const uint64_t* scores) {
  Table& t = *reinterpret_cast<Table*>(h);
  for (uint64_t i = 0; i < n; ++i) {
    const uint64_t k = keys[i];
    uint64_t b;
    int s;
    if (is_reserved(k) || !locate(t, k, route(t, k), &b, &s, false)) continue;
    const uint64_t p = pos_of(b, s);
    if (scores) t.score[p] = scores[i];
    if (t.tag_mode) {
      if (tags) t.tag[p] = tags[i];
    } else if (values) {
      for (uint32_t c = 0; c < t.dim; ++c) t.value[p * t.dim + c] = values[i * t.dim + c];
    }
  }
}

// find* (the pointer-returning reader of §4.1, measured in §5.3): instead of
// copying a resident key's value it reports where the value lives. Values are
// addressed by position (§3.6: row address = value base + (b * 128 + slot)
// rows), so the oracle reports the slot position; a miss (and a reserved key)
// gives found = 0 and position 2^64 - 1. contains is the same lookup with
// only the found flags kept.
void oracle_find_pos(oracle_table* h, uint64_t n, const uint64_t* keys, uint8_t* found_out,
                     uint64_t* pos_out) {
  Table& t = *reinterpret_cast<Table*>(h);
  for (uint64_t i = 0; i < n; ++i) {
    const uint64_t k = keys[i];
    uint64_t b;
    int s;
    const bool hit = !is_reserved(k) && locate(t, k, route(t, k), &b, &s, false);
    if (found_out) found_out[i] = hit;
    if (pos_out) pos_out[i] = hit ? pos_of(b, s) : ~0ull;
  }
}

// insert_and_evict (§4.1: an inserter that also hands back what it evicts).
// Reading of the order inside one call: the keys already resident when the
// call starts are updated first (value and score, as insert_or_assign does),
// then the other keys are inserted one at a time in input order (Algorithm 2,
// Algorithm 3 in dual mode). Output, compacted in the order it happens: every
// resident entry an insertion evicts (with the key, value or tag and score it
// held) and every offered entry that admission turns away. So the output is
// exactly the entries that were resident before the call or offered by it and
// are not resident after it, each with its last written value and score.
// Returns the number written (at most the number of keys not resident at the
// start). Reserved keys are skipped.
uint64_t oracle_insert_and_evict(oracle_table* h, uint64_t n, const uint64_t* keys, const float* values,
                                 const uint64_t* tags, const uint64_t* scores, uint64_t* ev_keys,
                                 float* ev_values, uint64_t* ev_tags, uint64_t* ev_scores) {
  Table& t = *reinterpret_cast<Table*>(h);
  const std::vector<char> res = resident_at_start(t, n, keys);
  for (uint64_t i = 0; i < n; ++i) {
    if (!res[i]) continue;
    const float* v = t.tag_mode ? nullptr : values + i * t.dim;
    upsert_one(t, keys[i], v, t.tag_mode ? tags[i] : 0, scores[i]);
  }
  uint64_t m = 0;
  for (uint64_t i = 0; i < n; ++i) {
    if (res[i] || is_reserved(keys[i])) continue;
    const float* v = t.tag_mode ? nullptr : values + i * t.dim;
    Departure d;
    const Outcome o = upsert_one(t, keys[i], v, t.tag_mode ? tags[i] : 0, scores[i], &d);
    if (o != kEvicted && o != kRejected) continue;
    if (ev_keys) ev_keys[m] = d.key;
    if (ev_scores) ev_scores[m] = d.score;
    if (t.tag_mode) {
      if (ev_tags) ev_tags[m] = d.tag;
    } else if (ev_values) {
      for (uint32_t c = 0; c < t.dim; ++c) ev_values[m * t.dim + c] = d.row[c];
    }
    ++m;
  }
  return m;
}

// find_or_insert (§4.1: lookup combined with insertion for cold starts).
// Reading: a key resident when the call starts is a hit: found = 1, its stored
// value (or tag) is written to the caller's row, and its score is replaced by
// the offered one (the call is an inserter, and the access refreshes the
// entry the way insert_or_assign's update does). Then every other key is
// inserted with the caller's row and score, one at a time in input order,
// exactly as insert_or_assign inserts (it may evict, or be turned away);
// found = 0 and the caller's row is left as it was. Reserved keys: found = 0,
// nothing else.
void oracle_find_or_insert(oracle_table* h, uint64_t n, const uint64_t* keys, float* values_inout,
                           uint64_t* tags_inout, const uint64_t* scores, uint8_t* found_out) {
  Table& t = *reinterpret_cast<Table*>(h);
  const std::vector<char> res = resident_at_start(t, n, keys);
  for (uint64_t i = 0; i < n; ++i) {
    if (found_out) found_out[i] = res[i];
    if (!res[i]) continue;
    uint64_t b;
    int s;
    locate(t, keys[i], route(t, keys[i]), &b, &s, false);
    const uint64_t p = pos_of(b, s);
    t.score[p] = scores[i];
    if (t.tag_mode) {
      tags_inout[i] = t.tag[p];
    } else {
      for (uint32_t c = 0; c < t.dim; ++c) values_inout[i * t.dim + c] = t.value[p * t.dim + c];
    }
  }
  for (uint64_t i = 0; i < n; ++i) {
    if (res[i] || is_reserved(keys[i])) continue;
    const float* v = t.tag_mode ? nullptr : values_inout + i * t.dim;
    upsert_one(t, keys[i], v, t.tag_mode ? tags_inout[i] : 0, scores[i]);
  }
}

// size: number of occupied slots in the table.
uint64_t oracle_size(const oracle_table* h) {
  const Table& t = *reinterpret_cast<const Table*>(h);
  uint64_t n = 0;
  for (uint64_t p = 0; p < t.capacity; ++p) n += (t.key[p] != kEmptyKey);
  return n;
}

// export: the occupied slots among positions [offset, offset + n_slots),
// in ascending position order. Returns how many were written.
uint64_t oracle_export(const oracle_table* h, uint64_t offset, uint64_t n_slots,
                       uint64_t* keys_out, float* values_out, uint64_t* scores_out,
                       uint64_t* pos_out, uint64_t* tags_out) {
  const Table& t = *reinterpret_cast<const Table*>(h);
  uint64_t end = offset + n_slots;
  if (end < offset || end > t.capacity) end = t.capacity;
  uint64_t m = 0;
  for (uint64_t p = offset; p < end; ++p) {
    if (t.key[p] == kEmptyKey) continue;
    if (keys_out) keys_out[m] = t.key[p];
    if (scores_out) scores_out[m] = t.score[p];
    if (pos_out) pos_out[m] = p;
    if (t.tag_mode) {
      if (tags_out) tags_out[m] = t.tag[p];
    } else if (values_out) {
      for (uint32_t c = 0; c < t.dim; ++c) values_out[m * t.dim + c] = t.value[p * t.dim + c];
    }
    ++m;
  }
  return m;
}

// Find instrumentation: [bucket scans, digest false positives].
void oracle_probe_stats(const oracle_table* h, uint64_t* out2) {
  const Table& t = *reinterpret_cast<const Table*>(h);
  out2[0] = t.probes;
  out2[1] = t.false_compares;
}

void oracle_reset_probe_stats(oracle_table* h) {
  Table& t = *reinterpret_cast<Table*>(h);
  t.probes = 0;
  t.false_compares = 0;
}

}  // extern "C"
