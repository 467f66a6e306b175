// gfx950 kernels of the cache-semantic bucketed hash table.
//
// Method: "HierarchicalKV: A GPU Hash Table with Cache Semantics for
// Continuous Online Embedding Storage" (arXiv 2603.17168).
//   find      - §3.2, Algorithm 1 (one 128-byte digest line per bucket, full
//               key compare only on digest match); two lines in dual mode (§3.4)
//   assign    - §3.5 updater: value/score writes to resident keys only
//   insert    - §3.3, Algorithm 2 (update / empty slot / evict-or-reject);
//               §3.4, Algorithm 3 (dual-bucket D1/D2 selection)
//   size, export - §3.5 readers, §4.1 export
//   find*, contains, insert_and_evict, find_or_insert - §4.1: the key-side
//               probe alone; the inserter with a hand-back of what leaves; the
//               inserter with stored rows copied out for resident keys
//   value rows - §3.6 / §4.2: addressed by position, split between HBM and
//               pinned host memory at a bucket boundary (the HBM watermark)
//
// Work decomposition (wave64, CDNA4):
//   * A "group" of G consecutive lanes of a wave serves one key. Lane l of a
//     group holds digest bytes [l*128/G, (l+1)*128/G) of the bucket's line, so
//     one vector load per lane fetches the whole 128-byte line coalesced.
//     Digest compares are SWAR byte compares; the lane that owns a matching
//     slot loads and compares that slot's key; a wave ballot picks the hit.
//   * Value rows are moved by the whole group in 16-byte pieces.
//   * Inserts need every bucket to see its keys one at a time (serializable
//     per bucket). Instead of spin locks, a link kernel threads the batch's
//     keys into one chain per target bucket with a single atomic exchange per
//     key; in the second kernel the chain's first-pushed key owns the bucket
//     exclusively and its group applies the chain's keys one after another.
//     No two groups ever write the same bucket inside a kernel, so no lock,
//     CAS retry or cross-XCD cache maintenance is needed; kernel boundaries
//     publish the result.
//   * In the inserter, slot s of a bucket belongs to lane s/8 of the
//     16-lane group: only that lane loads or stores the slot's key, score and
//     digest, so every read-after-write inside a chain is same-thread.
//
// Digest encoding: the digest of a key is bits 32..39 of its hash, except that
// the value 0 is stored as 1; 0 marks an empty slot, so empty slots never
// produce a candidate. This only affects the filter, never a result.
#include <hip/hip_ext.h>

#include "hkv_internal.h"

namespace hkv {
namespace {

constexpr int kSlots = 128;
constexpr uint64_t kLockedKey = ~0ull - 1;  // keys >= this are reserved
constexpr uint32_t kNoIdx = 0xFFFFFFFFu;    // chain end / empty chain head
// A chain head word: (epoch << 32) | batch index. This one is empty under
// every epoch: epoch 0 with no index.
constexpr uint64_t kEmptyHead = kNoIdx;
constexpr uint32_t kSkipIdx = 0xFFFFFFFEu;  // key takes no part in the insert
constexpr uint32_t kUpdIdx = 0xFFFFFFFCu;   // resident key updated (or its row read by
                                            // find_or_insert) with no claim to release
constexpr uint32_t kHitIdx = 0xFFFFFFFDu;   // resident key updated by this occurrence;
                                            // target[i] = its bucket (claim to clear)
constexpr uint32_t kFullBit = 0x80000000u;  // target word: the bucket was full at probe time
constexpr uint64_t kSecondSalt = 0x9E3779B97F4A7C15ull;
constexpr int kBlock = 256;
constexpr int kInsG = 16;  // lanes per key in the inserter (8 slots per lane)

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bool is_reserved(uint64_t k) { return k >= kLockedKey; }

// A key whose chain word is a batch index or kNoIdx was pushed onto a chain.
__device__ __forceinline__ bool in_chain(uint32_t nx) { return nx == kNoIdx || nx < kUpdIdx; }

// MurmurHash3's 64-bit finalizer, the table's hash (§3.2 names a Murmur3
// variant without giving it).
__device__ __forceinline__ uint64_t fmix64(uint64_t k) {
  k ^= k >> 33;
  k *= 0xff51afd7ed558ccdull;
  k ^= k >> 33;
  k *= 0xc4ceb9fe1a85ec53ull;
  k ^= k >> 33;
  return k;
}

__device__ __forceinline__ uint32_t bucket_of(const TableView& t, uint64_t h) {
  return t.pow2 ? static_cast<uint32_t>(h & t.nb_mask) : static_cast<uint32_t>(h % t.nb);
}

__device__ __forceinline__ uint32_t digest_of(uint64_t h) {
  const uint32_t d = static_cast<uint32_t>(h >> 32) & 0xFFu;
  return d == 0 ? 1u : d;
}

// Address of value row p. Rows are addressed by position (§3.6); positions
// below t.split live in the first region (HBM, or all rows), the others in the
// second (pinned host memory), whose base t.values_hi is offset by -split rows
// so that both use the same arithmetic. split is a multiple of 128, so one
// bucket's rows are contiguous in one region.
__device__ __forceinline__ float* row_of(const TableView& t, uint64_t p) {
  return (p < t.split ? t.values : t.values_hi) + p * t.dim;
}

// 0x80 in every byte of x that is zero, 0 in the others. Exact: the low seven
// bits are summed separately so no carry crosses a byte.
__device__ __forceinline__ uint32_t zero_bytes(uint32_t x) {
  const uint32_t t = (x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu;
  return ~(t | x | 0x7F7F7F7Fu);
}

__device__ __forceinline__ int wave_lane() { return static_cast<int>(threadIdx.x & 63); }

template <int G>
__device__ __forceinline__ uint64_t group_bits(uint64_t ballot) {
  const int base = wave_lane() & ~(G - 1);
  const uint64_t m = (G == 64) ? ~0ull : ((1ull << G) - 1);
  return (ballot >> base) & m;
}

template <int G>
__device__ __forceinline__ uint64_t group_min(uint64_t v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) {
    const uint64_t w = __shfl_xor(v, o, G);
    v = w < v ? w : v;
  }
  return v;
}

// Copies a row of dim floats with the G lanes of a group. Each lane loads up
// to R 16-byte pieces (4, or 2 for 16-lane groups) before storing any, so a
// row of up to 512 bytes costs one memory round trip. NT: nontemporal loads
// and stores (rows streamed out by find).
template <int G, bool V4, bool NT>
__device__ __forceinline__ void copy_row(float* __restrict__ dst, const float* __restrict__ src,
                                         uint32_t dim, int lane) {
  if constexpr (V4) {
    constexpr int R = G >= 16 ? 2 : 4;
    const f32x4* s4 = reinterpret_cast<const f32x4*>(src);
    f32x4* d4 = reinterpret_cast<f32x4*>(dst);
    const uint32_t n4 = dim >> 2;
    for (uint32_t c0 = lane; c0 < n4; c0 += R * G) {
      f32x4 v[R];
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (c0 + r * G < n4) v[r] = NT ? __builtin_nontemporal_load(s4 + c0 + r * G) : s4[c0 + r * G];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (c0 + r * G < n4) {
          if constexpr (NT) {
            __builtin_nontemporal_store(v[r], d4 + c0 + r * G);
          } else {
            d4[c0 + r * G] = v[r];
          }
        }
      }
    }
  } else {
    for (uint32_t c = lane; c < dim; c += G) dst[c] = src[c];
  }
}

// A row of at most P 16-byte pieces per lane (dim <= 4*G*P) held in the
// registers of the G lanes of a group, so that its load can be issued before
// a decision that its store waits for.
template <int G, int P = 1>
struct GroupRow {
  f32x4 v[P];
};

template <int G, int P>
__device__ __forceinline__ void group_row_load(GroupRow<G, P>& r, const float* __restrict__ src, uint32_t dim,
                                               int lane) {
#pragma unroll
  for (int q = 0; q < P; ++q)
    if (static_cast<uint32_t>(lane + q * G) < (dim >> 2))
      r.v[q] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src) + lane + q * G);
}

template <int G, int P>
__device__ __forceinline__ void group_row_store(const GroupRow<G, P>& r, float* __restrict__ dst, uint32_t dim,
                                                int lane) {
#pragma unroll
  for (int q = 0; q < P; ++q)
    if (static_cast<uint32_t>(lane + q * G) < (dim >> 2))
      __builtin_nontemporal_store(r.v[q], reinterpret_cast<f32x4*>(dst) + lane + q * G);
}

// Takes slot p's claim bit for this call; true for the first taker only.
__device__ __forceinline__ bool claim_slot(const TableView& t, uint64_t p) {
  const uint32_t bit = 1u << (p & 31);
  const uint32_t old = __hip_atomic_fetch_or(t.claim + (p >> 5), bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return (old & bit) == 0;
}

// Loads this lane's share (NW dwords) of a bucket's 128-byte digest line.
// KNT: with nontemporal loads (the find over host-resident rows, whose L2s
// are better spent on the rows that repeated keys read again).
template <int NW, bool KNT = false>
__device__ __forceinline__ void load_digest_words(const uint8_t* line, int lane, uint32_t (&w)[NW]) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(line) + lane * NW;
  if constexpr (NW == 2) {
    typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
    const u32x2_t v = KNT ? __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p)) : *reinterpret_cast<const u32x2_t*>(p);
    w[0] = v.x;
    w[1] = v.y;
  } else {
#pragma unroll
    for (int q = 0; q < NW; q += 4) {
      typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
      const u32x4_t v = KNT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + q)) : *reinterpret_cast<const u32x4_t*>(p + q);
      w[q] = v.x;
      w[q + 1] = v.y;
      w[q + 2] = v.z;
      w[q + 3] = v.w;
    }
  }
}

// One bit per zero byte of x (bit j for byte j): the 0x80 markers of
// zero_bytes gathered by a multiply that moves byte j's marker to bit 21 + j
// with no carries between the four partial products.
__device__ __forceinline__ uint32_t zero_byte_bits(uint32_t x) {
  return (((zero_bytes(x) >> 7) * 0x204081u) >> 21) & 0xFu;
}

// Candidate mask of this lane's share of a digest line: bit j is set when the
// digest of the lane's j-th slot equals the key's digest.
template <int NW>
__device__ __forceinline__ uint32_t candidate_mask(const uint32_t (&w)[NW], uint32_t pat) {
  uint32_t m = 0;
#pragma unroll
  for (int q = 0; q < NW; ++q) m |= zero_byte_bits(w[q] ^ pat) << (4 * q);
  return m;
}

// Full key compare of the candidate slots of up to two lines (mask m1 over
// positions base1 + j, mask m2 over base2 + j). The first two candidate keys
// are loaded back to back so that they cost one memory round trip; a third
// candidate in the same lane is rare (about 1 in 4000 lanes) and is looped.
// The key loads are cacheable: the key lines of recent lookups may then be
// served by the Infinity Cache, next to the digest lines. Returns the table
// position of the matching slot or -1.
// The candidate-key check split in two so that several keys' loads can be
// in flight together: cand_issue picks the first two candidate positions and
// loads their keys, cand_finish compares them and loops over any further
// candidates.
struct Cand {
  uint32_t m1, m2;
  uint64_t base1, base2;
  uint64_t p0, p1;
  uint64_t k0, k1;
  bool h0, h1;
};

template <bool KNT = false>
__device__ __forceinline__ void cand_issue(Cand& c, const uint64_t* __restrict__ keys, uint32_t m1,
                                           uint64_t base1, uint32_t m2, uint64_t base2) {
  // candidate positions in order: the bits of m1 (over base1), then of m2
  c.h0 = (m1 | m2) != 0;
  c.h1 = __builtin_popcount(m1) + __builtin_popcount(m2) >= 2;
  c.p0 = 0;
  c.p1 = 0;
  if (c.h0) {
    c.p0 = m1 ? base1 + __builtin_ctz(m1) : base2 + __builtin_ctz(m2);
    if (m1) m1 &= m1 - 1; else m2 &= m2 - 1;
  }
  if (c.h1) {
    c.p1 = m1 ? base1 + __builtin_ctz(m1) : base2 + __builtin_ctz(m2);
    if (m1) m1 &= m1 - 1; else m2 &= m2 - 1;
  }
  c.k0 = 0;
  c.k1 = 0;
  if (c.h0) c.k0 = KNT ? __builtin_nontemporal_load(keys + c.p0) : keys[c.p0];
  if (c.h1) c.k1 = KNT ? __builtin_nontemporal_load(keys + c.p1) : keys[c.p1];
  c.m1 = m1;
  c.m2 = m2;
  c.base1 = base1;
  c.base2 = base2;
}

template <bool KNT = false>
__device__ __forceinline__ int64_t cand_finish(Cand& c, const uint64_t* __restrict__ keys, uint64_t k) {
  int64_t hit = -1;
  if (c.h0 && c.k0 == k) hit = static_cast<int64_t>(c.p0);
  if (c.h1 && c.k1 == k) hit = static_cast<int64_t>(c.p1);
  while (c.m1) {
    const uint64_t p = c.base1 + __builtin_ctz(c.m1);
    c.m1 &= c.m1 - 1;
    if ((KNT ? __builtin_nontemporal_load(keys + p) : keys[p]) == k) hit = static_cast<int64_t>(p);
  }
  while (c.m2) {
    const uint64_t p = c.base2 + __builtin_ctz(c.m2);
    c.m2 &= c.m2 - 1;
    if ((KNT ? __builtin_nontemporal_load(keys + p) : keys[p]) == k) hit = static_cast<int64_t>(p);
  }
  return hit;
}

template <bool KNT = false>
__device__ __forceinline__ int64_t match_candidates(const uint64_t* __restrict__ keys, uint64_t k,
                                                    uint32_t m1, uint64_t base1, uint32_t m2,
                                                    uint64_t base2) {
  Cand c;
  cand_issue<KNT>(c, keys, m1, base1, m2, base2);
  return cand_finish<KNT>(c, keys, k);
}

// Occupied slots counted from a group's digest words: slots fill in order and
// an occupied slot never has digest 0 (group-uniform result).
template <int G, int NW>
__device__ __forceinline__ uint32_t line_occupancy(const uint32_t (&w)[NW]) {
  uint32_t c = 0;
#pragma unroll
  for (int q = 0; q < NW; ++q) c += 4 - __builtin_popcount(zero_byte_bits(w[q]));
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) c += __shfl_xor(c, o, G);
  return c;
}

// Group-wide probe of the key's candidate bucket(s). Returns the hit position
// (same value in every lane of the group) or -1. In dual mode the second
// bucket's line is read only when the first bucket does not hold the key. When
// occ1/occ2 are given they receive, for a key that is not found, the
// occupancy of the first / second candidate bucket.
template <int G, bool DUAL, bool KNT = false>
__device__ __forceinline__ int64_t probe(const TableView& t, uint64_t k, int lane, uint32_t* occ1 = nullptr,
                                         uint32_t* occ2 = nullptr) {
  constexpr int NW = kSlots / G / 4;
  const uint64_t h = fmix64(k);
  const uint32_t pat = digest_of(h) * 0x01010101u;
  const uint32_t b1 = bucket_of(t, h);
  uint32_t w1[NW];
  load_digest_words<NW, KNT>(t.digests + static_cast<uint64_t>(b1) * kSlots, lane, w1);
  const uint64_t off = static_cast<uint64_t>(lane) * (NW * 4);
  int64_t hit = -1;
  const bool rsv = is_reserved(k);
  if (!rsv) hit = match_candidates<KNT>(t.keys, k, candidate_mask<NW>(w1, pat), static_cast<uint64_t>(b1) * kSlots + off, 0, 0);
  uint64_t bits = group_bits<G>(__ballot(hit >= 0));
  if (occ1) *occ1 = line_occupancy<G, NW>(w1);
  if constexpr (DUAL) {
    // the second bucket only when the first does not hold the key
    const uint32_t b2 = bucket_of(t, fmix64(k ^ kSecondSalt));
    if (occ2) *occ2 = 0;
    if (bits == 0 && b2 != b1) {
      uint32_t w2[NW];
      load_digest_words<NW, KNT>(t.digests + static_cast<uint64_t>(b2) * kSlots, lane, w2);
      if (!rsv) hit = match_candidates<KNT>(t.keys, k, candidate_mask<NW>(w2, pat), static_cast<uint64_t>(b2) * kSlots + off, 0, 0);
      bits = group_bits<G>(__ballot(hit >= 0));
      if (occ2) *occ2 = line_occupancy<G, NW>(w2);
    }
  }
  if (bits == 0) return -1;
  return __shfl(hit, __ffsll(static_cast<unsigned long long>(bits)) - 1, G);
}

// probe() for K keys per group with their memory round trips overlapped: all
// K digest lines are requested before any is used, then all K keys'
// candidate keys (in dual mode, then the same for the second buckets of the
// keys their first bucket does not hold). hit[j] is group-uniform.
template <int G, bool DUAL, int K>
__device__ __forceinline__ void probe_many(const TableView& t, const uint64_t (&k)[K], int lane,
                                           int64_t (&hit)[K]) {
  constexpr int NW = kSlots / G / 4;
  uint32_t w[K][NW];
  uint32_t b1[K], pat[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const uint64_t h = fmix64(k[j]);
    pat[j] = digest_of(h) * 0x01010101u;
    b1[j] = bucket_of(t, h);
    load_digest_words<NW>(t.digests + static_cast<uint64_t>(b1[j]) * kSlots, lane, w[j]);
  }
  const uint64_t off = static_cast<uint64_t>(lane) * (NW * 4);
  Cand c[K];
#pragma unroll
  for (int j = 0; j < K; ++j)
    cand_issue(c[j], t.keys, is_reserved(k[j]) ? 0u : candidate_mask<NW>(w[j], pat[j]),
               static_cast<uint64_t>(b1[j]) * kSlots + off, 0, 0);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int64_t hj = cand_finish(c[j], t.keys, k[j]);
    const uint64_t bits = group_bits<G>(__ballot(hj >= 0));
    hit[j] = bits == 0 ? -1 : __shfl(hj, __ffsll(static_cast<unsigned long long>(bits)) - 1, G);
  }
  if constexpr (DUAL) {
    // the second buckets of the keys their first bucket does not hold, again
    // with every key's loads in flight together
    uint32_t b2[K];
    bool second[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      b2[j] = bucket_of(t, fmix64(k[j] ^ kSecondSalt));
      second[j] = hit[j] < 0 && b2[j] != b1[j] && !is_reserved(k[j]);
      if (second[j]) load_digest_words<NW>(t.digests + static_cast<uint64_t>(b2[j]) * kSlots, lane, w[j]);
    }
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (second[j]) cand_issue(c[j], t.keys, candidate_mask<NW>(w[j], pat[j]), static_cast<uint64_t>(b2[j]) * kSlots + off, 0, 0);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if (!second[j]) continue;
      const int64_t hj = cand_finish(c[j], t.keys, k[j]);
      const uint64_t bits = group_bits<G>(__ballot(hj >= 0));
      hit[j] = bits == 0 ? -1 : __shfl(hj, __ffsll(static_cast<unsigned long long>(bits)) - 1, G);
    }
  }
}

// probe() that also requests a row of the caller's (src, dim floats) into
// registers as soon as the digest lines show the group a candidate slot, so
// that its load overlaps the candidate-key loads (keys with no candidate are
// misses and load nothing).
template <int G, bool DUAL>
__device__ __forceinline__ int64_t probe_prefetch(const TableView& t, uint64_t k, int lane, uint32_t* occ1,
                                                  uint32_t* occ2, bool load_row, const float* src,
                                                  GroupRow<G>& rr) {
  constexpr int NW = kSlots / G / 4;
  const uint64_t h = fmix64(k);
  const uint32_t pat = digest_of(h) * 0x01010101u;
  const uint32_t b1 = bucket_of(t, h);
  uint32_t w1[NW];
  load_digest_words<NW>(t.digests + static_cast<uint64_t>(b1) * kSlots, lane, w1);
  const uint64_t off = static_cast<uint64_t>(lane) * (NW * 4);
  Cand c;
  cand_issue(c, t.keys, candidate_mask<NW>(w1, pat), static_cast<uint64_t>(b1) * kSlots + off, 0, 0);
  if (load_row && group_bits<G>(__ballot(c.h0)) != 0) group_row_load<G>(rr, src, t.dim, lane);
  int64_t hit = cand_finish(c, t.keys, k);
  uint64_t bits = group_bits<G>(__ballot(hit >= 0));
  if constexpr (DUAL) {
    // the second bucket only when the first does not hold the key
    const uint32_t b2 = bucket_of(t, fmix64(k ^ kSecondSalt));
    *occ2 = 0;
    if (bits == 0 && b2 != b1) {
      uint32_t w2[NW];
      load_digest_words<NW>(t.digests + static_cast<uint64_t>(b2) * kSlots, lane, w2);
      Cand c2;
      cand_issue(c2, t.keys, candidate_mask<NW>(w2, pat), static_cast<uint64_t>(b2) * kSlots + off, 0, 0);
      if (load_row && group_bits<G>(__ballot(c2.h0)) != 0) group_row_load<G>(rr, src, t.dim, lane);
      hit = cand_finish(c2, t.keys, k);
      bits = group_bits<G>(__ballot(hit >= 0));
      if (bits == 0) *occ2 = line_occupancy<G, NW>(w2);
    }
  }
  if (bits == 0) {
    // a miss: the occupancies choose its bucket (the result is group-uniform,
    // so the whole group takes this branch together)
    *occ1 = line_occupancy<G, NW>(w1);
    return -1;
  }
  return __shfl(hit, __ffsll(static_cast<unsigned long long>(bits)) - 1, G);
}

// ---------------------------------------------------------------- readers --

// find for key i by the G lanes of a group (Algorithm 1): probe, then the
// row, found flag and (optionally) score of a hit; a miss writes found = 0.
template <int G, bool V4, bool DUAL, bool NT, bool KNT = false>
__device__ __forceinline__ void find_one(const TableView& t, uint64_t i, uint64_t k, float* __restrict__ out,
                                         uint8_t* __restrict__ found, uint64_t* __restrict__ scores_out,
                                         int lane) {
  const int64_t p = probe<G, DUAL, KNT>(t, k, lane);
  if (p < 0) {
    if (lane == 0) found[i] = 0;
    return;
  }
  // The stored score is requested before the row, so both arrive in the
  // same round trip.
  uint64_t sc = 0;
  if (scores_out && lane == 0) sc = t.scores[p];
  // Host-resident rows are read with cacheable loads: repeated (hot) keys of
  // a batch then find their rows in L2 instead of crossing the host link again.
  if (static_cast<uint64_t>(p) >= t.split) {
    copy_row<G, V4, false>(out + i * t.dim, row_of(t, static_cast<uint64_t>(p)), t.dim, lane);
  } else {
    copy_row<G, V4, NT>(out + i * t.dim, row_of(t, static_cast<uint64_t>(p)), t.dim, lane);
  }
  if (lane == 0) {
    found[i] = 1;
    if (scores_out) scores_out[i] = sc;
  }
}

template <int G, bool V4, bool DUAL, bool NT>
__global__ __launch_bounds__(kBlock) void find_kernel(TableView t, uint64_t n,
                                                      const uint64_t* __restrict__ keys,
                                                      float* __restrict__ out,
                                                      uint8_t* __restrict__ found,
                                                      uint64_t* __restrict__ scores_out) {
  const uint64_t i = (static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x) / G;
  const int lane = static_cast<int>(threadIdx.x & (G - 1));
  if (i >= n) return;  // groups are lane-aligned, so a whole group leaves together
  find_one<G, V4, DUAL, NT>(t, i, keys[i], out, found, scores_out, lane);
}

// find when value rows live in host memory; its key-side reads (digest lines,
// candidate keys) are nontemporal, so that they do not push out of L2 the host
// rows that a batch's repeated keys read again (tiered Zipf(1.2) find: 1.587
// vs 1.615 ms per 2^20 draws). The XCDs of the GPU have an L2
// each, and workgroups are handed to the XCDs in turn (workgroup w to XCD
// w mod 8), so a hot key whose draws land in workgroups of several XCDs has
// its row fetched over the host link once per XCD. Here every chunk of
// kXcdChunk keys is served by kXcds consecutive workgroups, and workgroup x of
// a chunk serves only the chunk's keys whose hash bits 56..58 equal x: all
// draws of a key meet in one XCD's L2 and its row crosses the link once.
// Correctness does not depend on the placement (every key is served by
// exactly one workgroup); only the hit rate of the L2s does. Each workgroup
// reads the whole chunk's keys (8 bytes per key per workgroup, from L2).
constexpr int kXcds = 8;

template <int G, bool V4, bool DUAL, bool NT>
__global__ __launch_bounds__(kBlock) void find_xcd_kernel(TableView t, uint64_t n,
                                                          const uint64_t* __restrict__ keys,
                                                          float* __restrict__ out,
                                                          uint8_t* __restrict__ found,
                                                          uint64_t* __restrict__ scores_out) {
  constexpr int kGroups = kBlock / G;
  constexpr int kXcdChunk = kGroups * kXcds;  // on average one key per group
  __shared__ uint32_t s_idx[kXcdChunk];
  __shared__ uint32_t s_count;
  const uint32_t x = blockIdx.x % kXcds;
  const uint64_t c0 = static_cast<uint64_t>(blockIdx.x / kXcds) * kXcdChunk;
  if (threadIdx.x == 0) s_count = 0;
  __syncthreads();
  for (uint32_t j = threadIdx.x; j < static_cast<uint32_t>(kXcdChunk); j += kBlock) {
    const uint64_t i = c0 + j;
    if (i < n && static_cast<uint32_t>(fmix64(keys[i]) >> 56 & (kXcds - 1)) == x)
      s_idx[atomicAdd(&s_count, 1u)] = j;
  }
  __syncthreads();
  const uint32_t mine = s_count;
  const int lane = static_cast<int>(threadIdx.x & (G - 1));
  for (uint32_t e = threadIdx.x / G; e < mine; e += kGroups) {
    const uint64_t i = c0 + s_idx[e];
    find_one<G, V4, DUAL, NT, true>(t, i, keys[i], out, found, scores_out, lane);
  }
}

// find* (pointer-returning find) and contains, §4.1 / §5.3: the key-side half
// of find. A hit writes the device-accessible address of the key's value row
// (host-mapped when values live in host memory), found = 1 and the score; a
// miss writes a null address and found = 0. Every output is optional.
// A group serves K consecutive keys (probe_many), which multiplies the
// round trips each wave has in flight; a key past n is probed as a reserved
// key and writes nothing.
template <int G, bool DUAL, int K>
__global__ __launch_bounds__(kBlock) void locate_kernel(TableView t, uint64_t n,
                                                        const uint64_t* __restrict__ keys,
                                                        uint64_t* __restrict__ ptrs_out,
                                                        uint8_t* __restrict__ found,
                                                        uint64_t* __restrict__ scores_out) {
  const uint64_t i0 = (static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x) / G * K;
  const int lane = static_cast<int>(threadIdx.x & (G - 1));
  if (i0 >= n) return;
  uint64_t k[K];
#pragma unroll
  for (int j = 0; j < K; ++j) k[j] = i0 + j < n ? keys[i0 + j] : ~0ull;
  int64_t p[K];
  probe_many<G, DUAL, K>(t, k, lane, p);
  if (lane != 0) return;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const uint64_t i = i0 + j;
    if (i >= n) break;
    if (found) found[i] = p[j] >= 0 ? 1 : 0;
    if (ptrs_out)
      ptrs_out[i] = p[j] >= 0 ? reinterpret_cast<uint64_t>(row_of(t, static_cast<uint64_t>(p[j]))) : 0ull;
    if (scores_out && p[j] >= 0) scores_out[i] = t.scores[p[j]];
  }
}

__global__ __launch_bounds__(kBlock) void size_kernel(const uint32_t* __restrict__ occ, uint64_t nb,
                                                      unsigned long long* out) {
  __shared__ unsigned long long part[kBlock / 64];
  unsigned long long acc = 0;
  for (uint64_t b = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x; b < nb;
       b += static_cast<uint64_t>(gridDim.x) * kBlock)
    acc += occ[b];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (wave_lane() == 0) part[threadIdx.x / 64] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long total = 0;
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w) total += part[w];
    if (total) atomicAdd(out, total);
  }
}

__global__ void zero_u64_kernel(unsigned long long* p) { *p = 0; }

// export (§4.1): the occupied slots of positions [begin, end), compacted in
// unspecified order. Slots fill in order and nothing is erased, so the
// occupied slots of a bucket are [0, occ): the part of a bucket inside the
// range is one run of consecutive slots whose rows are one run of memory. A
// block takes kExportBuckets consecutive buckets, reserves room for all their
// occupied slots with one atomic add (one per wave serialized on the single
// counter: 12 ms for 2^26 slots), and its waves copy one bucket's run at a
// time: keys, scores and positions one slot per lane, the rows as one
// contiguous copy shared by the 64 lanes.
constexpr int kExportBuckets = 128;

template <bool V4>
__global__ __launch_bounds__(kBlock) void export_kernel(TableView t, uint64_t begin, uint64_t end,
                                                        uint64_t* __restrict__ keys_out,
                                                        float* __restrict__ values_out,
                                                        uint64_t* __restrict__ scores_out,
                                                        uint64_t* __restrict__ pos_out,
                                                        unsigned long long* count) {
  __shared__ uint32_t s_lo[kExportBuckets];   // first slot of the bucket's run
  __shared__ uint32_t s_n[kExportBuckets];    // its length
  __shared__ uint32_t s_off[kExportBuckets];  // its offset among the block's entries
  __shared__ unsigned long long s_base;
  const uint64_t b_first = begin / kSlots;
  const uint64_t b_end = (end + kSlots - 1) / kSlots;
  const uint64_t b0 = b_first + static_cast<uint64_t>(blockIdx.x) * kExportBuckets;
  const int lane = static_cast<int>(threadIdx.x & 63);
  if (threadIdx.x < 64) {
    // the first wave: runs of buckets 2*lane and 2*lane+1, then their offsets
    uint32_t lo[2], n[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint64_t b = b0 + 2 * lane + h;
      lo[h] = 0;
      n[h] = 0;
      if (b < b_end) {
        const uint64_t first = b * kSlots;
        lo[h] = begin > first ? static_cast<uint32_t>(begin - first) : 0u;
        const uint32_t hi = end < first + kSlots ? static_cast<uint32_t>(end - first) : static_cast<uint32_t>(kSlots);
        const uint32_t occ = t.occ[b];
        const uint32_t top = occ < hi ? occ : hi;
        n[h] = top > lo[h] ? top - lo[h] : 0u;
      }
    }
    uint32_t sum = n[0] + n[1];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(sum, o, 64);
      if (lane >= o) sum += y;
    }
    const uint32_t excl = sum - n[0] - n[1];
    s_lo[2 * lane] = lo[0];
    s_lo[2 * lane + 1] = lo[1];
    s_n[2 * lane] = n[0];
    s_n[2 * lane + 1] = n[1];
    s_off[2 * lane] = excl;
    s_off[2 * lane + 1] = excl + n[0];
    if (lane == 63) s_base = sum ? atomicAdd(count, static_cast<unsigned long long>(sum)) : 0ull;
  }
  __syncthreads();
  const unsigned long long base = s_base;
  for (int q = static_cast<int>(threadIdx.x >> 6); q < kExportBuckets; q += kBlock / 64) {
    const uint32_t n = s_n[q];
    if (n == 0) continue;
    const uint64_t p0 = (b0 + q) * kSlots + s_lo[q];
    const uint64_t j0 = base + s_off[q];
    for (uint32_t e = lane; e < n; e += 64) {
      keys_out[j0 + e] = t.keys[p0 + e];
      if (scores_out) scores_out[j0 + e] = t.scores[p0 + e];
      if (pos_out) pos_out[j0 + e] = p0 + e;
    }
    if (!values_out) continue;
    // the run's rows: n * dim consecutive floats (one bucket's rows share a region)
    const float* src = row_of(t, p0);
    float* dst = values_out + j0 * t.dim;
    const uint64_t total = static_cast<uint64_t>(n) * t.dim;
    if constexpr (V4) {
      const f32x4* s4 = reinterpret_cast<const f32x4*>(src);
      f32x4* d4 = reinterpret_cast<f32x4*>(dst);
      const uint64_t n4 = total >> 2;
      for (uint64_t c = lane; c < n4; c += 4 * 64) {
        f32x4 v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (c + r * 64 < n4) v[r] = s4[c + r * 64];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (c + r * 64 < n4) d4[c + r * 64] = v[r];
      }
    } else {
      for (uint64_t c = lane; c < total; c += 64) dst[c] = src[c];
    }
  }
}

// --------------------------------------------------------------- updaters --

template <int G, bool V4, bool DUAL>
__global__ __launch_bounds__(kBlock) void assign_kernel(TableView t, uint64_t n,
                                                        const uint64_t* __restrict__ keys,
                                                        const float* __restrict__ values,
                                                        const uint64_t* __restrict__ scores) {
  const uint64_t i = (static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x) / G;
  const int lane = static_cast<int>(threadIdx.x & (G - 1));
  if (i >= n) return;
  const int64_t p = probe<G, DUAL>(t, keys[i], lane);
  if (p < 0) return;
  if (values)
    copy_row<G, V4, true>(row_of(t, static_cast<uint64_t>(p)), values + i * t.dim, t.dim, lane);
  if (scores && lane == 0) t.scores[p] = scores[i];
}

// -------------------------------------------------------------- inserters --

// One bucket held by a 16-lane group: occupancy (group-uniform) and this
// lane's 8 digest bytes.
struct Owned {
  uint32_t b;
  uint32_t occ;
  uint32_t dig0, dig1;  // digest bytes of slots 8*lane .. 8*lane+7
};

__device__ __forceinline__ void own_load(Owned& o, const TableView& t, uint32_t b, int lane) {
  o.b = b;
  uint32_t occ = 0;
  if (lane == 0) occ = t.occ[b];  // lane 0 alone reads and writes the occupancy word
  o.occ = __shfl(occ, 0, kInsG);
  const uint2 v = *reinterpret_cast<const uint2*>(t.digests + static_cast<uint64_t>(b) * kSlots + lane * 8);
  o.dig0 = v.x;
  o.dig1 = v.y;
}

__device__ __forceinline__ void own_store_occ(const Owned& o, const TableView& t, int lane) {
  if (lane == 0) t.occ[o.b] = o.occ;
}

// Slot of key k in the owned bucket, or -1 (group-uniform). Only slots below
// the occupancy are compared (the rest are empty).
__device__ __forceinline__ int own_find(const Owned& o, const TableView& t, uint64_t k, uint32_t pat,
                                        int lane) {
  const int first = lane * 8;
  const int live = static_cast<int>(o.occ) - first;
  const uint32_t valid = live >= 8 ? 0xFFu : (live <= 0 ? 0u : ((1u << live) - 1));
  const uint32_t m = (zero_byte_bits(o.dig0 ^ pat) | (zero_byte_bits(o.dig1 ^ pat) << 4)) & valid;
  const uint64_t base = static_cast<uint64_t>(o.b) * kSlots + first;
  const int64_t p = match_candidates(t.keys, k, m, base, 0u, base);
  const int hit = p >= 0 ? static_cast<int>(p - static_cast<int64_t>(o.b) * kSlots) : -1;
  const uint64_t bits = group_bits<kInsG>(__ballot(hit >= 0));
  if (bits == 0) return -1;
  return __shfl(hit, __ffsll(static_cast<unsigned long long>(bits)) - 1, kInsG);
}

// Lowest (score, key) entry of a full owned bucket (group-uniform results).
// Each lane reads the scores and keys of its own 8 slots (written only by
// itself earlier in the kernel).
__device__ __forceinline__ void own_lowest(const Owned& o, const TableView& t, int lane,
                                           uint64_t* min_score, uint64_t* min_key, int* slot) {
  const uint64_t base = static_cast<uint64_t>(o.b) * kSlots + lane * 8;
  uint64_t sc[8];
#pragma unroll
  for (int u = 0; u < 8; u += 2) {
    const ulonglong2 v = *reinterpret_cast<const ulonglong2*>(t.scores + base + u);
    sc[u] = v.x;
    sc[u + 1] = v.y;
  }
  uint64_t ls = sc[0];
#pragma unroll
  for (int u = 1; u < 8; ++u) ls = sc[u] < ls ? sc[u] : ls;
  const uint64_t gs = group_min<kInsG>(ls);
  // Among the slots at the minimum score, the smallest key ranks lowest.
  uint64_t lk = ~0ull;
  int lslot = -1;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (sc[u] == gs) {
      const uint64_t kk = t.keys[base + u];
      if (lslot < 0 || kk < lk) {
        lk = kk;
        lslot = lane * 8 + u;
      }
    }
  }
  const uint64_t gk = group_min<kInsG>(lslot >= 0 ? lk : ~0ull);
  const uint64_t bits = group_bits<kInsG>(__ballot(lslot >= 0 && lk == gk));
  *min_score = gs;
  *min_key = gk;
  *slot = __shfl(lslot, __ffsll(static_cast<unsigned long long>(bits)) - 1, kInsG);
}

// Writes (key, digest, score) of slot s (by its owner lane) and keeps the
// group's register copies current. The value row is written by the caller.
__device__ __forceinline__ void own_write_slot(Owned& o, const TableView& t, int s, uint64_t k,
                                               uint32_t d, uint64_t score, int lane) {
  if (lane != (s >> 3)) return;
  const uint64_t p = static_cast<uint64_t>(o.b) * kSlots + s;
  t.keys[p] = k;
  t.scores[p] = score;
  t.digests[p] = static_cast<uint8_t>(d);
  const int sh = (s & 3) * 8;
  if (s & 4) {
    o.dig1 = (o.dig1 & ~(0xFFu << sh)) | (d << sh);
  } else {
    o.dig0 = (o.dig0 & ~(0xFFu << sh)) | (d << sh);
  }
}

__device__ __forceinline__ void own_write_score(Owned& o, const TableView& t, int s, uint64_t score,
                                                int lane) {
  if (lane != (s >> 3)) return;
  t.scores[static_cast<uint64_t>(o.b) * kSlots + s] = score;
}

template <bool V4>
__device__ __forceinline__ void own_write_row(const Owned& o, const TableView& t, int s,
                                              const float* row, int lane) {
  copy_row<kInsG, V4, true>(row_of(t, static_cast<uint64_t>(o.b) * kSlots + s), row, t.dim,
                            lane);
}

// A value row held in registers by a 16-lane group: up to two 16-byte pieces
// per lane (rows of up to 128 floats), loaded before the decision that needs
// them so that its latency overlaps the bucket loads.
struct RowRegs {
  f32x4 v[2];
};

__device__ __forceinline__ void row_regs_load(RowRegs& r, const float* src, uint32_t dim, int lane) {
  const f32x4* s4 = reinterpret_cast<const f32x4*>(src);
  const uint32_t n4 = dim >> 2;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t c = lane + u * kInsG;
    if (c < n4) r.v[u] = __builtin_nontemporal_load(s4 + c);
  }
}

__device__ __forceinline__ void row_regs_store(const RowRegs& r, float* dst, uint32_t dim, int lane) {
  f32x4* d4 = reinterpret_cast<f32x4*>(dst);
  const uint32_t n4 = dim >> 2;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t c = lane + u * kInsG;
    if (c < n4) __builtin_nontemporal_store(r.v[u], d4 + c);
  }
}

// Output of insert_and_evict: entries handed back, compacted through an
// atomic counter (keys == nullptr: nothing is handed back).
struct Evicted {
  uint64_t* keys;
  float* values;
  uint64_t* scores;
  unsigned long long* count;
};

// Staging of insert_and_evict's hand-back in the parallel inserter. Chain key
// i causes at most one departure; the owner kernel records it at index i and
// a compaction kernel moves the recorded entries to the output, one counter
// reservation per block instead of one contended atomic per entry.
//   kind[i]: 0 nothing left, 1 a resident was evicted (its key, score and row
//   are staged at i), 2 key i itself was turned away (key and score staged,
//   its row is the input row). Written for every chain key; keys outside the
//   chains (next[i] == kSkipIdx) are never read.
struct EvictStage {
  uint8_t* kind;
  uint64_t* keys;
  uint64_t* scores;
  float* rows;
};

// Hands back one entry with the 16 lanes of a group: lane 0 reserves the
// output index, the group copies the row from `src` (or from registers).
template <bool V4>
__device__ __forceinline__ void emit_entry(const Evicted& ev, const TableView& t, uint64_t k, uint64_t score,
                                           const float* src, const RowRegs* regs, int lane) {
  unsigned long long j = 0;
  if (lane == 0) {
    j = atomicAdd(ev.count, 1ull);
    ev.keys[j] = k;
    if (ev.scores) ev.scores[j] = score;
  }
  j = __shfl(j, 0, kInsG);
  if (!ev.values) return;
  float* dst = ev.values + j * t.dim;
  if (regs) {
    row_regs_store(*regs, dst, t.dim, lane);
  } else {
    copy_row<kInsG, V4, true>(dst, src, t.dim, lane);
  }
}

// Algorithm 2 for one key against an owned bucket: update if present, else
// the lowest empty slot, else evict the lowest-ranked entry if the key ranks
// higher, else reject. Empty slots are [occ, 128) because nothing is erased.
// The input row is prefetched on entry. A full bucket is decided from one
// round trip: each lane loads the scores and keys of its 8 slots, compares the
// key directly (no digest filter needed) and finds the lowest (score, key)
// in registers.
template <bool V4>
__device__ __forceinline__ void own_upsert(Owned& o, const TableView& t, uint64_t k, const float* row,
                                           uint64_t score, const Evicted& ev, int lane) {
  const bool in_regs = V4 && t.dim <= 8 * kInsG;
  RowRegs rr;
  if (in_regs) row_regs_load(rr, row, t.dim, lane);
  const uint64_t h = fmix64(k);
  const uint32_t d = digest_of(h);
  float* const table_rows = row_of(t, static_cast<uint64_t>(o.b) * kSlots);
  auto write_row = [&](int s) {
    if (in_regs) {
      row_regs_store(rr, table_rows + static_cast<uint64_t>(s) * t.dim, t.dim, lane);
    } else {
      own_write_row<V4>(o, t, s, row, lane);
    }
  };
  if (o.occ < kSlots) {
    const int hit = own_find(o, t, k, d * 0x01010101u, lane);
    if (hit >= 0) {
      own_write_score(o, t, hit, score, lane);
      write_row(hit);
      return;
    }
    const int s = static_cast<int>(o.occ);
    own_write_slot(o, t, s, k, d, score, lane);
    write_row(s);
    o.occ += 1;
    return;
  }
  // Full bucket: the lane's scores and keys (64 contiguous bytes each).
  const uint64_t base = static_cast<uint64_t>(o.b) * kSlots + lane * 8;
  uint64_t sc[8], kc[8];
#pragma unroll
  for (int u = 0; u < 8; u += 2) {
    const ulonglong2 a = *reinterpret_cast<const ulonglong2*>(t.scores + base + u);
    const ulonglong2 b = *reinterpret_cast<const ulonglong2*>(t.keys + base + u);
    sc[u] = a.x;
    sc[u + 1] = a.y;
    kc[u] = b.x;
    kc[u + 1] = b.y;
  }
  int lh = -1;
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (kc[u] == k) lh = lane * 8 + u;
  const uint64_t hb = group_bits<kInsG>(__ballot(lh >= 0));
  if (hb) {
    const int hit = __shfl(lh, __ffsll(static_cast<unsigned long long>(hb)) - 1, kInsG);
    own_write_score(o, t, hit, score, lane);
    write_row(hit);
    return;
  }
  uint64_t ls = sc[0];
#pragma unroll
  for (int u = 1; u < 8; ++u) ls = sc[u] < ls ? sc[u] : ls;
  const uint64_t gs = group_min<kInsG>(ls);
  uint64_t lk = ~0ull;
  int lslot = -1;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (sc[u] == gs && (lslot < 0 || kc[u] < lk)) {
      lk = kc[u];
      lslot = lane * 8 + u;
    }
  }
  const uint64_t gk = group_min<kInsG>(lslot >= 0 ? lk : ~0ull);
  if (score > gs || (score == gs && k > gk)) {
    const uint64_t vb = group_bits<kInsG>(__ballot(lslot >= 0 && lk == gk));
    const int vs = __shfl(lslot, __ffsll(static_cast<unsigned long long>(vb)) - 1, kInsG);
    if (ev.keys) emit_entry<V4>(ev, t, gk, gs, table_rows + static_cast<uint64_t>(vs) * t.dim, nullptr, lane);
    own_write_slot(o, t, vs, k, d, score, lane);
    write_row(vs);
  } else if (ev.keys) {
    emit_entry<V4>(ev, t, k, score, row, nullptr, lane);
  }
}

// Lowest (score, key) of a full bucket as recorded by the bucket's last owner
// (dual mode). Read-only while inserts are probed, so every group of one
// probe kernel sees the same values; a record that is stale (a resident key's
// score changed since) only makes the bucket choice less good, never the
// table inconsistent. A full bucket without a record (not produced by the
// owner kernel, which records every bucket it leaves full) counts as lowest.
// Read by the lane that links the key (the result is only used there).
__device__ __forceinline__ void cached_lowest(const TableView& t, uint32_t b, uint64_t* ms, uint64_t* mk) {
  const ulonglong2 c = *reinterpret_cast<const ulonglong2*>(t.bmin + 2 * static_cast<uint64_t>(b));
  uint64_t s = c.x, k = c.y;
  if (k == ~0ull) {
    s = 0;
    k = 0;
  }
  *ms = s;
  *mk = k;
}

// Insert, first kernel: a group of G lanes per key probes the key's
// candidate bucket(s). A resident key is updated in place (value row and
// score only, no structural change, so concurrent probes stay valid). A
// missing key is pushed onto the chain of the bucket it goes to: in
// single-bucket mode its bucket; in dual-bucket mode the bucket Algorithm 3
// picks: the less-occupied one if either has room (tie: the first; occupancy
// counted from the digest lines, which this kernel never changes), else the
// one whose recorded lowest (score, key) is lower (records are only written
// by the owner kernel). Every input of the choice is therefore fixed for the
// whole kernel, so two copies of one key always choose the same bucket.
// next[i] receives the previously pushed key of that chain, kNoIdx for the
// first one (whose group will own the bucket), kSkipIdx for keys that need
// nothing more; target[i] the bucket, with kFullBit set when the bucket had
// no empty slot. The updates all happen before any insert of the batch,
// which is one of the serial orders of the batch.
// FETCH (find_or_insert): a resident key's stored row is copied out to the
// caller's row instead, its score replaced, and found[i] (if given) tells
// hits from misses. link = false (serial inserter follows): missing keys are
// only marked (next[i] = kNoIdx) and no chain is built.
template <int G, bool V4, bool DUAL, bool NT, bool FETCH>
__global__ __launch_bounds__(kBlock) void upsert_probe_kernel(TableView t, uint64_t n,
                                                              const uint64_t* __restrict__ keys,
                                                              float* __restrict__ values,
                                                              const uint64_t* __restrict__ scores,
                                                              uint8_t* __restrict__ found,
                                                              uint32_t* __restrict__ next,
                                                              uint32_t* __restrict__ target, bool link) {
  const uint64_t i = (static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x) / G;
  const int lane = static_cast<int>(threadIdx.x & (G - 1));
  if (i >= n) return;
  const uint64_t k = keys[i];
  // loaded with the key: stored at the end without waiting behind the row
  const uint64_t score = scores[i];
  if (is_reserved(k)) {
    if (lane == 0) {
      next[i] = kSkipIdx;
      if (FETCH && found) found[i] = 0;
    }
    return;
  }
  uint32_t o1 = 0, o2 = 0;
  int64_t p;
  // (insert_or_assign with rows of one 16-byte piece per lane: the input
  // row, needed by a hit, is requested together with the candidate keys, as
  // soon as the digest lines show a candidate. Measured at 2^26 slots: dim 32
  // (8 lanes) 131 vs 134 us per 2^20 keys; at dim 64 the overlap no longer
  // pays for the rows read for missing keys with a false candidate, 160 vs
  // 157 us, so larger rows are read after the match.)
  const bool in_regs = !FETCH && V4 && t.dim <= 4 * G;
  GroupRow<G> rr;
  if constexpr (FETCH) {
    p = probe<G, DUAL>(t, k, lane, &o1, &o2);
  } else {
    p = probe_prefetch<G, DUAL>(t, k, lane, &o1, &o2, in_regs, values + i * t.dim, rr);
  }
  if (p >= 0) {
    if constexpr (FETCH) {
      // (host-resident rows: cacheable loads, as in find)
      if (static_cast<uint64_t>(p) >= t.split) {
        copy_row<G, V4, false>(values + i * t.dim, row_of(t, static_cast<uint64_t>(p)), t.dim, lane);
      } else {
        copy_row<G, V4, NT>(values + i * t.dim, row_of(t, static_cast<uint64_t>(p)), t.dim, lane);
      }
      if (lane == 0) {
        t.scores[p] = score;
        next[i] = kUpdIdx;
        if (found) found[i] = 1;
      }
    } else {
      // In-place update. Occurrences of one key in a batch would otherwise
      // write its row piece by piece at once; the slot's claim bit lets the
      // first one alone write the row and the score. A row of up to two
      // pieces per lane is loaded while the claim is in flight (one round
      // trip for both).
      const float* src = values + i * t.dim;
      float* dst = row_of(t, static_cast<uint64_t>(p));
      uint32_t won = 1;
      const bool pair = V4 && !in_regs && t.claims && t.dim <= 8 * G;
      GroupRow<G, 2> r2;
      if (t.claims) {
        uint32_t mine = 0;
        if (lane == 0) mine = claim_slot(t, static_cast<uint64_t>(p)) ? 1u : 0u;
        if (pair) group_row_load<G, 2>(r2, src, t.dim, lane);
        won = __shfl(mine, 0, G);
      }
      if (won) {
        if (in_regs) {
          group_row_store<G>(rr, dst, t.dim, lane);
        } else if (pair) {
          group_row_store<G, 2>(r2, dst, t.dim, lane);
        } else {
          copy_row<G, V4, NT>(dst, src, t.dim, lane);
        }
      }
      if (lane == 0) {
        if (won) t.scores[p] = score;
        if (won && t.claims) target[i] = static_cast<uint32_t>(static_cast<uint64_t>(p) / kSlots);
        next[i] = !won ? kSkipIdx : t.claims ? kHitIdx : kUpdIdx;
      }
    }
    return;
  }
  if (FETCH && found && lane == 0) found[i] = 0;
  if (!link) {
    if (lane == 0) next[i] = kNoIdx;
    return;
  }
  // the rest (bucket choice and chain link) is the work of one lane
  if (lane != 0) return;
  const uint64_t h = fmix64(k);
  uint32_t tb = bucket_of(t, h);
  uint32_t tocc = o1;
  if constexpr (DUAL) {
    const uint32_t b1 = tb;
    const uint32_t b2 = bucket_of(t, fmix64(k ^ kSecondSalt));
    if (b2 != b1) {
      if (o1 < kSlots || o2 < kSlots) {
        tb = (o1 <= o2) ? b1 : b2;
        tocc = (o1 <= o2) ? o1 : o2;
      } else {
        uint64_t s1, k1, s2, k2;
        cached_lowest(t, b1, &s1, &k1);
        cached_lowest(t, b2, &s2, &k2);
        tb = (s2 < s1 || (s2 == s1 && k2 < k1)) ? b2 : b1;
      }
    }
  }
  target[i] = tb | (tocc >= kSlots ? kFullBit : 0u);
  // the head carries this call's epoch, so a head left by an earlier call
  // reads as an empty chain and no kernel has to reset it (epoch 0, the
  // epoch of calls captured into a graph, whose owners reset their heads)
  const uint64_t old = __hip_atomic_exchange(t.head + tb, (static_cast<uint64_t>(t.epoch) << 32) | i,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  next[i] = static_cast<uint32_t>(old >> 32) == t.epoch ? static_cast<uint32_t>(old) : kNoIdx;
}

// Resets the claim bits of bucket b's 128 slots (one 16-byte store).
__device__ __forceinline__ void clear_claims(const TableView& t, uint32_t b) {
  *reinterpret_cast<uint4*>(t.claim + 4 * static_cast<uint64_t>(b)) = make_uint4(0u, 0u, 0u, 0u);
}

// State of a bucket owned by a 16-lane group in the owner kernel: its
// occupancy (group-uniform), this lane's 8 digest bytes and, once loaded, the
// scores of this lane's 8 slots (slots 8*lane .. 8*lane+7) and the keys it
// knows. Only the lane owning a slot reads or writes that slot's key, score
// and digest. The score column is loaded for a full bucket; keys are read
// only where a victim must be chosen among slots at the lowest score, a
// lane's 8 at a time (one 64-byte burst, the price of reading one), and every
// key the group writes stays known.
struct Bucket {
  uint32_t b;
  uint32_t occ;
  uint32_t dig0, dig1;
  bool scols;      // sc valid (group-uniform)
  uint32_t kval;   // this lane's slots whose kc is valid (bit u: slot 8*lane+u)
  uint32_t wmask;  // this lane's slots written by this kernel (their kc is valid)
  uint64_t sc[8];
  uint64_t kc[8];
};

__device__ __forceinline__ void bucket_load_scores(Bucket& o, const TableView& t, int lane) {
  const uint64_t base = static_cast<uint64_t>(o.b) * kSlots + lane * 8;
#pragma unroll
  for (int u = 0; u < 8; u += 2) {
    const ulonglong2 a = *reinterpret_cast<const ulonglong2*>(t.scores + base + u);
    o.sc[u] = a.x;
    o.sc[u + 1] = a.y;
  }
  o.scols = true;
}

// Lowest (score, key) entry of the owned full bucket (group-uniform score and
// key, and its slot). Keys of the slots at the lowest score that are not in
// registers yet are loaded (one round trip, none when all are known).
__device__ __forceinline__ int bucket_lowest(Bucket& o, const TableView& t, int lane, uint64_t* min_score,
                                             uint64_t* min_key) {
  if (!o.scols) bucket_load_scores(o, t, lane);
  uint64_t ls = o.sc[0];
#pragma unroll
  for (int u = 1; u < 8; ++u) ls = o.sc[u] < ls ? o.sc[u] : ls;
  const uint64_t gs = group_min<kInsG>(ls);
  // a lane with an unknown key at the lowest score reads all 8 of its keys:
  // the same 64-byte burst as one key, in four 16-byte loads
  bool need = false;
#pragma unroll
  for (int u = 0; u < 8; ++u) need |= o.sc[u] == gs && !((o.kval >> u) & 1u);
  if (need) {
    const uint64_t base = static_cast<uint64_t>(o.b) * kSlots + lane * 8;
#pragma unroll
    for (int u = 0; u < 8; u += 2) {
      const ulonglong2 c = *reinterpret_cast<const ulonglong2*>(t.keys + base + u);
      o.kc[u] = c.x;
      o.kc[u + 1] = c.y;
    }
    o.kval = 0xFFu;
  }
  uint64_t lk = ~0ull;
  int lslot = -1;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (o.sc[u] == gs && (lslot < 0 || o.kc[u] < lk)) {
      lk = o.kc[u];
      lslot = lane * 8 + u;
    }
  }
  const uint64_t gk = group_min<kInsG>(lslot >= 0 ? lk : ~0ull);
  const uint64_t vb = group_bits<kInsG>(__ballot(lslot >= 0 && lk == gk));
  *min_score = gs;
  *min_key = gk;
  return __shfl(lslot, __ffsll(static_cast<unsigned long long>(vb)) - 1, kInsG);
}

// Writes slot s (key only when `is_new`, then digest, score) through its owner
// lane and keeps the register copies current.
__device__ __forceinline__ void bucket_write(Bucket& o, const TableView& t, int s, bool is_new, uint64_t k,
                                             uint32_t d, uint64_t score, int lane) {
  if (lane != (s >> 3)) return;
  const uint64_t p = static_cast<uint64_t>(o.b) * kSlots + s;
  t.scores[p] = score;
  if (is_new) {
    t.keys[p] = k;
    t.digests[p] = static_cast<uint8_t>(d);
    const int sh = (s & 3) * 8;
    if (s & 4) {
      o.dig1 = (o.dig1 & ~(0xFFu << sh)) | (d << sh);
    } else {
      o.dig0 = (o.dig0 & ~(0xFFu << sh)) | (d << sh);
    }
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const bool here = u == (s & 7);
    if (o.scols) o.sc[u] = here ? score : o.sc[u];
    o.kc[u] = here ? k : o.kc[u];
  }
  o.kval |= 1u << (s & 7);
  o.wmask |= 1u << (s & 7);
}

// Algorithm 2 for one key against the owned bucket, with the input row already
// loaded. `fresh`: the key is known to be absent (a chain's first key, which
// the probe kernel found missing, before anything was inserted).
template <bool V4, bool EVICT>
__device__ __forceinline__ bool bucket_apply(Bucket& o, const TableView& t, uint64_t k, uint64_t score,
                                             const RowRegs& rr, const float* row, bool in_regs, bool fresh,
                                             const EvictStage& st, uint32_t idx, int lane) {
  const uint32_t d = digest_of(fmix64(k));
  float* const rows = row_of(t, static_cast<uint64_t>(o.b) * kSlots);
  auto write_row = [&](int s) {
    if (in_regs) {
      row_regs_store(rr, rows + static_cast<uint64_t>(s) * t.dim, t.dim, lane);
    } else {
      copy_row<kInsG, V4, true>(rows + static_cast<uint64_t>(s) * t.dim, row, t.dim, lane);
    }
  };
  // A chain key was absent when the probe kernel ran and only this group has
  // written the bucket since, so it can only be a key this group wrote (a
  // duplicate earlier in the chain): the hit check compares the written
  // slots, whose keys are in registers, and loads nothing.
  int hit = -1;
  if (!fresh) {
    int lh = -1;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (((o.wmask >> u) & 1u) && o.kc[u] == k) lh = lane * 8 + u;
    const uint64_t hb = group_bits<kInsG>(__ballot(lh >= 0));
    if (hb) hit = __shfl(lh, __ffsll(static_cast<unsigned long long>(hb)) - 1, kInsG);
  }
  if (hit >= 0) {
    bucket_write(o, t, hit, false, k, d, score, lane);
    write_row(hit);
    if (EVICT && lane == 0) st.kind[idx] = 0;
    return true;
  }
  if (o.occ < kSlots) {
    const int s = static_cast<int>(o.occ);
    bucket_write(o, t, s, true, k, d, score, lane);
    write_row(s);
    o.occ += 1;
    if (EVICT && lane == 0) st.kind[idx] = 0;
    return false;
  }
  uint64_t gs, gk;
  const int vs = bucket_lowest(o, t, lane, &gs, &gk);
  if (score > gs || (score == gs && k > gk)) {
    if constexpr (EVICT) {
      // the victim's row is staged (read by the lanes that wrote it, if this
      // kernel did) before the new row overwrites it
      copy_row<kInsG, V4, false>(st.rows + static_cast<uint64_t>(idx) * t.dim,
                                 rows + static_cast<uint64_t>(vs) * t.dim, t.dim, lane);
      if (lane == 0) {
        st.keys[idx] = gk;
        st.scores[idx] = gs;
        st.kind[idx] = 1;
      }
    }
    bucket_write(o, t, vs, true, k, d, score, lane);
    write_row(vs);
  } else if constexpr (EVICT) {
    if (lane == 0) {
      st.keys[idx] = k;
      st.scores[idx] = score;
      st.kind[idx] = 2;
    }
  }
  return false;
}

// Insert, second kernel: the first-pushed key of each chain (next ==
// kNoIdx) owns that bucket for the whole kernel. A block lists the owners
// among its kOwnerBlock keys in LDS and deals them out to its 16-lane groups
// in turn. An owner loads, in one round trip, the bucket's digest line, the
// chain head, its key's row and - when the probe kernel saw the bucket full -
// the scores of all slots; it applies its own key, then the chain from its
// head down to itself (Algorithm 2, each chain key costing one round trip for
// its inputs), and writes the occupancy if it changed. With distinct keys any
// order within a chain gives the same bucket contents. The kernel waits on
// memory more than anything else; blocks of 128 threads (two waves) gave
// 43 us per 2^20 keys of the 10 %-new mix against 46 us with 256 (a block
// waits at its barrier for its slowest wave) and 55 us with 512.
// STATS: the block's outcome counts (updated, inserted, evicted, rejected)
// are added to stat_slots[c * kStatSlots + block mod kStatSlots].
constexpr int kOwnerBlock = 128;

template <bool V4, bool DUAL, bool EVICT, bool STATS>
__global__ __launch_bounds__(kOwnerBlock) void upsert_owner_kernel(TableView t, uint64_t n,
                                                              const uint64_t* __restrict__ keys,
                                                              const float* __restrict__ values,
                                                              const uint64_t* __restrict__ scores,
                                                              const uint32_t* __restrict__ next,
                                                              const uint32_t* __restrict__ target,
                                                              EvictStage st, bool clear_all,
                                                              unsigned long long* __restrict__ stat_slots) {
  // The block's owners (keys with next == kNoIdx) are listed in LDS and dealt
  // out to its groups in turn, so that every group serves about the same
  // number of buckets.
  __shared__ uint32_t s_idx[kOwnerBlock];
  __shared__ uint32_t s_tgt[kOwnerBlock];
  __shared__ uint64_t s_key[kOwnerBlock];
  __shared__ uint64_t s_score[kOwnerBlock];
  __shared__ uint32_t s_count;
  __shared__ uint32_t s_stat[4];
  const uint64_t mine = static_cast<uint64_t>(blockIdx.x) * kOwnerBlock + threadIdx.x;
  const int lane = static_cast<int>(threadIdx.x & (kInsG - 1));
  if (threadIdx.x == 0) s_count = 0;
  if (STATS && threadIdx.x < 4) s_stat[threadIdx.x] = 0;
  __syncthreads();
  if constexpr (STATS) {
    // keys found resident by the probe kernel: updated in place (the claim
    // winner alone when claims are taken), or read by find_or_insert
    const uint32_t nx = mine < n ? next[mine] : kSkipIdx;
    const uint64_t upd = __ballot(nx == kHitIdx || nx == kUpdIdx);
    if (wave_lane() == 0 && upd) atomicAdd(&s_stat[0], static_cast<uint32_t>(__popcll(upd)));
  }
  if (mine < n) {
    const uint32_t nx = next[mine];
    if (nx == kNoIdx) {
      const uint32_t e = atomicAdd(&s_count, 1u);
      s_idx[e] = static_cast<uint32_t>(mine);
      s_tgt[e] = target[mine];
      s_key[e] = keys[mine];
      s_score[e] = scores[mine];
    } else if (nx == kHitIdx && !clear_all) {
      clear_claims(t, target[mine]);
    }
  }
  if (clear_all) {
    // the claims of the probe kernel, cleared wholesale: this block's share of
    // the buckets (chosen when that is cheaper than one store per update)
    const uint64_t per = (t.nb + gridDim.x - 1) / gridDim.x;
    const uint64_t b0 = static_cast<uint64_t>(blockIdx.x) * per;
    const uint64_t b1 = b0 + per < t.nb ? b0 + per : t.nb;
    for (uint64_t b = b0 + threadIdx.x; b < b1; b += kOwnerBlock) clear_claims(t, static_cast<uint32_t>(b));
  }
  __syncthreads();
  const uint32_t owners = s_count;
  const bool in_regs = V4 && t.dim <= 8 * kInsG;
  for (uint32_t e = threadIdx.x / kInsG; e < owners; e += kOwnerBlock / kInsG) {
    const uint32_t i = s_idx[e];
    const uint32_t tgt = s_tgt[e];
    const uint64_t k = s_key[e];
    const uint64_t score = s_score[e];
    Bucket o;
    o.b = tgt & ~kFullBit;
    o.scols = false;
    o.kval = 0;
    o.wmask = 0;
    // The head was set by the probe kernel's exchanges (this call's epoch,
    // as the bucket has an owner) and is published by the kernel boundary.
    // A call replayed from a graph runs with the epoch it was captured with
    // (0), so its owners reset the heads they used for the next replay.
    uint32_t head = 0;
    if (lane == 0) {
      head = static_cast<uint32_t>(t.head[o.b]);
      if (t.epoch == 0) t.head[o.b] = kEmptyHead;
    }
    const uint2 dv = *reinterpret_cast<const uint2*>(t.digests + static_cast<uint64_t>(o.b) * kSlots + lane * 8);
    RowRegs rr;
    const float* row = values + static_cast<uint64_t>(i) * t.dim;
    if (in_regs) row_regs_load(rr, row, t.dim, lane);
    if (tgt & kFullBit) bucket_load_scores(o, t, lane);
    o.dig0 = dv.x;
    o.dig1 = dv.y;
    uint32_t c = 8 - __builtin_popcount(zero_byte_bits(o.dig0)) - __builtin_popcount(zero_byte_bits(o.dig1));
#pragma unroll
    for (int sh = kInsG / 2; sh > 0; sh >>= 1) c += __shfl_xor(c, sh, kInsG);
    o.occ = c;
    const uint32_t occ0 = o.occ;
    // A chain holds only keys the probe found missing, so the owner's own
    // key, applied first, is known to be absent.
    bucket_apply<V4, EVICT>(o, t, k, score, rr, row, in_regs, true, st, i, lane);
    uint32_t occurrences = 1, repeats = 0;  // (outcome counts)
    // The chain holds at most n keys and ends at this owner's own key; the
    // index and step bounds only guard against a corrupted chain.
    uint32_t cur = __shfl(head, 0, kInsG);
    for (uint64_t step = 0; cur != i && cur < n && step < n; ++step) {
      const uint32_t after = next[cur];
      const uint64_t kc = keys[cur];
      const uint64_t scc = scores[cur];
      const float* rowc = values + static_cast<uint64_t>(cur) * t.dim;
      if (in_regs) row_regs_load(rr, rowc, t.dim, lane);
      const bool again = bucket_apply<V4, EVICT>(o, t, kc, scc, rr, rowc, in_regs, false, st, cur, lane);
      if constexpr (STATS) {
        occurrences += 1;
        repeats += again ? 1u : 0u;
      }
      cur = after;
    }
    if constexpr (STATS) {
      // Every slot written by this kernel holds one of the chain's keys at the
      // end (inserted); a written slot below the occupancy the call started
      // with held a key resident before the call, which has left (evicted);
      // the chain's other keys are not resident (rejected).
      const int first = lane * 8;
      const uint32_t before = occ0 >= static_cast<uint32_t>(first + 8) ? 0xFFu
                              : occ0 > static_cast<uint32_t>(first) ? (1u << (occ0 - first)) - 1u
                                                                     : 0u;
      uint32_t packed = static_cast<uint32_t>(__popc(o.wmask)) | (static_cast<uint32_t>(__popc(o.wmask & before)) << 16);
#pragma unroll
      for (int sh = kInsG / 2; sh > 0; sh >>= 1) packed += __shfl_xor(packed, sh, kInsG);
      if (lane == 0) {
        const uint32_t ins = packed & 0xFFFFu;
        atomicAdd(&s_stat[1], ins);
        atomicAdd(&s_stat[2], packed >> 16);
        atomicAdd(&s_stat[3], occurrences - repeats - ins);
      }
    }
    if (DUAL && o.occ >= kSlots && group_bits<kInsG>(__ballot(o.wmask != 0)) != 0) {
      // record the bucket's lowest (score, key) for later dual-bucket choices
      // (a chain that wrote nothing - every key turned away - leaves the
      // bucket, and so its record, as it was)
      uint64_t gs, gk;
      (void)bucket_lowest(o, t, lane, &gs, &gk);
      if (lane == 0) {
        ulonglong2 rec;
        rec.x = gs;
        rec.y = gk;
        *reinterpret_cast<ulonglong2*>(t.bmin + 2 * static_cast<uint64_t>(o.b)) = rec;
      }
    }
    if (lane == 0 && o.occ != occ0) t.occ[o.b] = o.occ;
  }
  if constexpr (STATS) {
    __syncthreads();
    if (threadIdx.x < 4 && s_stat[threadIdx.x] != 0)
      atomicAdd(stat_slots + threadIdx.x * kStatSlots + blockIdx.x % kStatSlots,
                static_cast<unsigned long long>(s_stat[threadIdx.x]));
  }
}

// Sums the outcome slots into the caller's four counters and clears them
// (one block of kStatSlots threads).
__global__ __launch_bounds__(kStatSlots) void outcome_flush_kernel(unsigned long long* __restrict__ slots,
                                                                   unsigned long long* __restrict__ out) {
  __shared__ unsigned long long part[4][kStatSlots / 64];
  const int w = static_cast<int>(threadIdx.x / 64);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    unsigned long long v = slots[c * kStatSlots + threadIdx.x];
    slots[c * kStatSlots + threadIdx.x] = 0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if (wave_lane() == 0) part[c][w] = v;
  }
  __syncthreads();
  if (threadIdx.x < 4) {
    unsigned long long sum = 0;
#pragma unroll
    for (int v = 0; v < kStatSlots / 64; ++v) sum += part[threadIdx.x][v];
    atomicAdd(out + threadIdx.x, sum);
  }
}

// insert_and_evict, parallel inserter: the staged departures are compacted
// in batch-index order without atomics. A chunk is 1024 consecutive batch
// indices (256 threads x 4); the count kernel writes each chunk's number of
// departures, the write kernel sums the counts of the chunks before its own
// (a few KB, cached), ranks its departures with wave ballots and copies them
// out, 16 lanes per row; the last chunk writes the total.
constexpr int kChunk = 4 * kBlock;

__device__ __forceinline__ bool departs(uint64_t i, uint64_t n, const uint32_t* next, const EvictStage& st,
                                        uint32_t* kd) {
  *kd = 0;
  if (i < n && in_chain(next[i])) *kd = st.kind[i];
  return *kd != 0;
}

__global__ __launch_bounds__(kBlock) void evict_count_kernel(uint64_t n, const uint32_t* __restrict__ next,
                                                             EvictStage st, uint32_t* __restrict__ chunk_count) {
  __shared__ uint32_t part[kBlock / 64];
  const uint64_t c0 = static_cast<uint64_t>(blockIdx.x) * kChunk;
  uint32_t cnt = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    uint32_t kd;
    cnt += departs(c0 + r * kBlock + threadIdx.x, n, next, st, &kd) ? 1u : 0u;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
  if (wave_lane() == 0) part[threadIdx.x / 64] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t total = 0;
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w) total += part[w];
    chunk_count[blockIdx.x] = total;
  }
}

template <bool V4>
__global__ __launch_bounds__(kBlock) void evict_write_kernel(TableView t, uint64_t n,
                                                             const uint32_t* __restrict__ next, EvictStage st,
                                                             const float* __restrict__ values,
                                                             const uint32_t* __restrict__ chunk_count,
                                                             Evicted out) {
  __shared__ unsigned long long red[kBlock / 64];
  __shared__ uint32_t cnt[4][kBlock / 64];
  __shared__ uint32_t src[kChunk];
  const int w = static_cast<int>(threadIdx.x / 64);
  const int lane = wave_lane();
  // departures of the chunks before this one
  unsigned long long before = 0;
  for (uint32_t c = threadIdx.x; c < blockIdx.x; c += kBlock) before += chunk_count[c];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) before += __shfl_xor(before, o, 64);
  if (lane == 0) red[w] = before;
  const uint64_t c0 = static_cast<uint64_t>(blockIdx.x) * kChunk;
  uint32_t kd[4];
  uint64_t bal[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const bool d = departs(c0 + r * kBlock + threadIdx.x, n, next, st, &kd[r]);
    bal[r] = __ballot(d);
    if (lane == 0) cnt[r][w] = static_cast<uint32_t>(__popcll(bal[r]));
  }
  __syncthreads();
  unsigned long long base = 0;
#pragma unroll
  for (int v = 0; v < kBlock / 64; ++v) base += red[v];
  // rank = departures at smaller indices in this chunk: order (r, wave, lane)
  uint32_t total = 0;
  uint32_t rank[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    uint32_t off = total;
#pragma unroll
    for (int v = 0; v < kBlock / 64; ++v) off += v < w ? cnt[r][v] : 0u;
    rank[r] = off + static_cast<uint32_t>(__popcll(bal[r] & ((1ull << lane) - 1)));
#pragma unroll
    for (int v = 0; v < kBlock / 64; ++v) total += cnt[r][v];
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) *out.count = base + total;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (kd[r] == 0) continue;
    const uint64_t i = c0 + r * kBlock + threadIdx.x;
    out.keys[base + rank[r]] = st.keys[i];
    if (out.scores) out.scores[base + rank[r]] = st.scores[i];
    src[rank[r]] = static_cast<uint32_t>(r * kBlock + threadIdx.x) | (kd[r] == 1 ? 0x80000000u : 0u);
  }
  if (!out.values) return;
  __syncthreads();
  const int g = static_cast<int>(threadIdx.x / kInsG);
  const int gl = static_cast<int>(threadIdx.x & (kInsG - 1));
  for (uint32_t e = g; e < total; e += kBlock / kInsG) {
    const uint32_t sv = src[e];
    const uint64_t j = c0 + (sv & 0x7FFFFFFFu);
    const float* from = (sv & 0x80000000u) ? st.rows + j * t.dim : values + j * t.dim;
    copy_row<kInsG, V4, true>(out.values + (base + e) * t.dim, from, t.dim, gl);
  }
}

// Serial inserter: one 16-lane group applies the whole batch in input order
// (Algorithm 2, or Algorithm 3 in dual mode, one key at a time). With `skip`
// (the marks of a probe pass that already updated the resident keys), only
// the keys marked kNoIdx are applied. ev.keys != nullptr: evicted and
// turned-away entries are handed back.
template <bool V4, bool DUAL>
__global__ __launch_bounds__(64) void upsert_serial_kernel(TableView t, uint64_t n,
                                                           const uint64_t* __restrict__ keys,
                                                           const float* __restrict__ values,
                                                           const uint64_t* __restrict__ scores,
                                                           const uint32_t* __restrict__ skip,
                                                           const uint32_t* __restrict__ skip_bucket, Evicted ev) {
  if (threadIdx.x >= kInsG) return;
  const int lane = static_cast<int>(threadIdx.x);
  for (uint64_t i = 0; i < n; ++i) {
    if (skip && skip[i] != kNoIdx) {
      // an update of the probe pass: its claim is released here
      if (skip[i] == kHitIdx && lane == 0) clear_claims(t, skip_bucket[i]);
      continue;
    }
    const uint64_t k = keys[i];
    if (is_reserved(k)) continue;
    const float* row = values + i * t.dim;
    const uint64_t score = scores[i];
    const uint64_t h = fmix64(k);
    const uint32_t d = digest_of(h);
    const uint32_t pat = d * 0x01010101u;
    const uint32_t b1 = bucket_of(t, h);
    const uint32_t b2 = DUAL ? bucket_of(t, fmix64(k ^ kSecondSalt)) : b1;
    Owned o1;
    own_load(o1, t, b1, lane);
    if (!DUAL || b2 == b1) {
      const uint32_t occ0 = o1.occ;
      own_upsert<V4>(o1, t, k, row, score, ev, lane);
      if (o1.occ != occ0) own_store_occ(o1, t, lane);
      continue;
    }
    int s = own_find(o1, t, k, pat, lane);
    if (s >= 0) {
      own_write_score(o1, t, s, score, lane);
      own_write_row<V4>(o1, t, s, row, lane);
      continue;
    }
    Owned o2;
    own_load(o2, t, b2, lane);
    s = own_find(o2, t, k, pat, lane);
    if (s >= 0) {
      own_write_score(o2, t, s, score, lane);
      own_write_row<V4>(o2, t, s, row, lane);
      continue;
    }
    if (o1.occ < kSlots || o2.occ < kSlots) {
      Owned& o = (o1.occ <= o2.occ) ? o1 : o2;
      s = static_cast<int>(o.occ);
      own_write_slot(o, t, s, k, d, score, lane);
      own_write_row<V4>(o, t, s, row, lane);
      o.occ += 1;
      own_store_occ(o, t, lane);
      continue;
    }
    uint64_t ms1, mk1, ms2, mk2;
    int v1, v2;
    own_lowest(o1, t, lane, &ms1, &mk1, &v1);
    own_lowest(o2, t, lane, &ms2, &mk2, &v2);
    const bool second = ms2 < ms1 || (ms2 == ms1 && mk2 < mk1);
    Owned& o = second ? o2 : o1;
    const uint64_t ms = second ? ms2 : ms1, mk = second ? mk2 : mk1;
    const int vs = second ? v2 : v1;
    if (score > ms || (score == ms && k > mk)) {
      if (ev.keys)
        emit_entry<V4>(ev, t, mk, ms, row_of(t, static_cast<uint64_t>(o.b) * kSlots + vs), nullptr,
                       lane);
      own_write_slot(o, t, vs, k, d, score, lane);
      own_write_row<V4>(o, t, vs, row, lane);
    } else if (ev.keys) {
      emit_entry<V4>(ev, t, k, score, row, nullptr, lane);
    }
  }
}

// ------------------------------------------------------------------ setup --

__global__ __launch_bounds__(kBlock) void init_kernel(TableView t) {
  const uint64_t cap = t.nb * kSlots;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
  for (uint64_t p = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x; p < cap; p += stride) {
    t.keys[p] = ~0ull;
    t.scores[p] = 0;
    t.digests[p] = 0;
    if (p < t.nb * 4) t.claim[p] = 0;
    if (p < t.nb) {
      t.occ[p] = 0;
      t.head[p] = kEmptyHead;
      if (t.bmin) {
        t.bmin[2 * p] = 0;
        t.bmin[2 * p + 1] = ~0ull;
      }
    }
  }
}

__global__ __launch_bounds__(kBlock) void reset_heads_kernel(TableView t) {
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
  for (uint64_t b = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x; b < t.nb; b += stride)
    t.head[b] = kEmptyHead;
}

uint32_t grid_for(uint64_t threads) {
  return static_cast<uint32_t>((threads + kBlock - 1) / kBlock);
}

// Lanes per key for find/assign/insert probes: 4 for rows up to 64 bytes,
// 8 up to 256 bytes (measured best at 256-byte rows), 16 above; t.lanes
// overrides it (4, 8 or 16).
int lanes_for(const TableView& t) {
  if (t.lanes == 4 || t.lanes == 8 || t.lanes == 16) return static_cast<int>(t.lanes);
  if (t.dim <= 16) return 4;
  if (t.dim <= 64) return 8;
  return 16;
}

// Launch, with the timer's event pair recorded by the dispatch when timing.
#define HKV_LAUNCH(timer, name, kernel, grid, block, stream, ...)                          \
  do {                                                                                      \
    hipEvent_t hkv_e0_ = nullptr, hkv_e1_ = nullptr;                                        \
    if ((timer) && (timer)->take(&hkv_e0_, &hkv_e1_)) {                                     \
      hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, hkv_e0_, hkv_e1_, 0, __VA_ARGS__); \
      (timer)->launched(name, hkv_e0_, hkv_e1_);                                            \
    } else {                                                                                \
      hipLaunchKernelGGL(kernel, grid, block, 0, stream, __VA_ARGS__);                      \
    }                                                                                       \
  } while (0)

template <int G, bool V4, bool DUAL>
hipError_t find_g(const TableView& t, uint64_t n, const uint64_t* keys, float* out, uint8_t* found,
                  uint64_t* sc, hipStream_t s, KernelTimer* tm) {
  if (t.split < t.nb * kSlots) {
    // some rows in host memory: keys partitioned over the XCDs
    const uint64_t chunk = static_cast<uint64_t>(kBlock / G) * kXcds;
    const uint64_t blocks = (n + chunk - 1) / chunk * kXcds;
    HKV_LAUNCH(tm, "find", (find_xcd_kernel<G, V4, DUAL, true>), dim3(static_cast<uint32_t>(blocks)),
               dim3(kBlock), s, t, n, keys, out, found, sc);
    return hipGetLastError();
  }
  HKV_LAUNCH(tm, "find", (find_kernel<G, V4, DUAL, true>), dim3(grid_for(n * G)), dim3(kBlock), s, t, n,
             keys, out, found, sc);
  return hipGetLastError();
}

template <int G, bool V4, bool DUAL>
hipError_t assign_g(const TableView& t, uint64_t n, const uint64_t* keys, const float* v,
                    const uint64_t* sc, hipStream_t s, KernelTimer* tm) {
  HKV_LAUNCH(tm, "assign", (assign_kernel<G, V4, DUAL>), dim3(grid_for(n * G)), dim3(kBlock), s, t, n,
             keys, v, sc);
  return hipGetLastError();
}

template <int G, bool V4, bool DUAL, bool FETCH>
hipError_t probe_g(const TableView& t, uint64_t n, const InsertCall& c, uint32_t* next, uint32_t* target,
                   bool link, hipStream_t s, KernelTimer* tm) {
  HKV_LAUNCH(tm, FETCH ? "probe_fetch" : "upsert_probe", (upsert_probe_kernel<G, V4, DUAL, true, FETCH>),
             dim3(grid_for(n * G)), dim3(kBlock), s, t, n, c.keys, c.values, c.scores, c.found, next, target,
             link);
  return hipGetLastError();
}

template <bool V4, bool DUAL, bool STATS>
hipError_t owner_l(const TableView& t, uint64_t n, const InsertCall& c, const uint32_t* next,
                   const uint32_t* target, hipStream_t s, KernelTimer* tm) {
  const EvictStage st{c.st_kind, c.st_keys, c.st_scores, c.st_rows};
  // Claims of the probe kernel: cleared wholesale (16 bytes per bucket) when
  // that costs less than one 16-byte store per update, else per update.
  // (find_or_insert takes no claims.)
  const bool clear_all = t.claims && !c.fetch && t.nb <= 4 * n;
  hipError_t e = hipSuccess;
  if (!c.ev_keys) {
    HKV_LAUNCH(tm, "upsert_owner", (upsert_owner_kernel<V4, DUAL, false, STATS>),
               dim3(static_cast<uint32_t>((n + kOwnerBlock - 1) / kOwnerBlock)), dim3(kOwnerBlock), s, t, n,
               c.keys, c.values, c.scores, next, target, st, clear_all, c.stat_slots);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else {
    HKV_LAUNCH(tm, "owner_evict", (upsert_owner_kernel<V4, DUAL, true, STATS>),
               dim3(static_cast<uint32_t>((n + kOwnerBlock - 1) / kOwnerBlock)), dim3(kOwnerBlock), s, t, n,
               c.keys, c.values, c.scores, next, target, st, clear_all, c.stat_slots);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const Evicted out{c.ev_keys, c.ev_values, c.ev_scores, c.ev_count};
    const uint32_t chunks = static_cast<uint32_t>((n + kChunk - 1) / kChunk);
    HKV_LAUNCH(tm, "evict_count", evict_count_kernel, dim3(chunks), dim3(kBlock), s, n, next, st,
               c.chunk_count);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    HKV_LAUNCH(tm, "evict_write", (evict_write_kernel<V4>), dim3(chunks), dim3(kBlock), s, t, n, next, st,
               c.values, c.chunk_count, out);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if constexpr (STATS) {
    HKV_LAUNCH(tm, "outcomes", outcome_flush_kernel, dim3(1), dim3(kStatSlots), s, c.stat_slots, c.outcomes);
    e = hipGetLastError();
  }
  return e;
}

template <bool V4, bool DUAL>
hipError_t find_d(const TableView& t, uint64_t n, const uint64_t* keys, float* out, uint8_t* found,
                  uint64_t* sc, hipStream_t s, KernelTimer* tm) {
  switch (lanes_for(t)) {
    case 4: return find_g<4, V4, DUAL>(t, n, keys, out, found, sc, s, tm);
    case 8: return find_g<8, V4, DUAL>(t, n, keys, out, found, sc, s, tm);
    default: return find_g<16, V4, DUAL>(t, n, keys, out, found, sc, s, tm);
  }
}

template <bool V4, bool DUAL>
hipError_t assign_d(const TableView& t, uint64_t n, const uint64_t* keys, const float* v,
                    const uint64_t* sc, hipStream_t s, KernelTimer* tm) {
  switch (lanes_for(t)) {
    case 4: return assign_g<4, V4, DUAL>(t, n, keys, v, sc, s, tm);
    case 8: return assign_g<8, V4, DUAL>(t, n, keys, v, sc, s, tm);
    default: return assign_g<16, V4, DUAL>(t, n, keys, v, sc, s, tm);
  }
}

template <bool V4, bool DUAL, bool FETCH>
hipError_t probe_d(const TableView& t, uint64_t n, const InsertCall& c, uint32_t* next, uint32_t* target,
                   bool link, hipStream_t s, KernelTimer* tm) {
  switch (lanes_for(t)) {
    case 4: return probe_g<4, V4, DUAL, FETCH>(t, n, c, next, target, link, s, tm);
    case 8: return probe_g<8, V4, DUAL, FETCH>(t, n, c, next, target, link, s, tm);
    default: return probe_g<16, V4, DUAL, FETCH>(t, n, c, next, target, link, s, tm);
  }
}

// Parallel: the probe kernel (updates of resident keys, chains of the
// others), then the owner kernel. Serial: insert_or_assign runs the serial
// kernel alone in input order; find_or_insert and insert_and_evict first run
// the probe kernel without chains (updates / stored rows of resident keys,
// marks of the others), then the serial kernel over the marked keys.
template <bool V4, bool DUAL>
hipError_t upsert_d(const TableView& t, uint64_t n, const InsertCall& c, uint32_t* next, uint32_t* target,
                    bool serial, hipStream_t s, KernelTimer* tm) {
  hipError_t e = hipSuccess;
  if (c.ev_count && (serial || n == 0)) {
    // (the parallel path's last compaction block writes the count itself)
    HKV_LAUNCH(tm, "zero", zero_u64_kernel, dim3(1), dim3(1), s, c.ev_count);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (n == 0) return hipSuccess;
  const bool two_phase = c.fetch || c.ev_keys;
  if (!serial || two_phase) {
    e = c.fetch ? probe_d<V4, DUAL, true>(t, n, c, next, target, !serial, s, tm)
                : probe_d<V4, DUAL, false>(t, n, c, next, target, !serial, s, tm);
    if (e != hipSuccess) return e;
  }
  if (serial) {
    const Evicted ev{c.ev_keys, c.ev_values, c.ev_scores, c.ev_count};
    HKV_LAUNCH(tm, "upsert_serial", (upsert_serial_kernel<V4, DUAL>), dim3(1), dim3(64), s, t, n, c.keys,
               c.values, c.scores, two_phase ? next : nullptr, two_phase ? target : nullptr, ev);
    return hipGetLastError();
  }
  return c.stat_slots ? owner_l<V4, DUAL, true>(t, n, c, next, target, s, tm)
                      : owner_l<V4, DUAL, false>(t, n, c, next, target, s, tm);
}

template <int G, bool DUAL>
hipError_t locate_g(const TableView& t, uint64_t n, const uint64_t* keys, uint64_t* ptrs, uint8_t* found,
                    uint64_t* sc, hipStream_t s, KernelTimer* tm) {
  const char* name = ptrs ? "find_ptr" : "contains";
  switch (t.keys_per_group) {
    case 1:
      HKV_LAUNCH(tm, name, (locate_kernel<G, DUAL, 1>), dim3(grid_for(n * G)), dim3(kBlock), s, t, n, keys, ptrs,
                 found, sc);
      break;
    case 4:
      HKV_LAUNCH(tm, name, (locate_kernel<G, DUAL, 4>), dim3(grid_for((n + 3) / 4 * G)), dim3(kBlock), s, t, n,
                 keys, ptrs, found, sc);
      break;
    default:
      HKV_LAUNCH(tm, name, (locate_kernel<G, DUAL, 2>), dim3(grid_for((n + 1) / 2 * G)), dim3(kBlock), s, t, n,
                 keys, ptrs, found, sc);
  }
  return hipGetLastError();
}

// Scratch of hkv_insert_or_assign_noalloc: the inserter's per-key chain and
// target words (next[0..max), target[max..2*max)) for calls that may not
// allocate. Each GPU the library runs on holds its own copy until the process
// ends; host code reaches it only through the address hipGetSymbolAddress
// returns for the current device (scratch_address below).
constexpr uint64_t kNoallocMaxKeys = 1ull << 21;
__device__ __align__(256) uint32_t scratch[2 * kNoallocMaxKeys];

}  // namespace

hipError_t scratch_address(uint32_t** out) {
  return hipGetSymbolAddress(reinterpret_cast<void**>(out), HIP_SYMBOL(scratch));
}

uint64_t noalloc_max_keys() { return kNoallocMaxKeys; }

hipError_t launch_init(const TableView& t, hipStream_t s) {
  const uint64_t cap = t.nb * kSlots;
  uint64_t blocks = (cap + kBlock - 1) / kBlock;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(init_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kBlock), 0, s, t);
  return hipGetLastError();
}

hipError_t launch_reset_heads(const TableView& t, hipStream_t s) {
  uint64_t blocks = (t.nb + kBlock - 1) / kBlock;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(reset_heads_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kBlock), 0, s, t);
  return hipGetLastError();
}

hipError_t launch_find(const TableView& t, uint64_t n, const uint64_t* keys, float* values_out,
                       uint8_t* found_out, uint64_t* scores_out, bool vec4, hipStream_t s,
                       KernelTimer* tm) {
  if (t.dual)
    return vec4 ? find_d<true, true>(t, n, keys, values_out, found_out, scores_out, s, tm)
                : find_d<false, true>(t, n, keys, values_out, found_out, scores_out, s, tm);
  return vec4 ? find_d<true, false>(t, n, keys, values_out, found_out, scores_out, s, tm)
              : find_d<false, false>(t, n, keys, values_out, found_out, scores_out, s, tm);
}

hipError_t launch_assign(const TableView& t, uint64_t n, const uint64_t* keys, const float* values,
                         const uint64_t* scores, bool vec4, hipStream_t s, KernelTimer* tm) {
  if (t.dual)
    return vec4 ? assign_d<true, true>(t, n, keys, values, scores, s, tm)
                : assign_d<false, true>(t, n, keys, values, scores, s, tm);
  return vec4 ? assign_d<true, false>(t, n, keys, values, scores, s, tm)
              : assign_d<false, false>(t, n, keys, values, scores, s, tm);
}

hipError_t launch_upsert(const TableView& t, uint64_t n, const InsertCall& c, uint32_t* next,
                         uint32_t* target, bool vec4, bool serial, hipStream_t s, KernelTimer* tm) {
  if (t.dual)
    return vec4 ? upsert_d<true, true>(t, n, c, next, target, serial, s, tm)
                : upsert_d<false, true>(t, n, c, next, target, serial, s, tm);
  return vec4 ? upsert_d<true, false>(t, n, c, next, target, serial, s, tm)
              : upsert_d<false, false>(t, n, c, next, target, serial, s, tm);
}

// Key-side probes need no row copy, so the group size does not follow dim:
// 8 lanes (one 16-byte digest load per line each) unless overridden.
hipError_t launch_locate(const TableView& t, uint64_t n, const uint64_t* keys, uint64_t* ptrs_out,
                         uint8_t* found_out, uint64_t* scores_out, hipStream_t s, KernelTimer* tm) {
  const int g = (t.lanes == 4 || t.lanes == 16) ? static_cast<int>(t.lanes) : 8;
  if (t.dual) {
    return g == 16 ? locate_g<16, true>(t, n, keys, ptrs_out, found_out, scores_out, s, tm)
                   : locate_g<8, true>(t, n, keys, ptrs_out, found_out, scores_out, s, tm);
  }
  switch (g) {
    case 4: return locate_g<4, false>(t, n, keys, ptrs_out, found_out, scores_out, s, tm);
    case 16: return locate_g<16, false>(t, n, keys, ptrs_out, found_out, scores_out, s, tm);
    default: return locate_g<8, false>(t, n, keys, ptrs_out, found_out, scores_out, s, tm);
  }
}

hipError_t launch_size(const TableView& t, unsigned long long* dev_out, hipStream_t s, KernelTimer* tm) {
  HKV_LAUNCH(tm, "zero", zero_u64_kernel, dim3(1), dim3(1), s, dev_out);
  // few blocks: each adds its partial sum to the one counter, and such adds
  // serialize (~12 ns each), so 128 blocks of 256 threads read the words
  uint64_t blocks = (t.nb + kBlock - 1) / kBlock;
  if (blocks > 128) blocks = 128;
  if (blocks == 0) blocks = 1;
  HKV_LAUNCH(tm, "size", size_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kBlock), s, t.occ, t.nb,
             dev_out);
  return hipGetLastError();
}

hipError_t launch_export(const TableView& t, uint64_t begin, uint64_t end, uint64_t* keys_out,
                         float* values_out, uint64_t* scores_out, uint64_t* pos_out,
                         unsigned long long* count_out, bool vec4, hipStream_t s, KernelTimer* tm) {
  HKV_LAUNCH(tm, "zero", zero_u64_kernel, dim3(1), dim3(1), s, count_out);
  if (end > begin) {
    const uint64_t buckets = (end + kSlots - 1) / kSlots - begin / kSlots;
    const dim3 grid(static_cast<uint32_t>((buckets + kExportBuckets - 1) / kExportBuckets));
    if (vec4)
      HKV_LAUNCH(tm, "export", export_kernel<true>, grid, dim3(kBlock), s, t, begin, end, keys_out, values_out,
                 scores_out, pos_out, count_out);
    else
      HKV_LAUNCH(tm, "export", export_kernel<false>, grid, dim3(kBlock), s, t, begin, end, keys_out, values_out,
                 scores_out, pos_out, count_out);
  }
  return hipGetLastError();
}

}  // namespace hkv
