// Access-pattern ceilings of find and of insert_or_assign's first kernel on
// this GPU: kernels that make exactly their memory accesses on a full
// single-bucket table of 2^26 slots with rows of `dim` floats (argument 1:
// 32, 64 or 128; default 64), with none of the hashing, digest matching or
// ballots. For find, per key (8 lanes): the 8-byte key (sequential), a
// 128-byte digest line (random in 64 MiB), one 8-byte candidate key (random
// in 512 MiB), for 90 % of keys a 4*dim-byte row (random) written out
// (sequential) and a found byte. Cache policies as in the kernels: digest
// lines and keys cacheable, rows nontemporal.
// Run twice: with every address depending on the value the previous load
// returned (find's chain: key -> line -> candidate -> row) and with all
// addresses computed from the key index. A benchmark tool, built by
// bench.build_pattern_ceiling(); it does not use the table.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

#define CK(x)                                                                    \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                                  \
    }                                                                            \
  } while (0)

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint64_t mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

// A comparison the compiler cannot fold, so the next address waits for the load.
__device__ __forceinline__ uint64_t after(uint64_t v) { return v == 0xDEADBEEFull ? 1ull : 0ull; }

// R: 16-byte pieces of a row per lane (dim / 32).
template <bool CHAIN, int R>
__global__ __launch_bounds__(256) void pattern_kernel(const uint64_t* __restrict__ keys,
                                                      const uint8_t* __restrict__ lines,
                                                      const uint64_t* __restrict__ cand,
                                                      const float* __restrict__ rows, float* __restrict__ out,
                                                      uint8_t* __restrict__ found, uint32_t n, uint64_t nlines,
                                                      uint64_t ncand, uint64_t nrows) {
  const uint32_t i = (blockIdx.x * 256u + threadIdx.x) / 8;
  const int lane = static_cast<int>(threadIdx.x & 7);
  if (i >= n) return;
  const uint64_t k = keys[i];
  const uint64_t h = mix(CHAIN ? k + i : i);
  const uint4 w = *reinterpret_cast<const uint4*>(lines + (h & (nlines - 1)) * 128 + lane * 16);
  const int owner = static_cast<int>((h >> 40) & 7);
  uint64_t c = 0;
  const uint32_t wl = w.x ^ w.y ^ w.z ^ w.w;  // the whole line is used
  if (lane == owner) c = cand[mix(h + (CHAIN ? after(wl) : 0)) & (ncand - 1)];
  c = __shfl(c, owner, 8);
  // without the chain, the line and candidate values only feed the flag
  const uint8_t sink = (!CHAIN && (k == 0xDEADBEEFull || wl == 0xDEADBEEFu || c == 0xDEADBEEFull)) ? 2 : 0;
  if (mix(i) % 10 == 0) {
    if (lane == 0) found[i] = sink;
    return;
  }
  const uint64_t r = mix(h + 7 + (CHAIN ? after(c) : 0)) & (nrows - 1);
  const f32x4* s4 = reinterpret_cast<const f32x4*>(rows + r * (32 * R));
  f32x4 v[R];
#pragma unroll
  for (int q = 0; q < R; ++q) v[q] = __builtin_nontemporal_load(s4 + lane + 8 * q);
  f32x4* d4 = reinterpret_cast<f32x4*>(out + static_cast<uint64_t>(i) * (32 * R));
#pragma unroll
  for (int q = 0; q < R; ++q) __builtin_nontemporal_store(v[q], d4 + lane + 8 * q);
  if (lane == 0) found[i] = 1 | sink;
}

// insert_or_assign's first kernel on the same table with 90 % resident keys:
// the same chain key -> line -> candidate, then for a resident key a 4*dim-byte
// input row (sequential, independent of the chain) written to a random row
// and an 8-byte score write next to the candidate's slot; for a missing key an
// atomic exchange on a random 4-byte chain head; 8 bytes of chain words
// (sequential) for every key.
template <int R>
__global__ __launch_bounds__(256) void upsert_pattern_kernel(const uint64_t* __restrict__ keys,
                                                             const uint8_t* __restrict__ lines,
                                                             const uint64_t* __restrict__ cand,
                                                             uint64_t* __restrict__ scores, float* __restrict__ rows,
                                                             const float* __restrict__ in_rows,
                                                             const uint64_t* __restrict__ in_scores,
                                                             uint32_t* __restrict__ heads, uint32_t* __restrict__ next,
                                                             uint32_t* __restrict__ target, uint32_t n, uint64_t nlines,
                                                             uint64_t ncand, uint64_t nrows) {
  const uint32_t i = (blockIdx.x * 256u + threadIdx.x) / 8;
  const int lane = static_cast<int>(threadIdx.x & 7);
  if (i >= n) return;
  const uint64_t k = keys[i];
  const uint64_t h = mix(k + i);
  const uint4 w = *reinterpret_cast<const uint4*>(lines + (h & (nlines - 1)) * 128 + lane * 16);
  const int owner = static_cast<int>((h >> 40) & 7);
  const uint64_t slot = mix(h + after(w.x ^ w.y ^ w.z ^ w.w)) & (ncand - 1);
  uint64_t c = 0;
  if (lane == owner) c = cand[slot];
  c = __shfl(c, owner, 8);
  if (mix(i) % 10 == 0) {
    if (lane == 0) {
      target[i] = static_cast<uint32_t>(slot >> 7);
      next[i] = __hip_atomic_exchange(heads + (slot >> 7), i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  const uint64_t r = (slot + after(c)) & (nrows - 1);
  const f32x4* s4 = reinterpret_cast<const f32x4*>(in_rows + static_cast<uint64_t>(i) * (32 * R));
  f32x4 v[R];
#pragma unroll
  for (int q = 0; q < R; ++q) v[q] = __builtin_nontemporal_load(s4 + lane + 8 * q);
  f32x4* d4 = reinterpret_cast<f32x4*>(rows + r * (32 * R));
#pragma unroll
  for (int q = 0; q < R; ++q) __builtin_nontemporal_store(v[q], d4 + lane + 8 * q);
  if (lane == 0) {
    scores[slot] = in_scores[i];
    next[i] = 0xFFFFFFFEu;
  }
}

__global__ void fill_keys(uint64_t* keys, uint32_t n) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i < n) keys[i] = mix(0x9E3779B97F4A7C15ull + i);
}

template <int R>
int run() {
  const uint64_t dim = 32 * R;
  const uint64_t nlines = 1ull << 19, ncand = 1ull << 26, nrows = 1ull << 26;
  const uint32_t n = 1u << 20;
  uint64_t *keys = nullptr, *cand = nullptr;
  uint8_t *lines = nullptr, *found = nullptr;
  float *rows = nullptr, *out = nullptr;
  CK(hipMalloc(&keys, n * 8ull));
  CK(hipMalloc(&cand, ncand * 8));
  CK(hipMalloc(&lines, nlines * 128));
  CK(hipMalloc(&rows, nrows * dim * 4));
  CK(hipMalloc(&out, n * dim * 4));
  CK(hipMalloc(&found, n));
  CK(hipMemset(cand, 0, ncand * 8));
  CK(hipMemset(lines, 0, nlines * 128));
  CK(hipMemset(rows, 0, nrows * dim * 4));
  hipLaunchKernelGGL(fill_keys, dim3(n / 256), dim3(256), 0, 0, keys, n);
  CK(hipGetLastError());
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  const double bytes = n * (8 + 128 + 4 + 0.9 * (8 + 8.0 * dim) + 1.0);  // find's algorithmic bytes, h = 0.9
  const dim3 grid(n * 8 / 256), block(256);
  std::printf("{\"dim\": %d, ", static_cast<int>(dim));
  for (int chain = 1; chain >= 0; --chain) {
    for (int w = 0; w < 3; ++w) {
      if (chain) hipLaunchKernelGGL((pattern_kernel<true, R>), grid, block, 0, 0, keys, lines, cand, rows, out, found, n, nlines, ncand, nrows);
      else hipLaunchKernelGGL((pattern_kernel<false, R>), grid, block, 0, 0, keys, lines, cand, rows, out, found, n, nlines, ncand, nrows);
    }
    CK(hipEventRecord(e0));
    const int reps = 20;
    for (int r = 0; r < reps; ++r) {
      if (chain) hipLaunchKernelGGL((pattern_kernel<true, R>), grid, block, 0, 0, keys, lines, cand, rows, out, found, n, nlines, ncand, nrows);
      else hipLaunchKernelGGL((pattern_kernel<false, R>), grid, block, 0, 0, keys, lines, cand, rows, out, found, n, nlines, ncand, nrows);
    }
    CK(hipEventRecord(e1));
    CK(hipEventSynchronize(e1));
    float ms = 0.f;
    CK(hipEventElapsedTime(&ms, e0, e1));
    const double us = ms * 1000.0 / reps;
    std::printf("\"%s\": {\"us_per_2p20_keys\": %.2f, \"algorithmic_GBps\": %.1f}%s", chain ? "dependent_chain" : "independent",
                us, bytes / (us * 1e-6) / 1e9, chain ? ", " : "");
  }
  // the upsert pattern: 8 key + 128 line + 4 false-positive keys
  // + 0.9 (8 key + 4*dim row in + 8 score in + 4*dim row + 8 score) + 0.1 * 8
  uint64_t *scores = nullptr, *in_scores = nullptr;
  uint32_t *heads = nullptr, *next = nullptr, *target = nullptr;
  float* in_rows = out;  // n rows, read sequentially
  CK(hipMalloc(&scores, ncand * 8));
  CK(hipMalloc(&in_scores, n * 8ull));
  CK(hipMalloc(&heads, (ncand / 128) * 4));
  CK(hipMalloc(&next, n * 4ull));
  CK(hipMalloc(&target, n * 4ull));
  CK(hipMemset(scores, 0, ncand * 8));
  CK(hipMemset(in_scores, 0, n * 8ull));
  CK(hipMemset(heads, 0xFF, (ncand / 128) * 4));
  const double ubytes = n * (8 + 128 + 4 + 0.9 * (8 + 8.0 * dim + 16) + 0.1 * 8);
  for (int w = 0; w < 3; ++w)
    hipLaunchKernelGGL(upsert_pattern_kernel<R>, grid, block, 0, 0, keys, lines, cand, scores, rows, in_rows, in_scores,
                       heads, next, target, n, nlines, ncand, nrows);
  CK(hipEventRecord(e0));
  const int ureps = 20;
  for (int r = 0; r < ureps; ++r)
    hipLaunchKernelGGL(upsert_pattern_kernel<R>, grid, block, 0, 0, keys, lines, cand, scores, rows, in_rows, in_scores,
                       heads, next, target, n, nlines, ncand, nrows);
  CK(hipEventRecord(e1));
  CK(hipEventSynchronize(e1));
  float ums = 0.f;
  CK(hipEventElapsedTime(&ums, e0, e1));
  const double uus = ums * 1000.0 / ureps;
  std::printf(", \"upsert_probe_dependent_chain\": {\"us_per_2p20_keys\": %.2f, \"algorithmic_GBps\": %.1f}}\n", uus,
              ubytes / (uus * 1e-6) / 1e9);
  CK(hipGetLastError());
  return 0;
}

int main(int argc, char** argv) {
  const int dim = argc > 1 ? std::atoi(argv[1]) : 64;
  if (dim == 32) return run<1>();
  if (dim == 64) return run<2>();
  if (dim == 128) return run<4>();
  std::fprintf(stderr, "dim must be 32, 64 or 128\n");
  return 2;
}
