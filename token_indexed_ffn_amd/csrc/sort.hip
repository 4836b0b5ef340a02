// Batch dedup and cache ranking on the GPU.
//
// Both are a sort of 64-bit keys whose low 32 bits make every key unique
// (a position, or a token ID), followed by a scan.  Keys are sorted with a
// bitonic network: a tile of up to kTile keys is sorted in LDS by one
// workgroup; longer arrays add global compare-exchange steps for the strides
// of at least kTile and LDS merges for the smaller strides.  Because every key
// is unique, the order is total, so the result is the stable order of the
// high 32 bits and no atomic decides any output.
//
// Dedup (STAPLE retrieval-path table, Prefill row: dedup once, one inverse
// token map for every layer): key = (id << 32) | position.  After the sort,
// a single-workgroup scan marks the first key of each ID run and writes the
// unique IDs, segment offsets, sorted positions and the inverse map.  A
// decode batch (at most 64 positions) is sorted and scanned by one wave in
// registers.
//
// Cache ranking (AI Radio episode on STAPLE: frequency-aware cache of about 5%
// of the vocabulary): key = ((2^31-1 - count) << 32) | id, so ascending key
// order is count descending, then ID ascending.
#include "common.h"

namespace staple {

constexpr int kSortThreads = 1024;
constexpr int kTile = 4096;            // keys per LDS tile (4 per thread)
constexpr uint64_t kPadKey = ~0ull;

__device__ __forceinline__ void cmp_swap(uint64_t& a, uint64_t& b, bool ascending) {
  const bool gt = a > b;
  if (gt == ascending) {
    const uint64_t t = a;
    a = b;
    b = t;
  }
}

// Bitonic stages (k, j) with j < tile size, on keys held in LDS.  `gbase` is
// the global index of s[0]; directions follow the global index.
__device__ void lds_bitonic(uint64_t* s, int n, int64_t gbase, int64_t k_from, int64_t k_to,
                            bool merge_only) {
  for (int64_t k = k_from; k <= k_to; k <<= 1) {
    const int64_t j0 = merge_only ? (n >> 1) : (k >> 1);
    for (int64_t j = j0; j >= 1; j >>= 1) {
      for (int p = threadIdx.x; p < (n >> 1); p += blockDim.x) {
        const int i = static_cast<int>((p / j) * 2 * j + (p % j));
        const int l = i + static_cast<int>(j);
        const bool asc = ((gbase + i) & k) == 0;
        uint64_t a = s[i], b = s[l];
        cmp_swap(a, b, asc);
        s[i] = a;
        s[l] = b;
      }
      __syncthreads();
    }
    if (merge_only) break;
  }
}

// Block-wide exclusive scan of one int per thread (blockDim.x a multiple of 64,
// at most 1024).  `total` receives the block sum.  `wave_tmp` is LDS of >= 16 ints.
__device__ int block_exclusive_scan(int v, int* wave_tmp, int& total) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wave_tmp[wid] = x;
  __syncthreads();
  if (wid == 0) {
    int w = lane < nw ? wave_tmp[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int y = __shfl_up(w, o, 64);
      if (lane >= o) w += y;
    }
    if (lane < nw) wave_tmp[lane] = w;
  }
  __syncthreads();
  const int before = wid > 0 ? wave_tmp[wid - 1] : 0;
  total = wave_tmp[nw - 1];
  __syncthreads();
  return before + x - v;
}

// ---------------------------------------------------------------------------
// Key generation
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t dedup_key(const int32_t* ids, int64_t i, int64_t n,
                                              int64_t vocab, int* err) {
  if (i >= n) return kPadKey;
  const int32_t t = ids[i];
  if (t < 0 || t >= vocab) flag_index_error(err);
  return (static_cast<uint64_t>(static_cast<uint32_t>(t)) << 32) | static_cast<uint64_t>(i);
}

__global__ void dedup_keys_kernel(const int32_t* ids, int64_t n, int64_t vocab, int64_t padded,
                                  uint64_t* keys, int* err) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < padded) keys[i] = dedup_key(ids, i, n, vocab, err);
}

__global__ void cache_keys_kernel(const int64_t* counts, int64_t vocab, int64_t padded,
                                  uint64_t* keys, int* err) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= padded) return;
  if (i >= vocab) {
    keys[i] = kPadKey;
    return;
  }
  int64_t c = counts[i];
  if (c < 0 || c > 0x7fffffffll) {
    flag_index_error(err);
    c = c < 0 ? 0 : 0x7fffffffll;
  }
  keys[i] = (static_cast<uint64_t>(0x7fffffffll - c) << 32) | static_cast<uint64_t>(i);
}

// ---------------------------------------------------------------------------
// Sort kernels over a padded power-of-two array in global memory
// ---------------------------------------------------------------------------
// Sorts each kTile-long tile completely (all stages k <= kTile).
__global__ __launch_bounds__(kSortThreads) void tile_sort_kernel(uint64_t* keys, int64_t padded) {
  __shared__ uint64_t s[kTile];
  const int n = static_cast<int>(padded < kTile ? padded : kTile);
  const int64_t base = static_cast<int64_t>(blockIdx.x) * n;
  for (int i = threadIdx.x; i < n; i += blockDim.x) s[i] = keys[base + i];
  __syncthreads();
  lds_bitonic(s, n, base, 2, n, false);
  for (int i = threadIdx.x; i < n; i += blockDim.x) keys[base + i] = s[i];
}

// One global compare-exchange stage (k, j) with j >= kTile.
__global__ void global_step_kernel(uint64_t* keys, int64_t padded, int64_t k, int64_t j) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (p >= (padded >> 1)) return;
  const int64_t i = (p / j) * 2 * j + (p % j);
  const int64_t l = i + j;
  uint64_t a = keys[i], b = keys[l];
  cmp_swap(a, b, (i & k) == 0);
  keys[i] = a;
  keys[l] = b;
}

// The stages j = kTile/2 .. 1 of merge step k, per tile in LDS.
__global__ __launch_bounds__(kSortThreads) void tile_merge_kernel(uint64_t* keys, int64_t k) {
  __shared__ uint64_t s[kTile];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kTile;
  for (int i = threadIdx.x; i < kTile; i += blockDim.x) s[i] = keys[base + i];
  __syncthreads();
  lds_bitonic(s, kTile, base, k, k, true);
  for (int i = threadIdx.x; i < kTile; i += blockDim.x) keys[base + i] = s[i];
}

static int64_t next_pow2(int64_t v) {
  int64_t p = 1;
  while (p < v) p <<= 1;
  return p;
}

// Sorts `padded` (a power of two, >= 2) keys in place.
static hipError_t sort_keys(uint64_t* keys, int64_t padded, hipStream_t s) {
  const int64_t tiles = padded <= kTile ? 1 : padded / kTile;
  tile_sort_kernel<<<dim3(static_cast<unsigned>(tiles)), dim3(kSortThreads), 0, s>>>(keys, padded);
  for (int64_t k = 2 * kTile; k <= padded; k <<= 1) {
    for (int64_t j = k >> 1; j >= kTile; j >>= 1) {
      const int64_t pairs = padded >> 1;
      global_step_kernel<<<dim3(static_cast<unsigned>((pairs + 255) / 256)), dim3(256), 0, s>>>(
          keys, padded, k, j);
    }
    tile_merge_kernel<<<dim3(static_cast<unsigned>(tiles)), dim3(kSortThreads), 0, s>>>(keys, k);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dedup outputs from sorted keys
// ---------------------------------------------------------------------------
// Emits uniq/seg_start/sorted_pos/inv for keys [0, n) read through `key_at`.
template <typename KeyAt>
__device__ void dedup_emit(KeyAt key_at, int64_t n, int32_t* uniq, int32_t* inv,
                           int32_t* sorted_pos, int32_t* seg_start, int32_t* n_unique,
                           int* wave_tmp) {
  constexpr int kItems = 4;
  int carry = 0;  // number of segments started before this chunk
  const int64_t chunk = static_cast<int64_t>(blockDim.x) * kItems;
  for (int64_t base = 0; base < n; base += chunk) {
    const int64_t p0 = base + static_cast<int64_t>(threadIdx.x) * kItems;
    uint64_t key[kItems];
    int flag[kItems];
    int local = 0;
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      const int64_t p = p0 + it;
      key[it] = p < n ? key_at(p) : kPadKey;
      const uint32_t id = static_cast<uint32_t>(key[it] >> 32);
      flag[it] = 0;
      if (p < n) flag[it] = (p == 0) || (static_cast<uint32_t>(key_at(p - 1) >> 32) != id);
      local += flag[it];
    }
    int total;
    const int before = block_exclusive_scan(local, wave_tmp, total);
    int seg = carry + before - 1;  // index of the segment holding the previous item
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      const int64_t p = p0 + it;
      if (p < n) {
        seg += flag[it];
        const int32_t id = static_cast<int32_t>(key[it] >> 32);
        const int32_t pos = static_cast<int32_t>(key[it] & 0xffffffffu);
        if (flag[it]) {
          uniq[seg] = id;
          seg_start[seg] = static_cast<int32_t>(p);
        }
        sorted_pos[p] = pos;
        inv[pos] = seg;
      }
    }
    carry += total;
  }
  if (threadIdx.x == 0) {
    *n_unique = carry;
    seg_start[carry] = static_cast<int32_t>(n);
  }
}

__global__ __launch_bounds__(kSortThreads) void dedup_emit_kernel(
    const uint64_t* keys, int64_t n, int32_t* uniq, int32_t* inv, int32_t* sorted_pos,
    int32_t* seg_start, int32_t* n_unique) {
  __shared__ int wave_tmp[16];
  dedup_emit([&](int64_t p) { return keys[p]; }, n, uniq, inv, sorted_pos, seg_start, n_unique,
             wave_tmp);
}

// Whole dedup of at most kTile positions in one workgroup.
__global__ __launch_bounds__(kSortThreads) void dedup_small_kernel(
    const int32_t* ids, int64_t n, int64_t padded, int64_t vocab, int32_t* uniq, int32_t* inv,
    int32_t* sorted_pos, int32_t* seg_start, int32_t* n_unique, int* err) {
  __shared__ uint64_t s[kTile];
  __shared__ int wave_tmp[16];
  const int np = static_cast<int>(padded);
  for (int i = threadIdx.x; i < np; i += blockDim.x) s[i] = dedup_key(ids, i, n, vocab, err);
  __syncthreads();
  if (np >= 2) lds_bitonic(s, np, 0, 2, np, false);
  dedup_emit([&](int64_t p) { return s[p]; }, n, uniq, inv, sorted_pos, seg_start, n_unique,
             wave_tmp);
}

// Whole dedup of at most 64 positions (a decode batch) in one wave: lane i
// holds key i, the bitonic network runs on registers with lane exchanges,
// and the segment starts come from a ballot, so there is no LDS and no
// barrier.  Same outputs as the workgroup kernels.
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  const uint32_t lo = static_cast<uint32_t>(__shfl_xor(static_cast<int>(v & 0xffffffffu), mask, 64));
  const uint32_t hi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(v >> 32), mask, 64));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__global__ __launch_bounds__(64) void dedup_wave_kernel(const int32_t* ids, int64_t n, int64_t vocab,
                                                        int32_t* uniq, int32_t* inv,
                                                        int32_t* sorted_pos, int32_t* seg_start,
                                                        int32_t* n_unique, int* err) {
  const int lane = threadIdx.x;
  uint64_t key = dedup_key(ids, lane, n, vocab, err);
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j >= 1; j >>= 1) {
      const uint64_t other = shfl_xor_u64(key, j);
      const bool asc = (lane & k) == 0;       // k = 64: the whole wave ascending
      const bool lower = (lane & j) == 0;
      key = (lower == asc) ? (key < other ? key : other) : (key < other ? other : key);
    }
  }
  const bool valid = lane < n;
  const int32_t id = static_cast<int32_t>(key >> 32);
  const int32_t prev = __shfl_up(id, 1, 64);
  const bool first = valid && (lane == 0 || prev != id);
  const uint64_t starts = __ballot(first);
  const int seg = __popcll(starts & ((2ull << lane) - 1)) - 1;   // segment of this position
  if (valid) {
    const int32_t pos = static_cast<int32_t>(key & 0xffffffffu);
    if (first) {
      uniq[seg] = id;
      seg_start[seg] = lane;
    }
    sorted_pos[lane] = pos;
    inv[pos] = seg;
  }
  if (lane == 0) {
    const int total = __popcll(starts);
    *n_unique = total;
    seg_start[total] = static_cast<int32_t>(n);
  }
}

// Dedup and cache probe of a decode batch (at most 64 tokens) in one wave:
// the one-wave dedup above, then every unique ID's cache slot (code[u] = slot
// on a hit, -1 - m on the m-th miss in ascending u), the miss list and, with
// row_src, each token's row source (its slot, or -1 - id for a row of the
// table; INT32_MIN for an ID outside the table).  The same outputs as
// staple_dedup followed by staple_cache_lookup, in one launch.
__global__ __launch_bounds__(64) void dedup_lookup_wave_kernel(
    const int32_t* ids, int64_t n, int64_t vocab, const int32_t* id_to_slot, int32_t* uniq,
    int32_t* inv, int32_t* sorted_pos, int32_t* seg_start, int32_t* n_unique, int32_t* code,
    int32_t* miss_uidx, int32_t* n_miss, int32_t* row_src, int* err) {
  const int lane = threadIdx.x;
  uint64_t key = dedup_key(ids, lane, n, vocab, err);
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j >= 1; j >>= 1) {
      const uint64_t other = shfl_xor_u64(key, j);
      const bool asc = (lane & k) == 0;
      const bool lower = (lane & j) == 0;
      key = (lower == asc) ? (key < other ? key : other) : (key < other ? other : key);
    }
  }
  const bool valid = lane < n;
  const int32_t id = static_cast<int32_t>(key >> 32);
  const int32_t prev = __shfl_up(id, 1, 64);
  const bool first = valid && (lane == 0 || prev != id);
  const uint64_t starts = __ballot(first);
  const int seg = __popcll(starts & ((2ull << lane) - 1)) - 1;
  const bool in_table = id >= 0 && id < vocab;
  const int32_t slot = valid && in_table ? id_to_slot[id] : -1;
  const bool miss = first && slot < 0;
  const uint64_t misses = __ballot(miss);
  if (valid) {
    const int32_t pos = static_cast<int32_t>(key & 0xffffffffu);
    if (first) {
      uniq[seg] = id;
      seg_start[seg] = lane;
      if (miss) {
        const int m = __popcll(misses & ((1ull << lane) - 1));
        code[seg] = -1 - m;
        miss_uidx[m] = seg;
      } else {
        code[seg] = slot;
      }
    }
    sorted_pos[lane] = pos;
    inv[pos] = seg;
    if (row_src) row_src[pos] = in_table ? (slot >= 0 ? slot : -1 - id) : INT32_MIN;
  }
  if (lane == 0) {
    const int total = __popcll(starts);
    *n_unique = total;
    seg_start[total] = static_cast<int32_t>(n);
    *n_miss = __popcll(misses);
  }
}

hipError_t launch_dedup_lookup_wave(const int32_t* ids, int64_t n, int64_t vocab,
                                    const int32_t* id_to_slot, int32_t* uniq, int32_t* inv,
                                    int32_t* sorted_pos, int32_t* seg_start, int32_t* n_unique,
                                    int32_t* code, int32_t* miss_uidx, int32_t* n_miss,
                                    int32_t* row_src, hipStream_t s, int* err) {
  if (n < 1 || n > 64) return hipErrorInvalidValue;
  dedup_lookup_wave_kernel<<<dim3(1), dim3(64), 0, s>>>(ids, n, vocab, id_to_slot, uniq, inv,
                                                        sorted_pos, seg_start, n_unique, code,
                                                        miss_uidx, n_miss, row_src, err);
  return hipGetLastError();
}

size_t dedup_workspace_bytes(int64_t n) {
  if (n <= kTile) return 0;
  return static_cast<size_t>(next_pow2(n)) * sizeof(uint64_t);
}

hipError_t launch_dedup(const int32_t* ids, int64_t n, int64_t vocab, int32_t* uniq, int32_t* inv,
                        int32_t* sorted_pos, int32_t* seg_start, int32_t* n_unique, void* ws,
                        hipStream_t s, int* err) {
  if (n <= 64) {
    dedup_wave_kernel<<<dim3(1), dim3(64), 0, s>>>(ids, n, vocab, uniq, inv, sorted_pos, seg_start,
                                                   n_unique, err);
    return hipGetLastError();
  }
  if (n <= kTile) {
    const int64_t padded = n <= 1 ? 1 : next_pow2(n);
    dedup_small_kernel<<<dim3(1), dim3(kSortThreads), 0, s>>>(ids, n, padded, vocab, uniq, inv,
                                                               sorted_pos, seg_start, n_unique, err);
    return hipGetLastError();
  }
  const int64_t padded = next_pow2(n);
  uint64_t* keys = static_cast<uint64_t*>(ws);
  dedup_keys_kernel<<<dim3(static_cast<unsigned>((padded + 255) / 256)), dim3(256), 0, s>>>(
      ids, n, vocab, padded, keys, err);
  hipError_t e = sort_keys(keys, padded, s);
  if (e != hipSuccess) return e;
  dedup_emit_kernel<<<dim3(1), dim3(kSortThreads), 0, s>>>(keys, n, uniq, inv, sorted_pos,
                                                            seg_start, n_unique);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Cache build
// ---------------------------------------------------------------------------
__global__ void cache_assign_kernel(const uint64_t* keys, int64_t vocab, int64_t capacity,
                                    int32_t* id_to_slot, int32_t* slot_to_id) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= vocab) return;
  const int32_t id = static_cast<int32_t>(keys[i] & 0xffffffffu);
  // every ID appears exactly once in the sorted keys, so each id_to_slot entry
  // is written exactly once
  if (i < capacity) {
    slot_to_id[i] = id;
    id_to_slot[id] = static_cast<int32_t>(i);
  } else {
    id_to_slot[id] = -1;
  }
}

size_t cache_build_workspace_bytes(int64_t vocab) {
  return static_cast<size_t>(next_pow2(vocab < 2 ? 2 : vocab)) * sizeof(uint64_t);
}

hipError_t launch_cache_build(const int64_t* counts, int64_t vocab, int64_t capacity,
                              int32_t* id_to_slot, int32_t* slot_to_id, void* ws, hipStream_t s,
                              int* err) {
  const int64_t padded = next_pow2(vocab < 2 ? 2 : vocab);
  uint64_t* keys = static_cast<uint64_t*>(ws);
  cache_keys_kernel<<<dim3(static_cast<unsigned>((padded + 255) / 256)), dim3(256), 0, s>>>(
      counts, vocab, padded, keys, err);
  hipError_t e = sort_keys(keys, padded, s);
  if (e != hipSuccess) return e;
  cache_assign_kernel<<<dim3(static_cast<unsigned>((vocab + 255) / 256)), dim3(256), 0, s>>>(
      keys, vocab, capacity, id_to_slot, slot_to_id);
  return hipGetLastError();
}

}  // namespace staple
