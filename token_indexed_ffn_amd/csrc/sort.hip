// Batch dedup and cache ranking on the GPU.
//
// Both are a stable LSD radix sort of (key, value) pairs followed by a scan.
// A pair travels as one 64-bit word, key in the high half and value in the
// low half; each pass orders the pairs stably by one digit of the key, from
// the least significant digit up, so after the last pass they are ordered by
// key and, for equal keys, by their order on input.  The result is unique, so
// no atomic decides any output.
//
// Dedup (STAPLE retrieval-path table, Prefill row: dedup once, one inverse
// token map for every layer): key = token ID, value = position, positions in
// ascending order on input, so the pairs end ordered by (ID, position).  The
// key has bit_length(vocab - 1) bits (17 at vocab 100352): three passes of
// 6-bit digits.  Then a scan marks the first position of each ID run and
// writes the unique IDs, segment offsets, sorted positions and inverse map.
//   * at most 64 positions (a decode batch): one wave, one key bit per pass,
//     each pass a split by two ballots and a lane permute; no LDS tables, no
//     barrier;
//   * at most 4096: one workgroup, the pairs in LDS;
//   * more: per pass one histogram launch (per-workgroup digit counts) and
//     one scatter launch (each workgroup derives its digit offsets from the
//     histograms, ranks its pairs stably and writes them), over at most 64
//     workgroups that each own a contiguous range; then a count launch and a
//     write launch for the scan, over the same ranges.
// Inside a workgroup a pass ranks 64 pairs at a time per wave: the lanes
// holding the same digit are found by one ballot per digit bit, a lane's rank
// is the wave's running count of its digit plus the number of such lanes
// below it, and the waves' counts are then turned into offsets in wave order.
//
// Cache ranking (AI Radio episode on STAPLE: frequency-aware cache of about 5%
// of the vocabulary): key = 2^31-1 - count, value = ID, IDs in ascending order
// on input, so ascending key order is count descending, then ID ascending.
#include "common.h"

namespace staple {

constexpr uint64_t kPadKey = ~0ull;
constexpr int kRadixWaves = 16;                              // waves per workgroup
constexpr int kRadixThreads = kRadixWaves * 64;
constexpr int kRadixSlots = 4;                               // 64-pair slots per wave per chunk
constexpr int kRadixChunk = kRadixWaves * kRadixSlots * 64;  // pairs per workgroup step: 4096
constexpr int kRadixDigitMax = 8;                            // widest digit
constexpr int kRadixBins = 1 << kRadixDigitMax;
constexpr int kRadixMaxBlocks = 64;                          // workgroups of one pass

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
// Pair sources
// ---------------------------------------------------------------------------
// Dedup input: (ID, position).  An ID outside [0, vocab) sets the error word.
struct DedupSource {
  const int32_t* ids;
  int64_t vocab;
  int* err;
  __device__ __forceinline__ uint64_t operator()(int64_t i) const {
    const int32_t t = ids[i];
    if (t < 0 || t >= vocab) flag_index_error(err);
    return (static_cast<uint64_t>(static_cast<uint32_t>(t)) << 32) | static_cast<uint64_t>(i);
  }
};

// Cache ranking input: (2^31-1 - count, ID); a count outside [0, 2^31-1]
// sets the error word and is clamped.
struct CacheSource {
  const int64_t* counts;
  int* err;
  __device__ __forceinline__ uint64_t operator()(int64_t i) const {
    int64_t c = counts[i];
    if (c < 0 || c > 0x7fffffffll) {
      flag_index_error(err);
      c = c < 0 ? 0 : 0x7fffffffll;
    }
    return (static_cast<uint64_t>(0x7fffffffll - c) << 32) | static_cast<uint64_t>(i);
  }
};

// The pairs of an earlier pass.
struct PairSource {
  const uint64_t* pairs;
  __device__ __forceinline__ uint64_t operator()(int64_t i) const { return pairs[i]; }
};

// ---------------------------------------------------------------------------
// One radix pass inside a workgroup
// ---------------------------------------------------------------------------
struct RadixLds {
  int cnt[kRadixWaves][kRadixBins];  // per-wave digit counts, then per-wave offsets
  int run[kRadixBins];               // the workgroup's next offset of each digit
  int wave_tmp[16];
};

__device__ __forceinline__ uint32_t radix_digit(uint64_t pair, int shift, int dbits) {
  return static_cast<uint32_t>(pair >> (32 + shift)) & ((1u << dbits) - 1u);
}

// The valid lanes of the wave whose digit equals this lane's.
__device__ __forceinline__ uint64_t radix_peers(uint32_t d, bool valid, int dbits) {
  uint64_t peers = __ballot(valid);
  for (int b = 0; b < dbits; ++b) {
    const bool bit = (d >> b) & 1u;
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

// Loads pairs [base, min(base + kRadixChunk, end)) (wave w owns the
// kRadixSlots x 64 pairs from base + 256 w, slot-major) and ranks each among
// the wave's pairs of the same digit, in order; L.cnt[w] ends holding the
// wave's digit counts.  Only wave w touches row w, and one wave's LDS
// accesses complete in program order, so the read-then-update of a count
// needs no barrier.
template <typename Load>
__device__ __forceinline__ void radix_rank_chunk(const Load& load, int64_t base, int64_t end,
                                                 int shift, int dbits, RadixLds& L,
                                                 uint64_t (&pair)[kRadixSlots],
                                                 int (&rank)[kRadixSlots]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = lane; i < (1 << dbits); i += 64) L.cnt[w][i] = 0;
  const uint64_t below = (1ull << lane) - 1;
#pragma unroll
  for (int s = 0; s < kRadixSlots; ++s) {
    const int64_t idx = base + (w * kRadixSlots + s) * 64 + lane;
    pair[s] = idx < end ? load(idx) : kPadKey;
  }
#pragma unroll
  for (int s = 0; s < kRadixSlots; ++s) {
    const bool valid = base + (w * kRadixSlots + s) * 64 + lane < end;
    const uint32_t d = radix_digit(pair[s], shift, dbits);
    const uint64_t peers = radix_peers(d, valid, dbits);
    const int before = __popcll(peers & below);
    const int c = valid ? L.cnt[w][d] : 0;
    rank[s] = c + before;
    if (valid && before == 0) L.cnt[w][d] = c + __popcll(peers);
  }
}

// After a barrier: each wave's first offset of each digit, the waves in
// order from L.run[d]; L.run[d] then moves past the chunk.  Ends with a
// barrier.
__device__ __forceinline__ void radix_wave_offsets(RadixLds& L, int dbits) {
  const int t = threadIdx.x;
  if (t < (1 << dbits)) {
    int s = L.run[t];
    for (int w = 0; w < kRadixWaves; ++w) {
      const int c = L.cnt[w][t];
      L.cnt[w][t] = s;
      s += c;
    }
    L.run[t] = s;
  }
  __syncthreads();
}

template <typename Store>
__device__ __forceinline__ void radix_scatter_chunk(const Store& store, int64_t base, int64_t end,
                                                    int shift, int dbits, const RadixLds& L,
                                                    const uint64_t (&pair)[kRadixSlots],
                                                    const int (&rank)[kRadixSlots]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int s = 0; s < kRadixSlots; ++s) {
    if (base + (w * kRadixSlots + s) * 64 + lane < end)
      store(L.cnt[w][radix_digit(pair[s], shift, dbits)] + rank[s], pair[s]);
  }
}

// ---------------------------------------------------------------------------
// Multi-workgroup passes: workgroup b owns pairs [b per, min(n, (b+1) per))
// ---------------------------------------------------------------------------
// hist[d * gridDim.x + b] = number of pairs of workgroup b whose digit is d.
template <typename Load>
__global__ __launch_bounds__(kRadixThreads) void radix_hist_kernel(Load load, int64_t n, int64_t per,
                                                                   int shift, int dbits,
                                                                   int32_t* __restrict__ hist) {
  __shared__ int h[kRadixBins];
  const int bins = 1 << dbits;
  for (int i = threadIdx.x; i < bins; i += blockDim.x) h[i] = 0;
  __syncthreads();
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t b1 = b0 + per < n ? b0 + per : n;
  for (int64_t i = b0 + threadIdx.x; i < b1; i += blockDim.x)
    atomicAdd(&h[radix_digit(load(i), shift, dbits)], 1);
  __syncthreads();
  for (int i = threadIdx.x; i < bins; i += blockDim.x) hist[i * gridDim.x + blockIdx.x] = h[i];
}

// Writes workgroup b's pairs to their places in `out` for this digit: digit
// d starts after every pair of a smaller digit and after the pairs of digit d
// of workgroups before b; within the workgroup the order is kept.
template <typename Load>
__global__ __launch_bounds__(kRadixThreads) void radix_scatter_kernel(
    Load load, int64_t n, int64_t per, int shift, int dbits, const int32_t* __restrict__ hist,
    uint64_t* __restrict__ out) {
  __shared__ RadixLds L;
  const int t = threadIdx.x, bins = 1 << dbits;
  const int nb = static_cast<int>(gridDim.x), b = static_cast<int>(blockIdx.x);
  int tot = 0, pre = 0;
  if (t < bins) {
    for (int j = 0; j < nb; ++j) {
      const int c = hist[t * nb + j];
      tot += c;
      if (j < b) pre += c;
    }
  }
  int all;
  const int start = block_exclusive_scan(t < bins ? tot : 0, L.wave_tmp, all);
  if (t < bins) L.run[t] = start + pre;
  const int64_t b0 = static_cast<int64_t>(b) * per;
  const int64_t b1 = b0 + per < n ? b0 + per : n;
  uint64_t pair[kRadixSlots];
  int rank[kRadixSlots];
  for (int64_t base = b0; base < b1; base += kRadixChunk) {
    radix_rank_chunk(load, base, b1, shift, dbits, L, pair, rank);
    __syncthreads();
    radix_wave_offsets(L, dbits);
    radix_scatter_chunk([&](int64_t i, uint64_t v) { if (static_cast<uint64_t>(i) < static_cast<uint64_t>(n)) out[i] = v; },
                        base, b1, shift, dbits, L, pair, rank);
    __syncthreads();
  }
}

struct RadixPlan {
  int passes = 1, dbits = 1;  // passes of dbits-wide digits
  int64_t blocks = 1, per = kRadixChunk;  // workgroups of a pass; pairs per workgroup
};

static int bit_length(uint64_t v) {
  int b = 0;
  while (v) {
    ++b;
    v >>= 1;
  }
  return b;
}

static RadixPlan radix_plan(int64_t n, int key_bits) {
  RadixPlan p;
  const int bits = key_bits < 1 ? 1 : key_bits;
  p.passes = (bits + kRadixDigitMax - 1) / kRadixDigitMax;
  p.dbits = (bits + p.passes - 1) / p.passes;
  const int64_t chunks = (n + kRadixChunk - 1) / kRadixChunk;
  p.per = (chunks + kRadixMaxBlocks - 1) / kRadixMaxBlocks * kRadixChunk;
  p.blocks = (n + p.per - 1) / p.per;
  return p;
}

// Workspace of a multi-workgroup sort of n pairs: two pair buffers, the
// histograms, the per-workgroup counts of the dedup scan.
static size_t radix_pairs_bytes(int64_t n) { return align_up(static_cast<size_t>(n) * 8, 256); }
static size_t radix_workspace_bytes(int64_t n) {
  return 2 * radix_pairs_bytes(n) + static_cast<size_t>(kRadixBins) * kRadixMaxBlocks * 4 +
         kRadixMaxBlocks * 4;
}

// Sorts the n pairs produced by `first` (n >= 1) by their low key_bits key
// bits; returns the buffer holding the result.
template <typename First>
static hipError_t radix_sort(const First& first, int64_t n, int key_bits, void* ws, hipStream_t s,
                             uint64_t** result) {
  const RadixPlan p = radix_plan(n, key_bits);
  uint64_t* buf[2] = {static_cast<uint64_t*>(ws),
                      reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + radix_pairs_bytes(n))};
  int32_t* hist = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + 2 * radix_pairs_bytes(n));
  const dim3 grid(static_cast<unsigned>(p.blocks)), block(kRadixThreads);
  for (int k = 0; k < p.passes; ++k) {
    const int shift = k * p.dbits;
    uint64_t* out = buf[k & 1];
    if (k == 0) {
      radix_hist_kernel<<<grid, block, 0, s>>>(first, n, p.per, shift, p.dbits, hist);
      radix_scatter_kernel<<<grid, block, 0, s>>>(first, n, p.per, shift, p.dbits, hist, out);
    } else {
      const PairSource src{buf[(k - 1) & 1]};
      radix_hist_kernel<<<grid, block, 0, s>>>(src, n, p.per, shift, p.dbits, hist);
      radix_scatter_kernel<<<grid, block, 0, s>>>(src, n, p.per, shift, p.dbits, hist, out);
    }
  }
  *result = buf[(p.passes - 1) & 1];
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dedup outputs from sorted pairs
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool run_start(uint64_t pair, uint64_t prev, int64_t p) {
  return p == 0 || static_cast<uint32_t>(prev >> 32) != static_cast<uint32_t>(pair >> 32);
}

// Emits uniq/seg_start/sorted_pos/inv for sorted positions [p0, p1) of n_all
// read through `key_at`, numbering their segments from `carry` (the runs
// started before p0); returns the number of runs started in [p0, p1).  (The
// inverse-map store is bounded by n_all, so no value can write outside it.)
template <typename KeyAt>
__device__ int dedup_emit_range(KeyAt key_at, int64_t n_all, int64_t p0, int64_t p1, int carry,
                                int32_t* uniq,
                                int32_t* inv, int32_t* sorted_pos, int32_t* seg_start,
                                int* wave_tmp) {
  constexpr int kItems = 4;
  const int first = carry;
  const int64_t chunk = static_cast<int64_t>(blockDim.x) * kItems;
  for (int64_t base = p0; base < p1; base += chunk) {
    const int64_t q0 = base + static_cast<int64_t>(threadIdx.x) * kItems;
    uint64_t key[kItems];
    int flag[kItems];
    int local = 0;
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      const int64_t p = q0 + it;
      key[it] = p < p1 ? key_at(p) : kPadKey;
      flag[it] = p < p1 && run_start(key[it], p > 0 ? key_at(p - 1) : 0, p);
      local += flag[it];
    }
    int total;
    const int before = block_exclusive_scan(local, wave_tmp, total);
    int seg = carry + before - 1;  // index of the segment holding the previous item
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      const int64_t p = q0 + it;
      if (p < p1) {
        seg += flag[it];
        const int32_t id = static_cast<int32_t>(key[it] >> 32);
        const int32_t pos = static_cast<int32_t>(key[it] & 0xffffffffu);
        if (flag[it]) {
          uniq[seg] = id;
          seg_start[seg] = static_cast<int32_t>(p);
        }
        sorted_pos[p] = pos;
        if (static_cast<uint32_t>(pos) < static_cast<uint64_t>(n_all)) inv[pos] = seg;
      }
    }
    carry += total;
  }
  return carry - first;
}

// counts[b] = number of ID runs starting in workgroup b's range.
__global__ __launch_bounds__(kRadixThreads) void dedup_count_kernel(const uint64_t* __restrict__ pairs,
                                                                    int64_t n, int64_t per,
                                                                    int32_t* __restrict__ counts) {
  __shared__ int wave_tmp[16];
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t b1 = b0 + per < n ? b0 + per : n;
  int local = 0;
  for (int64_t p = b0 + threadIdx.x; p < b1; p += blockDim.x)
    local += run_start(pairs[p], p > 0 ? pairs[p - 1] : 0, p);
  int total;
  (void)block_exclusive_scan(local, wave_tmp, total);
  if (threadIdx.x == 0) counts[blockIdx.x] = total;
}

// The scan over workgroup b's range, its segments numbered after the runs of
// the ranges before it; the last workgroup writes *n_unique and seg_start[U].
__global__ __launch_bounds__(kRadixThreads) void dedup_write_kernel(
    const uint64_t* __restrict__ pairs, int64_t n, int64_t per, const int32_t* __restrict__ counts,
    int32_t* uniq, int32_t* inv, int32_t* sorted_pos, int32_t* seg_start, int32_t* n_unique) {
  __shared__ int wave_tmp[16];
  int carry = 0;
  for (unsigned j = 0; j < blockIdx.x; ++j) carry += counts[j];
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t b1 = b0 + per < n ? b0 + per : n;
  const int mine = dedup_emit_range([&](int64_t p) { return pairs[p]; }, n, b0, b1, carry, uniq,
                                    inv, sorted_pos, seg_start, wave_tmp);
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) {
    *n_unique = carry + mine;
    seg_start[carry + mine] = static_cast<int32_t>(n);
  }
}

// Whole dedup of at most kRadixChunk positions in one workgroup, the pairs in
// LDS.
__global__ __launch_bounds__(kRadixThreads) void dedup_small_kernel(
    const int32_t* ids, int64_t n, int64_t vocab, int passes, int dbits, int32_t* uniq,
    int32_t* inv, int32_t* sorted_pos, int32_t* seg_start, int32_t* n_unique, int* err) {
  __shared__ uint64_t buf[2][kRadixChunk];
  __shared__ RadixLds L;
  const int t = threadIdx.x, bins_max = 1 << dbits;
  uint64_t pair[kRadixSlots];
  int rank[kRadixSlots];
  for (int k = 0; k < passes; ++k) {
    const int shift = k * dbits;
    if (k == 0)
      radix_rank_chunk(DedupSource{ids, vocab, err}, 0, n, shift, dbits, L, pair, rank);
    else
      radix_rank_chunk([&](int64_t i) { return buf[(k - 1) & 1][i]; }, 0, n, shift, dbits, L, pair,
                       rank);
    __syncthreads();
    int tot = 0;
    if (t < bins_max)
      for (int w = 0; w < kRadixWaves; ++w) tot += L.cnt[w][t];
    int all;
    const int start = block_exclusive_scan(t < bins_max ? tot : 0, L.wave_tmp, all);
    if (t < bins_max) L.run[t] = start;
    __syncthreads();
    radix_wave_offsets(L, dbits);
    uint64_t* out = buf[k & 1];
    radix_scatter_chunk([&](int64_t i, uint64_t v) { if (static_cast<uint64_t>(i) < static_cast<uint64_t>(n)) out[i] = v; },
                        0, n, shift, dbits, L, pair, rank);
    __syncthreads();
  }
  const uint64_t* sorted = buf[(passes - 1) & 1];
  const int u = dedup_emit_range([&](int64_t p) { return sorted[p]; }, n, 0, n, 0, uniq, inv,
                                 sorted_pos, seg_start, L.wave_tmp);
  if (t == 0) {
    *n_unique = u;
    seg_start[u] = static_cast<int32_t>(n);
  }
}

// Stable LSD radix sort of one wave's (key, value) pairs by the low `bits`
// key bits, one bit per pass: the lanes whose bit is 0 keep their order and
// move to the front, those whose bit is 1 follow in order (a split by two
// ballots, then each lane pushes its pair to its new lane).  The valid pairs
// are those of lanes [0, n); the other lanes keep their place.
__device__ __forceinline__ void wave_radix_sort(uint32_t& key, uint32_t& val, bool valid, int bits) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1;
  for (int b = 0; b < bits; ++b) {
    const bool one = (key >> b) & 1u;
    const uint64_t zeros = __ballot(valid && !one);
    const uint64_t ones = __ballot(valid && one);
    const int dest = !valid ? lane
                     : one  ? __popcll(zeros) + __popcll(ones & below)
                            : __popcll(zeros & below);
    key = static_cast<uint32_t>(__builtin_amdgcn_ds_permute(dest << 2, static_cast<int>(key)));
    val = static_cast<uint32_t>(__builtin_amdgcn_ds_permute(dest << 2, static_cast<int>(val)));
  }
}

// Key bits of a dedup: IDs below vocab.
static int dedup_key_bits(int64_t vocab) { return bit_length(static_cast<uint64_t>(vocab - 1)); }

// Whole dedup of at most 64 positions (a decode batch) in one wave: lane i
// starts with (ids[i], i), the wave radix sort orders the pairs, and the
// segment starts come from a ballot, so there is no LDS table and no
// barrier.  Same outputs as the workgroup kernels.
__global__ __launch_bounds__(64) void dedup_wave_kernel(const int32_t* ids, int64_t n, int64_t vocab,
                                                        int bits, int32_t* uniq, int32_t* inv,
                                                        int32_t* sorted_pos, int32_t* seg_start,
                                                        int32_t* n_unique, int* err) {
  const int lane = threadIdx.x;
  const bool valid = lane < n;
  uint32_t id = 0, pos = static_cast<uint32_t>(lane);
  if (valid) {
    const int32_t t = ids[lane];
    if (t < 0 || t >= vocab) flag_index_error(err);
    id = static_cast<uint32_t>(t);
  }
  wave_radix_sort(id, pos, valid, bits);
  const uint32_t prev = static_cast<uint32_t>(__shfl_up(static_cast<int>(id), 1, 64));
  const bool first = valid && (lane == 0 || prev != id);
  const uint64_t starts = __ballot(first);
  const int seg = __popcll(starts & ((2ull << lane) - 1)) - 1;   // segment of this position
  if (valid) {
    if (first) {
      uniq[seg] = static_cast<int32_t>(id);
      seg_start[seg] = lane;
    }
    sorted_pos[lane] = static_cast<int32_t>(pos);
    if (pos < n) inv[pos] = seg;
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
    const int32_t* ids, int64_t n, int64_t vocab, int bits, const int32_t* id_to_slot,
    int32_t* uniq, int32_t* inv, int32_t* sorted_pos, int32_t* seg_start, int32_t* n_unique,
    int32_t* code, int32_t* miss_uidx, int32_t* n_miss, int32_t* row_src, int* err) {
  const int lane = threadIdx.x;
  const bool valid = lane < n;
  uint32_t key = 0, pos_u = static_cast<uint32_t>(lane);
  if (valid) {
    const int32_t t = ids[lane];
    if (t < 0 || t >= vocab) flag_index_error(err);
    key = static_cast<uint32_t>(t);
  }
  wave_radix_sort(key, pos_u, valid, bits);
  const int32_t id = static_cast<int32_t>(key);
  const int32_t prev = __shfl_up(id, 1, 64);
  const bool first = valid && (lane == 0 || prev != id);
  const uint64_t starts = __ballot(first);
  const int seg = __popcll(starts & ((2ull << lane) - 1)) - 1;
  const bool in_table = id >= 0 && id < vocab;
  const int32_t slot = valid && in_table ? id_to_slot[id] : -1;
  const bool miss = first && slot < 0;
  const uint64_t misses = __ballot(miss);
  if (valid) {
    const int32_t pos = static_cast<int32_t>(pos_u);
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
    if (pos < n) {
      inv[pos] = seg;
      if (row_src) row_src[pos] = in_table ? (slot >= 0 ? slot : -1 - id) : INT32_MIN;
    }
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
  dedup_lookup_wave_kernel<<<dim3(1), dim3(64), 0, s>>>(ids, n, vocab, dedup_key_bits(vocab),
                                                        id_to_slot, uniq, inv, sorted_pos,
                                                        seg_start, n_unique, code, miss_uidx,
                                                        n_miss, row_src, err);
  return hipGetLastError();
}

size_t dedup_workspace_bytes(int64_t n) {
  if (n <= kRadixChunk) return 0;
  return radix_workspace_bytes(n);
}

hipError_t launch_dedup(const int32_t* ids, int64_t n, int64_t vocab, int32_t* uniq, int32_t* inv,
                        int32_t* sorted_pos, int32_t* seg_start, int32_t* n_unique, void* ws,
                        hipStream_t s, int* err) {
  const int bits = dedup_key_bits(vocab);
  if (n <= 64) {
    dedup_wave_kernel<<<dim3(1), dim3(64), 0, s>>>(ids, n, vocab, bits, uniq, inv, sorted_pos,
                                                   seg_start, n_unique, err);
    return hipGetLastError();
  }
  if (n <= kRadixChunk) {
    const RadixPlan p = radix_plan(n, bits);
    dedup_small_kernel<<<dim3(1), dim3(kRadixThreads), 0, s>>>(ids, n, vocab, p.passes, p.dbits,
                                                                uniq, inv, sorted_pos, seg_start,
                                                                n_unique, err);
    return hipGetLastError();
  }
  uint64_t* sorted = nullptr;
  hipError_t e = radix_sort(DedupSource{ids, vocab, err}, n, bits, ws, s, &sorted);
  if (e != hipSuccess) return e;
  const RadixPlan p = radix_plan(n, bits);
  int32_t* counts = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + 2 * radix_pairs_bytes(n) +
                                               static_cast<size_t>(kRadixBins) * kRadixMaxBlocks * 4);
  const dim3 grid(static_cast<unsigned>(p.blocks)), block(kRadixThreads);
  dedup_count_kernel<<<grid, block, 0, s>>>(sorted, n, p.per, counts);
  dedup_write_kernel<<<grid, block, 0, s>>>(sorted, n, p.per, counts, uniq, inv, sorted_pos,
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
  if (id < 0 || id >= vocab) return;   // (cannot happen: the values are the IDs 0 .. vocab-1)
  // every ID appears exactly once in the sorted keys, so each id_to_slot entry
  // is written exactly once
  if (i < capacity) {
    slot_to_id[i] = id;
    id_to_slot[id] = static_cast<int32_t>(i);
  } else {
    id_to_slot[id] = -1;
  }
}

size_t cache_build_workspace_bytes(int64_t vocab) { return radix_workspace_bytes(vocab); }

hipError_t launch_cache_build(const int64_t* counts, int64_t vocab, int64_t capacity,
                              int32_t* id_to_slot, int32_t* slot_to_id, void* ws, hipStream_t s,
                              int* err) {
  uint64_t* sorted = nullptr;
  hipError_t e = radix_sort(CacheSource{counts, err}, vocab, 31, ws, s, &sorted);
  if (e != hipSuccess) return e;
  cache_assign_kernel<<<dim3(static_cast<unsigned>((vocab + 255) / 256)), dim3(256), 0, s>>>(
      sorted, vocab, capacity, id_to_slot, slot_to_id);
  return hipGetLastError();
}

}  // namespace staple
