// Row movement kernels: cache count pass, cache probe with miss compaction,
// row gather / compact-block assembly, and the table-row gradient
// segment-sum.
#include "common.h"

namespace staple {

// Block-wide exclusive scan (same contract as the one in sort.hip; kept local
// to this translation unit).
__device__ static int scan_block(int v, int* wave_tmp, int& total) {
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
// Count pass over a calibration stream.
// ---------------------------------------------------------------------------
__global__ void count_kernel(const int32_t* ids, int64_t n, int64_t vocab,
                             unsigned long long* counts, int* err) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t t = ids[i];
  if (t < 0 || t >= vocab) {
    flag_index_error(err);
    return;
  }
  atomicAdd(&counts[t], 1ull);
}

hipError_t launch_cache_count(const int32_t* ids, int64_t n, int64_t vocab, int64_t* counts,
                              hipStream_t s, int* err) {
  if (n == 0) return hipSuccess;
  count_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s>>>(
      ids, n, vocab, reinterpret_cast<unsigned long long*>(counts), err);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Cache probe + stable miss compaction (one workgroup; U is at most a batch).
// With row_src, also each token's row source for the decode kernels' direct
// reads: row_src[t] = the cache slot of the token's row when cached, else
// -1 - id (the row of the table), INT32_MIN when inv or the ID is out of range.
// ---------------------------------------------------------------------------
constexpr int kLookupThreads = 1024;

__global__ __launch_bounds__(kLookupThreads) void lookup_kernel(
    const int32_t* uniq, const int32_t* n_unique_p, int64_t max_unique, const int32_t* id_to_slot,
    int64_t vocab, int32_t* code, int32_t* miss_uidx, int32_t* miss_ids, int32_t* n_miss,
    const int32_t* inv, int64_t n_tokens, int32_t* row_src, int* err) {
  __shared__ int wave_tmp[16];
  int64_t nu = *n_unique_p;
  if (nu < 0 || nu > max_unique) {
    if (threadIdx.x == 0) flag_index_error(err);
    nu = nu < 0 ? 0 : max_unique;
  }
  int carry = 0;
  for (int64_t base = 0; base < nu; base += blockDim.x) {
    const int64_t u = base + threadIdx.x;
    int32_t slot = 0;
    int32_t id = 0;
    int miss = 0;
    if (u < nu) {
      id = uniq[u];
      if (id < 0 || id >= vocab) {
        flag_index_error(err);
        slot = -1;
      } else {
        slot = id_to_slot[id];
      }
      miss = slot < 0;
    }
    int total;
    const int before = scan_block(miss, wave_tmp, total);
    if (u < nu) {
      if (miss) {
        const int m = carry + before;
        code[u] = -1 - m;
        miss_uidx[m] = static_cast<int32_t>(u);
        if (miss_ids) miss_ids[m] = id;
      } else {
        code[u] = slot;
      }
    }
    carry += total;
  }
  if (threadIdx.x == 0) *n_miss = carry;
  if (!row_src) return;
  __syncthreads();   // code[] of the whole batch written
  for (int64_t t = threadIdx.x; t < n_tokens; t += blockDim.x) {
    const int32_t u = inv[t];
    int32_t src = INT32_MIN;
    if (u < 0 || u >= nu) {
      flag_index_error(err);
    } else {
      const int32_t id = uniq[u];
      if (id >= 0 && id < vocab) {
        const int32_t c = code[u];
        src = c >= 0 ? c : -1 - id;
      }
    }
    row_src[t] = src;
  }
}

hipError_t launch_cache_lookup(const int32_t* uniq, const int32_t* n_unique, int64_t max_unique,
                               const int32_t* id_to_slot, int64_t vocab, int32_t* code,
                               int32_t* miss_uidx, int32_t* miss_ids, int32_t* n_miss,
                               hipStream_t s, int* err, const int32_t* inv, int64_t n_tokens,
                               int32_t* row_src) {
  lookup_kernel<<<dim3(1), dim3(kLookupThreads), 0, s>>>(uniq, n_unique, max_unique, id_to_slot,
                                                         vocab, code, miss_uidx, miss_ids, n_miss,
                                                         inv, n_tokens, row_src, err);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Token split by cache outcome (one workgroup, stable): the token positions
// whose row is cached and those whose row was a miss, each in ascending
// order, and every token's row in its source (cache slot or miss index).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kLookupThreads) void split_tokens_kernel(
    const int32_t* inv, int64_t n, const int32_t* code, const int32_t* n_unique_p,
    int64_t max_unique, int32_t* hit_pos, int32_t* miss_pos, int32_t* tok_row, int32_t* counts,
    int* err) {
  __shared__ int wave_tmp[16];
  int64_t nu = *n_unique_p;
  if (nu < 0 || nu > max_unique) {
    if (threadIdx.x == 0) flag_index_error(err);
    nu = nu < 0 ? 0 : max_unique;
  }
  int hits = 0, misses = 0;
  for (int64_t base = 0; base < n; base += blockDim.x) {
    const int64_t t = base + threadIdx.x;
    int hit = 0, miss = 0;
    int32_t row = -1;
    if (t < n) {
      const int32_t u = inv[t];
      if (u < 0 || u >= nu) {
        flag_index_error(err);   // kept with the hits, row -1: the gate/up epilogue flags it again
        hit = 1;
      } else {
        const int32_t c = code[u];
        hit = c >= 0;
        miss = !hit;
        row = hit ? c : -1 - c;
      }
    }
    int total_hit, total_miss;
    const int bh = scan_block(hit, wave_tmp, total_hit);
    const int bm = scan_block(miss, wave_tmp, total_miss);
    if (t < n) {
      tok_row[t] = row;
      if (hit) hit_pos[hits + bh] = static_cast<int32_t>(t);
      if (miss) miss_pos[misses + bm] = static_cast<int32_t>(t);
    }
    hits += total_hit;
    misses += total_miss;
  }
  if (threadIdx.x == 0) {
    counts[0] = hits;
    counts[1] = misses;
  }
}

hipError_t launch_split_tokens(const int32_t* inv, int64_t n, const int32_t* code,
                               const int32_t* n_unique, int64_t max_unique, int32_t* hit_pos,
                               int32_t* miss_pos, int32_t* tok_row, int32_t* counts, hipStream_t s,
                               int* err) {
  split_tokens_kernel<<<dim3(1), dim3(kLookupThreads), 0, s>>>(inv, n, code, n_unique, max_unique,
                                                               hit_pos, miss_pos, tok_row, counts,
                                                               err);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row copies.  One workgroup per destination row; 16-byte vectors.
// ---------------------------------------------------------------------------
constexpr int kRowThreads = 256;

// Four 16-byte loads in flight per thread before the stores (a row read over
// PCIe from pinned host memory has a long latency).
__device__ __forceinline__ void copy_row16(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                           int64_t vecs) {
  int64_t v = threadIdx.x;
  for (; v + 3 * kRowThreads < vecs; v += 4 * kRowThreads) {
    uint4 t[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) t[j] = src[v + j * kRowThreads];
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[v + j * kRowThreads] = t[j];
  }
  for (; v < vecs; v += kRowThreads) dst[v] = src[v];
}

// Row copies run one workgroup per row (grid-stride over rows when the grid
// is capped).  Copies whose source is host memory cap the grid so that their
// long-latency workgroups occupy one slot on a few CUs and a concurrent
// kernel (the gate/up GEMM the copy overlaps) still fits beside them.

// dst[r] = src[index[r]]  (r < n, n from the device scalar when given)
__global__ __launch_bounds__(kRowThreads) void gather_rows_kernel(
    const void* src, int64_t src_rows, const int32_t* index, const int32_t* n_rows_p,
    int64_t max_rows, int64_t row_bytes, void* dst, int* err) {
  const int64_t n = n_rows_p ? min(static_cast<int64_t>(*n_rows_p), max_rows) : max_rows;
  for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
    const int32_t i = index[r];
    if (i < 0 || i >= src_rows) {
      if (threadIdx.x == 0) flag_index_error(err);
      continue;
    }
    copy_row16(reinterpret_cast<const uint4*>(static_cast<const char*>(src) + i * row_bytes),
               reinterpret_cast<uint4*>(static_cast<char*>(dst) + r * row_bytes), row_bytes / 16);
  }
}

static unsigned row_grid(int64_t rows, unsigned max_workgroups) {
  return static_cast<unsigned>(max_workgroups > 0 && rows > max_workgroups ? max_workgroups : rows);
}

hipError_t launch_gather_rows(const void* src, int64_t src_rows, const int32_t* index,
                              const int32_t* n_rows, int64_t max_rows, int64_t row_bytes,
                              void* dst, hipStream_t s, int* err, unsigned max_workgroups) {
  if (max_rows == 0) return hipSuccess;
  gather_rows_kernel<<<dim3(row_grid(max_rows, max_workgroups)), dim3(kRowThreads), 0, s>>>(
      src, src_rows, index, n_rows, max_rows, row_bytes, dst, err);
  return hipGetLastError();
}

// rows[u] = code[u] >= 0 ? cache_rows[code[u]] : miss_rows[-1 - code[u]]
__global__ __launch_bounds__(kRowThreads) void assemble_rows_kernel(
    const void* cache_rows, int64_t capacity, const void* miss_rows, int64_t max_miss,
    const int32_t* code, const int32_t* n_unique_p, int64_t row_bytes, void* rows, int* err) {
  const int64_t u = blockIdx.x;
  if (u >= *n_unique_p) return;
  const int32_t c = code[u];
  const char* src;
  if (c >= 0) {
    if (c >= capacity) {
      if (threadIdx.x == 0) flag_index_error(err);
      return;
    }
    src = static_cast<const char*>(cache_rows) + c * row_bytes;
  } else {
    const int64_t m = -1 - static_cast<int64_t>(c);
    if (m >= max_miss) {
      if (threadIdx.x == 0) flag_index_error(err);
      return;
    }
    src = static_cast<const char*>(miss_rows) + m * row_bytes;
  }
  copy_row16(reinterpret_cast<const uint4*>(src),
             reinterpret_cast<uint4*>(static_cast<char*>(rows) + u * row_bytes), row_bytes / 16);
}

hipError_t launch_assemble_rows(const void* cache_rows, int64_t capacity, const void* miss_rows,
                                int64_t max_miss, const int32_t* code, const int32_t* n_unique,
                                int64_t max_unique, int64_t row_bytes, void* rows, hipStream_t s,
                                int* err) {
  if (max_unique == 0) return hipSuccess;
  assemble_rows_kernel<<<dim3(static_cast<unsigned>(max_unique)), dim3(kRowThreads), 0, s>>>(
      cache_rows, capacity, miss_rows, max_miss, code, n_unique, row_bytes, rows, err);
  return hipGetLastError();
}

// rows[u] = code[u] >= 0 ? cache_rows[code[u]] : table[uniq[u]]: hits from the
// HBM cache, misses read straight from the table (device memory or pinned
// host memory read over PCIe, one whole row per workgroup).
__global__ __launch_bounds__(kRowThreads) void assemble_rows_table_kernel(
    const void* cache_rows, int64_t capacity, const void* table, int64_t vocab,
    const int32_t* uniq, const int32_t* code, const int32_t* n_unique_p, int64_t max_unique,
    int64_t row_bytes, void* rows, int* err) {
  const int64_t n = min(static_cast<int64_t>(*n_unique_p), max_unique);
  for (int64_t u = blockIdx.x; u < n; u += gridDim.x) {
    const int32_t c = code[u];
    const char* src;
    if (c >= 0) {
      if (c >= capacity) {
        if (threadIdx.x == 0) flag_index_error(err);
        continue;
      }
      src = static_cast<const char*>(cache_rows) + c * row_bytes;
    } else {
      const int32_t id = uniq[u];
      if (id < 0 || id >= vocab) {
        if (threadIdx.x == 0) flag_index_error(err);
        continue;
      }
      src = static_cast<const char*>(table) + id * row_bytes;
    }
    copy_row16(reinterpret_cast<const uint4*>(src),
               reinterpret_cast<uint4*>(static_cast<char*>(rows) + u * row_bytes), row_bytes / 16);
  }
}

hipError_t launch_assemble_rows_table(const void* cache_rows, int64_t capacity, const void* table,
                                      int64_t vocab, const int32_t* uniq, const int32_t* code,
                                      const int32_t* n_unique, int64_t max_unique,
                                      int64_t row_bytes, void* rows, hipStream_t s, int* err,
                                      unsigned max_workgroups) {
  if (max_unique == 0) return hipSuccess;
  assemble_rows_table_kernel<<<dim3(row_grid(max_unique, max_workgroups)), dim3(kRowThreads), 0, s>>>(
      cache_rows, capacity, table, vocab, uniq, code, n_unique, max_unique, row_bytes, rows, err);
  return hipGetLastError();
}

// The same assembly for several layers at once (the tables of a layer stack
// share one cache map): work item k = (layer k / max_unique, unique row
// k % max_unique).  A workgroup takes R consecutive work items and loads all
// of their rows before storing any.  R = 4 when the grid is capped to run
// beside another kernel on a few CUs, or when there are enough items for
// four per workgroup to fill the grid: many rows' PCIe reads are then in
// flight per workgroup.  R = 1 otherwise (a decode step's few rows spread
// over as many workgroups as possible).  Table l's token rows are
// table_ld[l] bytes apart (row_bytes for a table of its own, more when
// several layers' tables are interleaved token-major).

// a grid capped below this many workgroups shares the GPU with another kernel
constexpr unsigned kRowDeepCap = 256;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u32x4_t* grow_src_t;
typedef __attribute__((address_space(1))) u32x4_t* grow_dst_t;

// Source and destination of work item k of a multi-layer assembly, or false
// when it has nothing to copy (past the unique rows, or a bad slot or ID,
// which it flags).  Global-address-space pointers: device memory or pinned
// host memory mapped for the device.
__device__ __forceinline__ bool layer_row_ends(const LayerRowSources& src, int64_t k, int64_t total,
                                               int64_t n, int64_t max_unique, int64_t capacity,
                                               int64_t vocab, const int32_t* uniq,
                                               const int32_t* code, int64_t row_bytes, int* err,
                                               grow_src_t& from, grow_dst_t& to) {
  if (k >= total) return false;
  const int l = static_cast<int>(k / max_unique);
  const int64_t u = k - static_cast<int64_t>(l) * max_unique;
  if (u >= n) return false;
  const int32_t c = code[u];
  const char* f;
  if (c >= 0) {
    if (c >= capacity) {
      if (threadIdx.x == 0) flag_index_error(err);
      return false;
    }
    f = static_cast<const char*>(src.cache_rows[l]) + c * row_bytes;
  } else {
    const int32_t id = uniq[u];
    if (id < 0 || id >= vocab) {
      if (threadIdx.x == 0) flag_index_error(err);
      return false;
    }
    f = static_cast<const char*>(src.table[l]) + id * src.table_ld[l];
  }
  from = (grow_src_t)(f);
  to = (grow_dst_t)(static_cast<char*>(src.rows[l]) + u * row_bytes);
  return true;
}

template <int R>
__global__ __launch_bounds__(kRowThreads) void assemble_rows_layers_kernel(
    LayerRowSources src, int n_layers, int64_t capacity, int64_t vocab, const int32_t* uniq,
    const int32_t* code, const int32_t* n_unique_p, int64_t max_unique, int64_t row_bytes,
    int* err) {
  const int64_t n = min(static_cast<int64_t>(*n_unique_p), max_unique);
  const int64_t total = static_cast<int64_t>(n_layers) * max_unique;
  const int64_t vecs = row_bytes / 16;
  for (int64_t k0 = static_cast<int64_t>(blockIdx.x) * R; k0 < total;
       k0 += static_cast<int64_t>(gridDim.x) * R) {
    grow_src_t f[R] = {};
    grow_dst_t d[R] = {};
    bool ok[R];
#pragma unroll
    for (int j = 0; j < R; ++j)
      ok[j] = layer_row_ends(src, k0 + j, total, n, max_unique, capacity, vocab, uniq, code,
                             row_bytes, err, f[j], d[j]);
    // a group with nothing to copy is skipped; an empty place of a group
    // repeats its first row (the same bytes to the same place, by the same
    // thread), so the copy below needs no per-row predicate
    int first = -1;
#pragma unroll
    for (int j = R - 1; j >= 0; --j)
      if (ok[j]) first = j;
    if (first < 0) continue;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      if (!ok[j]) {
        f[j] = f[first];
        d[j] = d[first];
      }
    }
    // whole passes of 4 pieces per thread: every row's pieces loaded, then stored
    int64_t v0 = 0;
    for (; v0 + 4 * kRowThreads <= vecs; v0 += 4 * kRowThreads) {
      u32x4_t t[R][4];
#pragma unroll
      for (int j = 0; j < R; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) t[j][i] = f[j][v0 + threadIdx.x + i * kRowThreads];
#pragma unroll
      for (int j = 0; j < R; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) d[j][v0 + threadIdx.x + i * kRowThreads] = t[j][i];
    }
    for (int64_t v = v0 + threadIdx.x; v < vecs; v += kRowThreads) {
      u32x4_t t[R];
#pragma unroll
      for (int j = 0; j < R; ++j) t[j] = f[j][v];
#pragma unroll
      for (int j = 0; j < R; ++j) d[j][v] = t[j];
    }
  }
}

hipError_t launch_assemble_rows_layers(const LayerRowSources& src, int n_layers, int64_t capacity,
                                       int64_t vocab, const int32_t* uniq, const int32_t* code,
                                       const int32_t* n_unique, int64_t max_unique,
                                       int64_t row_bytes, hipStream_t s, int* err,
                                       unsigned max_workgroups) {
  if (max_unique == 0 || n_layers == 0) return hipSuccess;
  const int64_t items = static_cast<int64_t>(n_layers) * max_unique;
  const int64_t groups4 = (items + 3) / 4;
  if (max_workgroups < kRowDeepCap || groups4 >= max_workgroups)
    assemble_rows_layers_kernel<4><<<dim3(row_grid(groups4, max_workgroups)), dim3(kRowThreads), 0,
                                     s>>>(src, n_layers, capacity, vocab, uniq, code, n_unique,
                                          max_unique, row_bytes, err);
  else
    assemble_rows_layers_kernel<1><<<dim3(row_grid(items, max_workgroups)), dim3(kRowThreads), 0,
                                     s>>>(src, n_layers, capacity, vocab, uniq, code, n_unique,
                                          max_unique, row_bytes, err);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Table-row gradient: d_rows[u, c] = sum over sorted positions p of segment u
// of du[sorted_pos[p], c], accumulated in fp32.
//
// Token frequencies are Zipf-skewed (one ID can hold ~13% of a batch), so the
// work is split over fixed chunks of kSegChunk sorted positions rather than
// over segments (one wave per (chunk, 512 columns), four waves of
// neighbouring column blocks per workgroup, the column blocks of a chunk
// dispatched together so its du rows are read whole within a short time).  Pass 1: each wave walks its
// positions in order; a segment that starts and ends inside the chunk is
// written to d_rows directly; the run of a segment that began in an earlier
// chunk goes to first[chunk], the run of a segment that continues into the
// next chunk goes to last[chunk].  Pass 2: each segment spanning chunks
// c0 < c1 sums last[c0] + first[c0+1] + ... + first[c1] in that order (done
// by the wave of chunk c0).
// Every sum has a fixed order, so the result is deterministic.
// du lives at column offset du_col of rows with stride du_ld (elements);
// each lane owns 8 consecutive columns (one 16-byte bf16 load, two for fp32).
// ---------------------------------------------------------------------------
constexpr int kSegCols = 512;   // 64 lanes x 8 columns
constexpr int kSegAhead = 8;    // du rows in flight per lane (chunk pass)
constexpr int kFixAhead = 8;    // partials in flight per lane (fixup pass)
constexpr int kSegWaves = 4;    // column blocks per workgroup (one wave each)

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]);

template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float (&v)[8]) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void store8f(float* p, const float (&v)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Segment of sorted position p: the inverse map of its token (two loads; an
// out-of-range entry sets the error word and counts as segment 0).
__device__ __forceinline__ int64_t segment_of(int64_t p, int64_t n_tokens, int64_t nu,
                                              const int32_t* sorted_pos, const int32_t* inv,
                                              int* err) {
  const int32_t t = sorted_pos[p];
  if (t < 0 || t >= n_tokens) {
    flag_index_error(err);
    return 0;
  }
  const int32_t s = inv[t];
  if (s < 0 || s >= nu) {
    flag_index_error(err);
    return 0;
  }
  return s;
}

template <typename T>
__global__ __launch_bounds__(64 * kSegWaves) void segsum_chunk_kernel(
    const T* __restrict__ du, int64_t du_ld, int64_t du_col, int64_t n_tokens, int64_t d_ff,
    const int32_t* __restrict__ sorted_pos, const int32_t* __restrict__ inv,
    const int32_t* __restrict__ seg_start, const int32_t* __restrict__ n_unique_p,
    int64_t max_unique, float* __restrict__ d_rows, float* __restrict__ first,
    float* __restrict__ last, int* err) {
  const int lane = threadIdx.x & 63;
  const int64_t c = blockIdx.y;
  const int64_t col = (static_cast<int64_t>(blockIdx.x) * kSegWaves + (threadIdx.x >> 6)) * kSegCols +
                      lane * 8;
  const int64_t p0 = c * kSegChunk;
  const int64_t p1 = min(p0 + kSegChunk, n_tokens);
  // a unique count past the rows d_rows holds is an index error: nothing is written
  const int64_t nu = *n_unique_p;
  if (nu > max_unique) {
    if (threadIdx.x == 0 && blockIdx.x == 0 && blockIdx.y == 0) flag_index_error(err);
    return;
  }
  // whole waves past d_ff leave; inside a wave every lane stays for the row
  // exchange and only lanes with col < d_ff load and store
  if (col - lane * 8 >= d_ff || nu <= 0) return;
  const bool col_ok = col < d_ff;
  const int64_t lcol = col_ok ? col : 0;
  int64_t sg = segment_of(p0, n_tokens, nu, sorted_pos, inv, err);
  int64_t s_begin = seg_start[sg], s_end = seg_start[sg + 1];
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  // the chunk's rows: lane i holds the row of position p0 + i % 32
  static_assert(kSegChunk <= 64, "one position per lane");
  int32_t my_row = 0;
  {
    const int64_t p = p0 + (lane % kSegChunk);
    if (p < p1) {
      my_row = sorted_pos[p];
      if (my_row < 0 || my_row >= n_tokens) {
        flag_index_error(err);
        my_row = 0;
      }
    }
  }
  // positions in groups of kSegAhead: the group's rows are loaded together,
  // then added in position order (the order of the sums does not change)
  for (int64_t pb = p0; pb < p1; pb += kSegAhead) {
    float v[kSegAhead][8];
#pragma unroll
    for (int j = 0; j < kSegAhead; ++j) {
      const int64_t p = pb + j < p1 ? pb + j : p1 - 1;
      const int64_t row = __shfl(my_row, static_cast<int>(p - p0), 64);
      load8<T>(du + row * du_ld + du_col + lcol, v[j]);
    }
#pragma unroll
    for (int j = 0; j < kSegAhead; ++j) {
      const int64_t p = pb + j;
      if (p >= p1) break;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[j][i];
      const bool seg_ends = (p + 1 == s_end);
      if (seg_ends || p + 1 == p1) {
        float* dst;
        if (s_begin >= p0 && s_end <= p1) dst = d_rows + sg * d_ff + col;   // whole segment here
        else if (s_begin < p0) dst = first + c * d_ff + col;                // began in an earlier chunk
        else dst = last + c * d_ff + col;                                   // continues past p1
        if (col_ok) store8f(dst, acc);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        if (seg_ends && sg + 1 < nu) {
          ++sg;
          s_begin = s_end;
          s_end = seg_start[sg + 1];
        }
      }
    }
  }
}

// One wave per (chunk, 512 columns): the chunk whose last run starts a
// segment that continues past it owns that segment's final sum.
__global__ __launch_bounds__(64 * kSegWaves) void segsum_fixup_kernel(
    int64_t n_tokens, int64_t d_ff, const int32_t* __restrict__ sorted_pos,
    const int32_t* __restrict__ inv, const int32_t* __restrict__ seg_start,
    const int32_t* __restrict__ n_unique_p, int64_t max_unique, const float* __restrict__ first,
    const float* __restrict__ last, float* __restrict__ d_rows, int* err) {
  const int64_t c0 = blockIdx.y;
  const int64_t col = (static_cast<int64_t>(blockIdx.x) * kSegWaves + (threadIdx.x >> 6)) * kSegCols +
                      (threadIdx.x & 63) * 8;
  const int64_t nu = *n_unique_p;
  if (col >= d_ff || nu <= 0 || nu > max_unique) return;   // flagged by the chunk pass
  const int64_t p0 = c0 * kSegChunk;
  const int64_t p1 = min(p0 + kSegChunk, n_tokens);
  const int64_t lo = segment_of(p1 - 1, n_tokens, nu, sorted_pos, inv, err);
  const int64_t b = seg_start[lo], e = seg_start[lo + 1];
  if (b < p0 || e <= p1) return;   // not a segment that starts here and continues
  const int64_t c1 = (e - 1) / kSegChunk;
  float acc[8];
  load8<float>(last + c0 * d_ff + col, acc);
  // kFixAhead partials loaded together, added in chunk order
  for (int64_t cb = c0 + 1; cb <= c1; cb += kFixAhead) {
    float v[kFixAhead][8];
#pragma unroll
    for (int j = 0; j < kFixAhead; ++j) {
      const int64_t c = cb + j <= c1 ? cb + j : c1;
      load8<float>(first + c * d_ff + col, v[j]);
    }
#pragma unroll
    for (int j = 0; j < kFixAhead; ++j) {
      if (cb + j <= c1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += v[j][i];
      }
    }
  }
  store8f(d_rows + lo * d_ff + col, acc);
}

size_t segment_sum_workspace_bytes(int64_t n_tokens, int64_t d_ff) {
  const int64_t chunks = (n_tokens + kSegChunk - 1) / kSegChunk;
  return static_cast<size_t>(2 * chunks * d_ff) * sizeof(float);
}

hipError_t launch_segment_sum(int dtype, const void* du, int64_t du_ld, int64_t du_col,
                              int64_t n_tokens, int64_t d_ff, const int32_t* sorted_pos,
                              const int32_t* inv, const int32_t* seg_start,
                              const int32_t* n_unique,
                              int64_t max_unique, float* d_rows, void* ws, hipStream_t s, int* err) {
  if (max_unique == 0 || n_tokens == 0) return hipSuccess;
  const int64_t chunks = (n_tokens + kSegChunk - 1) / kSegChunk;
  float* first = static_cast<float*>(ws);
  float* last = first + chunks * d_ff;
  const unsigned cb = static_cast<unsigned>((d_ff + kSegCols * kSegWaves - 1) / (kSegCols * kSegWaves));
  if (dtype == STAPLE_BF16)
    segsum_chunk_kernel<bf16_t><<<dim3(cb, static_cast<unsigned>(chunks)), dim3(64 * kSegWaves), 0, s>>>(
        static_cast<const bf16_t*>(du), du_ld, du_col, n_tokens, d_ff, sorted_pos, inv, seg_start,
        n_unique, max_unique, d_rows, first, last, err);
  else
    segsum_chunk_kernel<float><<<dim3(cb, static_cast<unsigned>(chunks)), dim3(64 * kSegWaves), 0, s>>>(
        static_cast<const float*>(du), du_ld, du_col, n_tokens, d_ff, sorted_pos, inv, seg_start,
        n_unique, max_unique, d_rows, first, last, err);
  segsum_fixup_kernel<<<dim3(cb, static_cast<unsigned>(chunks)), dim3(64 * kSegWaves), 0, s>>>(
      n_tokens, d_ff, sorted_pos, inv, seg_start, n_unique, max_unique, first, last, d_rows, err);
  return hipGetLastError();
}

// The fixup pass alone, after a chunk pass done elsewhere (the dh GEMM's
// epilogue over sorted positions) into d_rows and the partials at ws.
hipError_t launch_segment_sum_fixup(int64_t n_tokens, int64_t d_ff, const int32_t* sorted_pos,
                                    const int32_t* inv, const int32_t* seg_start,
                                    const int32_t* n_unique, int64_t max_unique, float* d_rows,
                                    void* ws, hipStream_t s, int* err) {
  if (max_unique == 0 || n_tokens == 0) return hipSuccess;
  const int64_t chunks = (n_tokens + kSegChunk - 1) / kSegChunk;
  float* first = static_cast<float*>(ws);
  float* last = first + chunks * d_ff;
  const unsigned cb = static_cast<unsigned>((d_ff + kSegCols * kSegWaves - 1) / (kSegCols * kSegWaves));
  segsum_fixup_kernel<<<dim3(cb, static_cast<unsigned>(chunks)), dim3(64 * kSegWaves), 0, s>>>(
      n_tokens, d_ff, sorted_pos, inv, seg_start, n_unique, max_unique, first, last, d_rows, err);
  return hipGetLastError();
}

}  // namespace staple
