// AdamW step on the touched rows of a token-indexed table, on the device and
// on the host, and the refresh of cached copies of updated rows.
//
// The tables are trained with AdamW and their moments kept in fp32 beside
// the bf16 table, in host memory in the offloaded design (STAPLE Figure 4
// caption: bf16 tables and fp32 AdamW moments in host DRAM; Table 3: peak
// learning rate and weight decay of the table group).  Only the rows of the
// batch's unique IDs are updated: a row absent from the batch keeps its
// parameters and moments, and the bias correction uses the global step.
//
// Per element, in fp32 (decay = 1 - lr wd, step_size = lr / (1 - beta1^t),
// inv_sqrt_bc2 = 1 / sqrt(1 - beta2^t), the last two formed once in double):
//
//   p = p decay;  m = beta1 m + (1 - beta1) g;  v = beta2 v + (1 - beta2) g g
//   p = p - step_size m / (sqrt(v) inv_sqrt_bc2 + eps)
//
// and p is stored back in the table's type (bf16 rounded to nearest even).
#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "common.h"
#include "host_pool.h"

namespace staple {

AdamWConsts adamw_consts(float lr, float beta1, float beta2, float eps, float weight_decay,
                         int64_t step) {
  const double bc1 = 1.0 - std::pow(static_cast<double>(beta1), static_cast<double>(step));
  const double bc2 = 1.0 - std::pow(static_cast<double>(beta2), static_cast<double>(step));
  AdamWConsts c;
  c.decay = static_cast<float>(1.0 - static_cast<double>(lr) * weight_decay);
  c.beta1 = beta1;
  c.one_m_beta1 = static_cast<float>(1.0 - beta1);
  c.beta2 = beta2;
  c.one_m_beta2 = static_cast<float>(1.0 - beta2);
  c.step_size = static_cast<float>(lr / bc1);
  c.inv_sqrt_bc2 = static_cast<float>(1.0 / std::sqrt(bc2));
  c.eps = eps;
  return c;
}

__host__ __device__ __forceinline__ void adamw_element(float& p, float& m, float& v, float g,
                                                       const AdamWConsts& c) {
  p = p * c.decay;
  m = c.beta1 * m + c.one_m_beta1 * g;
  v = c.beta2 * v + c.one_m_beta2 * (g * g);
  p = p - c.step_size * m / (__builtin_sqrtf(v) * c.inv_sqrt_bc2 + c.eps);
}

// ---------------------------------------------------------------------------
// Device: one workgroup per listed row (grid-stride over rows), each thread
// 8 consecutive elements per pass (16-byte bf16 / 32-byte fp32 accesses).
// ---------------------------------------------------------------------------
constexpr int kAdamThreads = 256;

// One 8-element piece of a row: parameters, moments and gradient in fp32.
struct AdamPiece {
  float p[8], m[8], v[8], g[8];
};

template <typename PT>
__device__ __forceinline__ void adam_load(const PT* table, const float* m, const float* v,
                                          const float* grad, int64_t pe, int64_t ge, AdamPiece& x) {
  const float4* mp = reinterpret_cast<const float4*>(m + pe);
  const float4* vp = reinterpret_cast<const float4*>(v + pe);
  const float4* gp = reinterpret_cast<const float4*>(grad + ge);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float4 a = mp[h], b = vp[h], q = gp[h];
    x.m[4 * h] = a.x; x.m[4 * h + 1] = a.y; x.m[4 * h + 2] = a.z; x.m[4 * h + 3] = a.w;
    x.v[4 * h] = b.x; x.v[4 * h + 1] = b.y; x.v[4 * h + 2] = b.z; x.v[4 * h + 3] = b.w;
    x.g[4 * h] = q.x; x.g[4 * h + 1] = q.y; x.g[4 * h + 2] = q.z; x.g[4 * h + 3] = q.w;
  }
  if constexpr (sizeof(PT) == 2) {
    const uint4 raw = *reinterpret_cast<const uint4*>(table + pe);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x.p[2 * i] = __uint_as_float(w[i] << 16);
      x.p[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const float4* pp = reinterpret_cast<const float4*>(table + pe);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float4 a = pp[h];
      x.p[4 * h] = a.x; x.p[4 * h + 1] = a.y; x.p[4 * h + 2] = a.z; x.p[4 * h + 3] = a.w;
    }
  }
}

template <typename PT>
__device__ __forceinline__ void adam_update_store(PT* table, float* m, float* v, int64_t pe,
                                                  AdamPiece& x, const AdamWConsts& c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) adamw_element(x.p[i], x.m[i], x.v[i], x.g[i], c);
  float4* mo = reinterpret_cast<float4*>(m + pe);
  float4* vo = reinterpret_cast<float4*>(v + pe);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    mo[h] = make_float4(x.m[4 * h], x.m[4 * h + 1], x.m[4 * h + 2], x.m[4 * h + 3]);
    vo[h] = make_float4(x.v[4 * h], x.v[4 * h + 1], x.v[4 * h + 2], x.v[4 * h + 3]);
  }
  if constexpr (sizeof(PT) == 2) {
    uint4 o;
    o.x = pack_bf16x2(x.p[0], x.p[1]);
    o.y = pack_bf16x2(x.p[2], x.p[3]);
    o.z = pack_bf16x2(x.p[4], x.p[5]);
    o.w = pack_bf16x2(x.p[6], x.p[7]);
    *reinterpret_cast<uint4*>(table + pe) = o;
  } else {
    float4* po = reinterpret_cast<float4*>(table + pe);
#pragma unroll
    for (int h = 0; h < 2; ++h)
      po[h] = make_float4(x.p[4 * h], x.p[4 * h + 1], x.p[4 * h + 2], x.p[4 * h + 3]);
  }
}

// Two pieces per thread are loaded before either is updated, so each thread
// keeps twice the loads in flight.
template <typename PT>
__global__ __launch_bounds__(kAdamThreads) void adamw_rows_kernel(
    PT* __restrict__ table, float* __restrict__ m, float* __restrict__ v, int64_t vocab,
    int64_t d_ff, const int32_t* __restrict__ rows, const int32_t* __restrict__ n_rows_p,
    int64_t max_rows, const float* __restrict__ grad, AdamWConsts c, int* err) {
  const int64_t n = n_rows_p ? min(static_cast<int64_t>(*n_rows_p), max_rows) : max_rows;
  constexpr int64_t kPass = kAdamThreads * 8;
  for (int64_t k = blockIdx.x; k < n; k += gridDim.x) {
    const int32_t r = rows[k];
    if (r < 0 || r >= vocab) {
      if (threadIdx.x == 0) flag_index_error(err);
      continue;
    }
    const int64_t base = static_cast<int64_t>(r) * d_ff;
    const int64_t gbase = k * d_ff;
    for (int64_t e = static_cast<int64_t>(threadIdx.x) * 8; e < d_ff; e += 2 * kPass) {
      const bool two = e + kPass < d_ff;
      AdamPiece a, b;
      adam_load(table, m, v, grad, base + e, gbase + e, a);
      if (two) adam_load(table, m, v, grad, base + e + kPass, gbase + e + kPass, b);
      adam_update_store(table, m, v, base + e, a, c);
      if (two) adam_update_store(table, m, v, base + e + kPass, b, c);
    }
  }
}

hipError_t launch_adamw_rows(void* table, int dtype, float* m, float* v, int64_t vocab, int64_t d_ff,
                             const int32_t* rows, const int32_t* n_rows, int64_t max_rows,
                             const float* grad, const AdamWConsts& c, hipStream_t s, int* err) {
  if (max_rows == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>(std::min<int64_t>(max_rows, 65535));
  if (dtype == STAPLE_BF16)
    adamw_rows_kernel<uint16_t><<<grid, kAdamThreads, 0, s>>>(static_cast<uint16_t*>(table), m, v, vocab,
                                                              d_ff, rows, n_rows, max_rows, grad, c, err);
  else
    adamw_rows_kernel<float><<<grid, kAdamThreads, 0, s>>>(static_cast<float*>(table), m, v, vocab, d_ff,
                                                           rows, n_rows, max_rows, grad, c, err);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Host: the same update with host threads over rows.  A row is processed in
// 8-element chunks with branch-free bf16 conversions (round to nearest even,
// NaN kept quiet) so the compiler vectorizes it; an AVX2/FMA build of the
// loop is chosen at run time on CPUs that have those instructions.
// ---------------------------------------------------------------------------
typedef float hf8 __attribute__((ext_vector_type(8)));
typedef uint32_t hu8 __attribute__((ext_vector_type(8)));
typedef uint16_t hh8 __attribute__((ext_vector_type(8)));

// 8 elements at a time in vector registers (SSE2: two 4-wide halves; AVX2:
// one 8-wide register), the element update written out in the order of
// adamw_element.
template <bool BF16>
static inline void host_adamw_row(void* __restrict__ prow, float* __restrict__ mr,
                                  float* __restrict__ vr, const float* __restrict__ gr,
                                  int64_t d_ff, const AdamWConsts c) {
  int64_t e = 0;
  for (; e + 8 <= d_ff; e += 8) {
    hf8 p, m, v, g;
    std::memcpy(&m, mr + e, 32);
    std::memcpy(&v, vr + e, 32);
    std::memcpy(&g, gr + e, 32);
    if constexpr (BF16) {
      hh8 b;
      std::memcpy(&b, static_cast<const uint16_t*>(prow) + e, 16);
      p = __builtin_bit_cast(hf8, __builtin_convertvector(b, hu8) << 16);
    } else {
      std::memcpy(&p, static_cast<const float*>(prow) + e, 32);
    }
    p = p * c.decay;
    m = c.beta1 * m + c.one_m_beta1 * g;
    v = c.beta2 * v + c.one_m_beta2 * (g * g);
    p = p - c.step_size * m / (__builtin_elementwise_sqrt(v) * c.inv_sqrt_bc2 + c.eps);
    std::memcpy(mr + e, &m, 32);
    std::memcpy(vr + e, &v, 32);
    if constexpr (BF16) {
      const hu8 u = __builtin_bit_cast(hu8, p);
      const hu8 rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
      const hu8 quiet = (u >> 16) | 0x40u;
      const hu8 out = ((u & 0x7fffffffu) > 0x7f800000u) ? quiet : rounded;
      const hh8 b = __builtin_convertvector(out, hh8);
      std::memcpy(static_cast<uint16_t*>(prow) + e, &b, 16);
    } else {
      std::memcpy(static_cast<float*>(prow) + e, &p, 32);
    }
  }
  for (; e < d_ff; ++e) {
    float p;
    if constexpr (BF16) {
      const uint32_t u = static_cast<uint32_t>(static_cast<const uint16_t*>(prow)[e]) << 16;
      std::memcpy(&p, &u, 4);
    } else {
      p = static_cast<const float*>(prow)[e];
    }
    adamw_element(p, mr[e], vr[e], gr[e], c);
    if constexpr (BF16) {
      uint32_t u;
      std::memcpy(&u, &p, 4);
      const bool nan = (u & 0x7fffffffu) > 0x7f800000u;
      static_cast<uint16_t*>(prow)[e] =
          static_cast<uint16_t>(nan ? ((u >> 16) | 0x40u) : ((u + 0x7fffu + ((u >> 16) & 1u)) >> 16));
    } else {
      static_cast<float*>(prow)[e] = p;
    }
  }
}

static void host_adamw_range(void* table, int dtype, float* m, float* v, int64_t d_ff,
                             const int32_t* rows, const float* grad, const AdamWConsts& c,
                             int64_t lo, int64_t hi) {
  for (int64_t k = lo; k < hi; ++k) {
    const int64_t base = static_cast<int64_t>(rows[k]) * d_ff;
    if (dtype == STAPLE_BF16)
      host_adamw_row<true>(static_cast<uint16_t*>(table) + base, m + base, v + base, grad + k * d_ff,
                           d_ff, c);
    else
      host_adamw_row<false>(static_cast<float*>(table) + base, m + base, v + base, grad + k * d_ff,
                            d_ff, c);
  }
}

__attribute__((target("avx2,fma"))) static void host_adamw_range_avx2(
    void* table, int dtype, float* m, float* v, int64_t d_ff, const int32_t* rows,
    const float* grad, const AdamWConsts& c, int64_t lo, int64_t hi) {
  for (int64_t k = lo; k < hi; ++k) {
    const int64_t base = static_cast<int64_t>(rows[k]) * d_ff;
    if (dtype == STAPLE_BF16)
      host_adamw_row<true>(static_cast<uint16_t*>(table) + base, m + base, v + base, grad + k * d_ff,
                           d_ff, c);
    else
      host_adamw_row<false>(static_cast<float*>(table) + base, m + base, v + base, grad + k * d_ff,
                            d_ff, c);
  }
}

void host_adamw_rows(void* table, int dtype, float* m, float* v, int64_t d_ff, const int32_t* rows,
                     int64_t n_rows, const float* grad, const AdamWConsts& c, int n_threads) {
  const bool avx2 = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma");
  auto run = [&](int64_t lo, int64_t hi) {
    if (avx2) host_adamw_range_avx2(table, dtype, m, v, d_ff, rows, grad, c, lo, hi);
    else host_adamw_range(table, dtype, m, v, d_ff, rows, grad, c, lo, hi);
  };
  const int64_t nt = std::max<int64_t>(1, std::min<int64_t>(n_threads, n_rows));
  host_parallel_for(n_rows, static_cast<int>(std::min<int64_t>(nt, kHostPoolMax)), run);
}

// ---------------------------------------------------------------------------
// Cache refresh: cache_rows[code[u]] = table[uniq[u]] for every u < n with
// code[u] >= 0 (the cached rows among those just updated).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void cache_refresh_kernel(
    const void* __restrict__ table, int64_t vocab, const int32_t* __restrict__ uniq,
    const int32_t* __restrict__ code, const int32_t* __restrict__ n_unique_p, int64_t max_unique,
    int64_t row_bytes, void* __restrict__ cache_rows, int64_t capacity, int* err) {
  const int64_t n = min(static_cast<int64_t>(*n_unique_p), max_unique);
  for (int64_t u = blockIdx.x; u < n; u += gridDim.x) {
    const int32_t c = code[u];
    if (c < 0) continue;
    const int32_t id = uniq[u];
    if (c >= capacity || id < 0 || id >= vocab) {
      if (threadIdx.x == 0) flag_index_error(err);
      continue;
    }
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(table) + id * row_bytes);
    uint4* dst = reinterpret_cast<uint4*>(static_cast<char*>(cache_rows) + c * row_bytes);
    for (int64_t i = threadIdx.x; i < row_bytes / 16; i += 256) dst[i] = src[i];
  }
}

hipError_t launch_cache_refresh(const void* table, int64_t vocab, const int32_t* uniq,
                                const int32_t* code, const int32_t* n_unique, int64_t max_unique,
                                int64_t row_bytes, void* cache_rows, int64_t capacity, hipStream_t s,
                                int* err, unsigned max_workgroups) {
  if (max_unique == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>(
      max_workgroups > 0 && max_unique > max_workgroups ? max_workgroups : std::min<int64_t>(max_unique, 65535));
  cache_refresh_kernel<<<grid, 256, 0, s>>>(table, vocab, uniq, code, n_unique, max_unique, row_bytes,
                                            cache_rows, capacity, err);
  return hipGetLastError();
}

}  // namespace staple

// ---------------------------------------------------------------------------
// Host update overlapped with the GPU: the gradient rows come to the host in
// chunks on a copy stream as soon as the backward has formed them (an event
// recorded right after the table-row segment sum), and a worker thread of
// the update updates each chunk with the library's host threads as it lands,
// while the GPU goes on with the rest of the backward.  The rows are updated
// by the same routine as staple_adamw_rows_host, each row once and
// independently, so the result is the same bits as the serial update.
// ---------------------------------------------------------------------------
#include <condition_variable>
#include <mutex>
#include <new>

#include "dma.h"

using staple::SdmaCopier;

struct staple_host_adamw {
  static constexpr int kChunks = 8;
  // workgroups of one refresh launch: the rows come over PCIe, and 16
  // workgroups keep enough reads in flight while leaving nearly every CU to
  // the backward's GEMMs running beside them
  static constexpr unsigned kRefreshWorkgroups = 16;
  int device = 0;
  int64_t max_rows = 0, d_ff = 0;
  float* grad_host = nullptr;      // pinned [max_rows x d_ff]
  int32_t* meta_host = nullptr;    // pinned [1 + max_rows]: the row count, then the row IDs
  hipEvent_t ev_rows = nullptr, ev_meta = nullptr, ev_done = nullptr;
  hipEvent_t ev_chunk[kChunks] = {};
  SdmaCopier sdma;                 // the gradient chunks' copies, when available
  std::thread worker;
  std::mutex mu;
  std::condition_variable cv;
  bool job = false, busy = false, quit = false;
  staple_status_t result = STAPLE_OK;
  // the current job
  void* table = nullptr;
  float* m = nullptr;
  float* v = nullptr;
  int64_t vocab = 0;
  int dtype = STAPLE_BF16;
  const float* grad_dev = nullptr;
  const int32_t* uniq_dev = nullptr;
  const int32_t* n_unique_dev = nullptr;
  const int32_t* code = nullptr;   // NULL: no cache refresh
  void* cache_rows = nullptr;
  int64_t capacity = 0;
  int* err = nullptr;
  hipStream_t copy = nullptr;
  staple::AdamWConsts c{};
  int n_threads = 0;

  // ev_done is recorded on the copy stream whatever the outcome, so that
  // finish orders the caller's stream after every refresh launched, also
  // when the job stopped part way.
  staple_status_t run_job() {
    if (hipSetDevice(device) != hipSuccess) return STAPLE_ERR_HIP;
    const staple_status_t r = run_job_steps();
    const bool rec = hipEventRecord(ev_done, copy) == hipSuccess;
    return r == STAPLE_OK && !rec ? STAPLE_ERR_HIP : r;
  }

  staple_status_t run_job_steps() {
    if (sdma.ready) {
      // the row count and IDs on the DMA engines as soon as the rows are
      // complete (a copy kernel could wait behind the GEMMs for a CU)
      if (hipEventSynchronize(ev_rows) != hipSuccess) return STAPLE_ERR_HIP;
      const bool a = sdma.start_d2h(kChunks, meta_host, n_unique_dev, sizeof(int32_t));
      const bool b = a && sdma.start_d2h(kChunks + 1, meta_host + 1, uniq_dev,
                                     static_cast<size_t>(max_rows) * sizeof(int32_t));
      const bool wa = a && sdma.wait(kChunks);
      const bool wb = b && sdma.wait(kChunks + 1);
      if (!(wa && wb)) return STAPLE_ERR_HIP;
    } else if (hipEventSynchronize(ev_meta) != hipSuccess) {
      return STAPLE_ERR_HIP;
    }
    const int64_t n = meta_host[0];
    if (n < 0 || n > max_rows) return STAPLE_ERR_INDEX_RANGE;
    if (n == 0) return STAPLE_OK;
    const int32_t* ids = meta_host + 1;
    for (int64_t k = 0; k < n; ++k)
      if (ids[k] < 0 || ids[k] >= vocab) return STAPLE_ERR_HOST;
    const int parts = static_cast<int>(std::min<int64_t>(kChunks, n));
    // the rows are complete (ev_rows, or ev_meta after it on the copy stream)
    for (int p = 0; p < parts; ++p) {
      const int64_t lo = n * p / parts, hi = n * (p + 1) / parts;
      const size_t bytes = static_cast<size_t>(hi - lo) * d_ff * sizeof(float);
      if (sdma.ready) {
        if (!sdma.start_d2h(p, grad_host + lo * d_ff, grad_dev + lo * d_ff, bytes)) {
          for (int q = 0; q < p; ++q) (void)sdma.wait(q);   // none left writing the staging
          return STAPLE_ERR_HIP;
        }
      } else if (hipMemcpyAsync(grad_host + lo * d_ff, grad_dev + lo * d_ff, bytes,
                                hipMemcpyDeviceToHost, copy) != hipSuccess ||
                 hipEventRecord(ev_chunk[p], copy) != hipSuccess) {
        (void)hipStreamSynchronize(copy);
        return STAPLE_ERR_HIP;
      }
    }
    for (int p = 0; p < parts; ++p) {
      const int64_t lo = n * p / parts, hi = n * (p + 1) / parts;
      if (sdma.ready ? !sdma.wait(p) : hipEventSynchronize(ev_chunk[p]) != hipSuccess) {
        for (int q = p + 1; q < parts; ++q) {
          if (sdma.ready) (void)sdma.wait(q);
          else (void)hipEventSynchronize(ev_chunk[q]);
        }
        return STAPLE_ERR_HIP;
      }
      staple::host_adamw_rows(table, dtype, m, v, d_ff, ids + lo, hi - lo, grad_host + lo * d_ff, c,
                              n_threads);
      // the cached copies of this chunk's rows, read from the updated host
      // table while the next chunk is updated (*n_unique >= hi, so the
      // launch's row count is hi - lo)
      if (code && capacity > 0 &&
          staple::launch_cache_refresh(table, vocab, uniq_dev + lo, code + lo, n_unique_dev, hi - lo,
                                       d_ff * (dtype == STAPLE_BF16 ? 2 : 4), cache_rows, capacity,
                                       copy, err, kRefreshWorkgroups) != hipSuccess)
        return STAPLE_ERR_HIP;
    }
    return STAPLE_OK;
  }

  void loop() {
    std::unique_lock<std::mutex> lk(mu);
    for (;;) {
      cv.wait(lk, [&] { return job || quit; });
      if (quit) return;
      job = false;
      lk.unlock();
      const staple_status_t r = run_job();
      lk.lock();
      result = r;
      busy = false;
      cv.notify_all();
    }
  }
};

using namespace staple;

// The worker sleeps while it waits for a copy (blocking-sync events) rather
// than spinning on a core the update's threads could use.
constexpr unsigned kWaitFlags = hipEventDisableTiming | hipEventBlockingSync;

extern "C" {

staple_status_t staple_host_adamw_create(int64_t max_rows, int64_t d_ff, staple_host_adamw_t** out) {
  if (!out || max_rows < 1 || max_rows > 0x7fffffffll || d_ff <= 0) return STAPLE_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  staple_host_adamw_t* h = new (std::nothrow) staple_host_adamw_t();
  if (!h) return STAPLE_ERR_HOST;
  h->max_rows = max_rows;
  h->d_ff = d_ff;
  bool ok = hipGetDevice(&h->device) == hipSuccess &&
            hipHostMalloc(reinterpret_cast<void**>(&h->grad_host),
                          static_cast<size_t>(max_rows) * d_ff * sizeof(float), hipHostMallocDefault) == hipSuccess &&
            hipHostMalloc(reinterpret_cast<void**>(&h->meta_host),
                          static_cast<size_t>(max_rows + 1) * sizeof(int32_t), hipHostMallocDefault) == hipSuccess &&
            hipEventCreateWithFlags(&h->ev_rows, kWaitFlags) == hipSuccess &&
            hipEventCreateWithFlags(&h->ev_meta, kWaitFlags) == hipSuccess &&
            hipEventCreateWithFlags(&h->ev_done, hipEventDisableTiming) == hipSuccess;
  for (int p = 0; ok && p < staple_host_adamw_t::kChunks; ++p)
    ok = hipEventCreateWithFlags(&h->ev_chunk[p], kWaitFlags) == hipSuccess;
  if (ok) h->sdma.init(h->device, staple_host_adamw_t::kChunks + 2);   // chunks, count, IDs
  if (ok) {
    try {
      h->worker = std::thread(&staple_host_adamw_t::loop, h);
    } catch (...) {
      ok = false;
    }
  }
  if (!ok) {
    staple_host_adamw_destroy(h);
    return STAPLE_ERR_HIP;
  }
  *out = h;
  return STAPLE_OK;
}

void* staple_host_adamw_event(staple_host_adamw_t* h) { return h ? h->ev_rows : nullptr; }

staple_status_t staple_host_adamw_start(staple_host_adamw_t* h, void* table, float* m, float* v,
                                        int64_t vocab, int32_t dtype, const int32_t* uniq,
                                        const int32_t* n_unique, const float* grad, float lr,
                                        float beta1, float beta2, float eps, float weight_decay,
                                        int64_t step, int32_t n_threads, const int32_t* code,
                                        void* cache_rows, int64_t capacity, void* copy_stream) {
  if (!h || !table || !m || !v || !uniq || !n_unique || !grad || vocab < 1 || capacity < 0 ||
      (dtype != STAPLE_BF16 && dtype != STAPLE_F32))
    return STAPLE_ERR_INVALID_ARGUMENT;
  const int64_t row_bytes = h->d_ff * (dtype == STAPLE_BF16 ? 2 : 4);
  int* err = nullptr;
  if (code && capacity > 0) {
    // the refresh kernels read the host table: it must be pinned
    hipPointerAttribute_t attr{};
    if (!cache_rows || row_bytes % 16 != 0 || reinterpret_cast<uintptr_t>(table) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(cache_rows) % 16 != 0)
      return STAPLE_ERR_INVALID_ARGUMENT;
    if (hipPointerGetAttributes(&attr, table) != hipSuccess) {
      (void)hipGetLastError();
      return STAPLE_ERR_INVALID_ARGUMENT;
    }
    if (attr.type != hipMemoryTypeHost) return STAPLE_ERR_INVALID_ARGUMENT;
    err = device_error_word();
    if (!err) return STAPLE_ERR_HIP;
  }
  if (!(step >= 1 && std::isfinite(lr) && lr >= 0.0f && beta1 >= 0.0f && beta1 < 1.0f &&
        beta2 >= 0.0f && beta2 < 1.0f && std::isfinite(eps) && eps >= 0.0f &&
        std::isfinite(weight_decay) && weight_decay >= 0.0f))
    return STAPLE_ERR_INVALID_ARGUMENT;
  std::unique_lock<std::mutex> lk(h->mu);
  if (h->busy) return STAPLE_ERR_INVALID_ARGUMENT;   // the previous update was not finished
  hipStream_t cs = static_cast<hipStream_t>(copy_stream);
  // the copy stream carries the refreshes (and, without the DMA engines, the
  // copies): nothing on it before the rows are complete
  if (hipStreamWaitEvent(cs, h->ev_rows, 0) != hipSuccess) return STAPLE_ERR_HIP;
  if (!h->sdma.ready &&
      (hipMemcpyAsync(h->meta_host, n_unique, sizeof(int32_t), hipMemcpyDeviceToHost, cs) != hipSuccess ||
       hipMemcpyAsync(h->meta_host + 1, uniq, static_cast<size_t>(h->max_rows) * sizeof(int32_t),
                      hipMemcpyDeviceToHost, cs) != hipSuccess ||
       hipEventRecord(h->ev_meta, cs) != hipSuccess))
    return STAPLE_ERR_HIP;
  h->table = table;
  h->m = m;
  h->v = v;
  h->vocab = vocab;
  h->dtype = dtype;
  h->grad_dev = grad;
  h->uniq_dev = uniq;
  h->n_unique_dev = n_unique;
  h->code = capacity > 0 ? code : nullptr;
  h->cache_rows = cache_rows;
  h->capacity = capacity;
  h->err = err;
  h->copy = cs;
  h->c = adamw_consts(lr, beta1, beta2, eps, weight_decay, step);
  // by default two threads fewer than the pool's maximum: the caller's
  // thread keeps feeding the GPU meanwhile
  const int hw = static_cast<int>(std::max(1u, std::thread::hardware_concurrency()));
  h->n_threads = n_threads > 0 ? n_threads : std::max(1, std::min(hw, kHostPoolMax) - 2);
  h->result = STAPLE_OK;
  h->busy = true;
  h->job = true;
  h->cv.notify_all();
  return STAPLE_OK;
}

staple_status_t staple_host_adamw_finish(staple_host_adamw_t* h, void* stream) {
  if (!h) return STAPLE_ERR_INVALID_ARGUMENT;
  std::unique_lock<std::mutex> lk(h->mu);
  h->cv.wait(lk, [&] { return !h->busy; });
  // also after a failed job: its refreshes may still be running
  if (hipStreamWaitEvent(static_cast<hipStream_t>(stream), h->ev_done, 0) != hipSuccess &&
      h->result == STAPLE_OK)
    return STAPLE_ERR_HIP;
  return h->result;
}

void staple_host_adamw_destroy(staple_host_adamw_t* h) {
  if (!h) return;
  if (h->worker.joinable()) {
    {
      std::unique_lock<std::mutex> lk(h->mu);
      h->cv.wait(lk, [&] { return !h->busy; });
      h->quit = true;
      h->cv.notify_all();
    }
    h->worker.join();
  }
  for (int p = 0; p < staple_host_adamw_t::kChunks; ++p)
    if (h->ev_chunk[p]) (void)hipEventDestroy(h->ev_chunk[p]);
  h->sdma.release();
  if (h->ev_meta) (void)hipEventDestroy(h->ev_meta);
  if (h->ev_done) (void)hipEventDestroy(h->ev_done);
  if (h->ev_rows) (void)hipEventDestroy(h->ev_rows);
  if (h->meta_host) (void)hipHostFree(h->meta_host);
  if (h->grad_host) (void)hipHostFree(h->grad_host);
  delete h;
}

}  // extern "C"
