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
