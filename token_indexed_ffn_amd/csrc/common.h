// Shared device/host helpers of libstaple (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <atomic>

#include "../../include/staple.h"

namespace staple {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

// Pointers into LDS (local address space), e.g. for loads straight from
// global memory into LDS.
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;

// vmcnt wait with the other counters left alone (gfx9 encoding: vmcnt bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Compute units of the current device, looked up once per device (256 when
// the query fails).
inline int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Workgroup barrier for LDS pipelines whose global->LDS loads are counted by
// hand: this wave's LDS reads have completed, then s_barrier, with compiler
// fences on both sides so no memory access moves across it.  Unlike
// __syncthreads() it does not wait for outstanding global loads.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4));   // lgkmcnt(0) only
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// bfloat16 storage type (raw bits).
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Two floats -> two bfloat16 (lo in bits 0-15), rounded to nearest with ties
// to even (NaN stays NaN), by gfx950's packed conversion (one
// v_cvt_pk_bf16_f32 per pair instead of an integer rounding sequence per
// element).
typedef float cvt_f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 cvt_bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const cvt_f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, cvt_bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return static_cast<uint16_t>(pack_bf16x2(f, 0.0f));
}

// Element access for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static float load(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  __device__ __forceinline__ static void store(void* p, int64_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
  // value as it would be stored (identity for fp32)
  __device__ __forceinline__ static float quantize(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static float load(const void* p, int64_t i) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  }
  __device__ __forceinline__ static void store(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
  }
  __device__ __forceinline__ static float quantize(float v) { return bf16_to_f32(f32_to_bf16(v)); }
};

// 1 / (1 + e^-z) with the hardware exponential and reciprocal (v_rcp_f32,
// about 1 ulp) rather than an IEEE division.
__device__ __forceinline__ float sigmoidf_(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Kernels that meet an out-of-range ID or index OR this bit into the
// per-device error word whose address they receive as `err`.
constexpr int kErrIndexRange = 1;

__device__ __forceinline__ void flag_index_error(int* err) { atomicOr(err, kErrIndexRange); }

// Address of the calling device's error word (defined in api.hip).
int* device_error_word();

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Sorted positions per chunk of the table-row gradient's segment sum (its
// chunk pass and the dh GEMM epilogue that can do that pass share it).
constexpr int kSegChunk = 32;

// Bump allocator over a caller-provided workspace.
struct Workspace {
  char* base;
  size_t size;
  size_t used;
  Workspace(void* b, size_t s) : base(static_cast<char*>(b)), size(s), used(0) {}
  template <typename P> P* take(size_t bytes) {
    size_t off = align_up(used, 256);
    used = off + bytes;
    return used <= size ? reinterpret_cast<P*>(base + off) : nullptr;
  }
};

}  // namespace staple

#define STAPLE_HIP_CHECK(expr)                          \
  do {                                                  \
    hipError_t _e = (expr);                             \
    if (_e != hipSuccess) return STAPLE_ERR_HIP;        \
  } while (0)

// Constants of one AdamW step (optim.hip): decay = 1 - lr wd,
// step_size = lr / (1 - beta1^t), inv_sqrt_bc2 = 1 / sqrt(1 - beta2^t).
namespace staple {
struct AdamWConsts {
  float decay, beta1, one_m_beta1, beta2, one_m_beta2, step_size, inv_sqrt_bc2, eps;
};

// Per-layer row sources of a multi-layer row assembly (passed by value as a
// kernel argument; a longer stack is assembled in slices of this many layers).
constexpr int kMaxAssembleLayers = 32;
constexpr unsigned kLayerRowWorkgroups = 512;
struct LayerRowSources {
  const void* cache_rows[kMaxAssembleLayers];
  const void* table[kMaxAssembleLayers];
  int64_t table_ld[kMaxAssembleLayers];   // bytes between consecutive token rows of the table
  void* rows[kMaxAssembleLayers];
};

// Compact-row copies carried by a decode gate/up launch (a copy wave per
// workgroup, see decode.hip): for each of n_layers layers j and the unique
// rows u = part, part + parts, ... below U = *n_unique,
// rows[j][u] = code[u] >= 0 ? cache_rows[j][code[u]] : table[j][uniq[u]].
constexpr int kCopyJobLayers = 4;
struct RowCopyJob {
  const void* cache_rows[kCopyJobLayers];
  const void* table[kCopyJobLayers];
  int64_t table_ld[kCopyJobLayers];       // bytes between consecutive token rows of table j
  void* rows[kCopyJobLayers];
  const int32_t* uniq;
  const int32_t* code;
  const int32_t* n_unique;
  int64_t max_unique, capacity, vocab, row_bytes;
  int n_layers, part, parts;
  // this launch's rows: unique rows u = part + parts i (i = 0, 1, ...) below
  // *n_unique, each for the n_layers layers; rows_max of them at most, each
  // cut into `per` segments of at most `seg` 16-byte pieces
  int rows_max, per, seg;
};
}  // namespace staple

#define STAPLE_LAUNCH_CHECK()                           \
  do {                                                  \
    hipError_t _e = hipGetLastError();                  \
    if (_e != hipSuccess) return STAPLE_ERR_HIP;        \
  } while (0)
