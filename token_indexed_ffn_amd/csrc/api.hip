// C ABI of libstaple: argument validation, workspace sizing and dispatch to
// the kernels.  Nothing here allocates device memory.
#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>
#include <cmath>
#include <thread>
#include <vector>

#include "common.h"
#include "dma.h"
#include "host_pool.h"

namespace staple {

// kernels (sort.hip)
size_t dedup_workspace_bytes(int64_t n);
hipError_t launch_dedup(const int32_t* ids, int64_t n, int64_t vocab, int32_t* uniq, int32_t* inv,
                        int32_t* sorted_pos, int32_t* seg_start, int32_t* n_unique, void* ws,
                        hipStream_t s, int* err);
hipError_t launch_dedup_lookup_wave(const int32_t* ids, int64_t n, int64_t vocab,
                                    const int32_t* id_to_slot, int32_t* uniq, int32_t* inv,
                                    int32_t* sorted_pos, int32_t* seg_start, int32_t* n_unique,
                                    int32_t* code, int32_t* miss_uidx, int32_t* n_miss,
                                    int32_t* row_src, hipStream_t s, int* err);
size_t cache_build_workspace_bytes(int64_t vocab);
hipError_t launch_cache_build(const int64_t* counts, int64_t vocab, int64_t capacity,
                              int32_t* id_to_slot, int32_t* slot_to_id, void* ws, hipStream_t s,
                              int* err);
// kernels (rows.hip)
hipError_t launch_cache_count(const int32_t* ids, int64_t n, int64_t vocab, int64_t* counts,
                              hipStream_t s, int* err);
hipError_t launch_split_tokens(const int32_t* inv, int64_t n, const int32_t* code,
                               const int32_t* n_unique, int64_t max_unique, int32_t* hit_pos,
                               int32_t* miss_pos, int32_t* tok_row, int32_t* counts, hipStream_t s,
                               int* err);
hipError_t launch_cache_lookup(const int32_t* uniq, const int32_t* n_unique, int64_t max_unique,
                               const int32_t* id_to_slot, int64_t vocab, int32_t* code,
                               int32_t* miss_uidx, int32_t* miss_ids, int32_t* n_miss,
                               hipStream_t s, int* err, const int32_t* inv = nullptr,
                               int64_t n_tokens = 0, int32_t* row_src = nullptr);
hipError_t launch_gather_rows(const void* src, int64_t src_rows, const int32_t* index,
                              const int32_t* n_rows, int64_t max_rows, int64_t row_bytes,
                              void* dst, hipStream_t s, int* err, unsigned max_workgroups);
hipError_t launch_assemble_rows(const void* cache_rows, int64_t capacity, const void* miss_rows,
                                int64_t max_miss, const int32_t* code, const int32_t* n_unique,
                                int64_t max_unique, int64_t row_bytes, void* rows, hipStream_t s,
                                int* err);
hipError_t launch_assemble_rows_table(const void* cache_rows, int64_t capacity, const void* table,
                                      int64_t vocab, const int32_t* uniq, const int32_t* code,
                                      const int32_t* n_unique, int64_t max_unique,
                                      int64_t row_bytes, void* rows, hipStream_t s, int* err,
                                      unsigned max_workgroups);
hipError_t launch_assemble_rows_layers(const LayerRowSources& src, int n_layers, int64_t capacity,
                                       int64_t vocab, const int32_t* uniq, const int32_t* code,
                                       const int32_t* n_unique, int64_t max_unique,
                                       int64_t row_bytes, hipStream_t s, int* err,
                                       unsigned max_workgroups = kLayerRowWorkgroups);
size_t segment_sum_workspace_bytes(int64_t n_tokens, int64_t d_ff);
hipError_t launch_segment_sum_fixup(int64_t n_tokens, int64_t d_ff, const int32_t* sorted_pos,
                                    const int32_t* inv, const int32_t* seg_start,
                                    const int32_t* n_unique, int64_t max_unique, float* d_rows,
                                    void* ws, hipStream_t s, int* err);
hipError_t dh_seg_kt(int64_t n, int64_t d, int64_t f, const void* dy, const void* wd_t,
                     const void* g, const void* u, void* dgu, const int32_t* sorted_pos,
                     const int32_t* inv, const int32_t* seg_start, const int32_t* n_unique,
                     int64_t max_unique, float* d_rows, float* first, float* last, hipStream_t s,
                     int* err);
hipError_t launch_segment_sum(int dtype, const void* du, int64_t du_ld, int64_t du_col,
                              int64_t n_tokens, int64_t d_ff, const int32_t* sorted_pos,
                              const int32_t* inv, const int32_t* seg_start,
                              const int32_t* n_unique,
                              int64_t max_unique, float* d_rows, void* ws, hipStream_t s, int* err);
// kernels (gemm.hip)
template <typename T>
hipError_t gateup_fwd(int64_t n_sel, const int32_t* pos, int64_t n_tokens, int64_t d, int64_t f,
                      const void* x, const void* wg, const void* wu, const void* rows,
                      int64_t n_rows, const int32_t* row_index, void* h, void* g_out, void* u_out,
                      hipStream_t s, int* err);
template <typename T>
hipError_t down_fwd(int64_t n, int64_t d, int64_t f, const void* h, const void* wd, void* y,
                    int out_dtype, hipStream_t s);
template <typename T>
hipError_t dh_act(int64_t n, int64_t d, int64_t f, const void* dy, const void* wd, const void* g,
                  const void* u, void* dgu, float* du32, hipStream_t s);
template <typename T>
hipError_t recompute_h(int64_t n, int64_t f, const void* g, const void* u, void* h, hipStream_t s);
template <typename T>
hipError_t lowrank_expand(int64_t max_rows, const int32_t* n_dev, int64_t r, int64_t f,
                          const void* rows_r, const void* proj, void* z, hipStream_t s);
template <typename T>
hipError_t lowrank_bwd(int64_t max_rows, const int32_t* n_dev, int64_t r, int64_t f,
                       const float* dz, const void* rows_r, const void* proj, float* d_rows_r,
                       float* d_proj, void* ws, hipStream_t s);
template <typename T>
hipError_t dx_bwd(int64_t n, int64_t d, int64_t f, const void* dgu, const void* wg,
                  const void* wu, void* dx, int out_dtype, hipStream_t s);
template <typename T>
hipError_t dwdown_bwd(int64_t n, int64_t d, int64_t f, const void* dy, const void* h, float* dwd,
                      hipStream_t s);
template <typename T>
hipError_t dwgu_bwd(int64_t n, int64_t d, int64_t f, const void* dgu, const void* x, float* dwg,
                    float* dwu, bool freeze_up, hipStream_t s);
hipError_t transpose_bf16(const void* src, int64_t rows, int64_t cols, int64_t ld_src, void* dst,
                          int64_t dst_cols, int64_t ld_dst, hipStream_t s);
hipError_t dh_act_kt(int64_t n, int64_t d, int64_t f, const void* dy, const void* wd_t,
                     const void* g, const void* u, void* dgu, float* du32, hipStream_t s);
hipError_t dx_bwd_kt(int64_t n, int64_t d, int64_t k, const void* dgu, int64_t ld_dgu,
                     const void* w_t, void* dx, int out_dtype, hipStream_t s);
hipError_t dwdown_bwd_kt(int64_t n, int64_t d, int64_t f, const void* dy_t, int64_t ld_t,
                         const void* h, float* dwd, hipStream_t s);
hipError_t dwgu_bwd_kt(int64_t n, int64_t d, int64_t f, const void* x_t, int64_t ld_t,
                       const void* dgu, float* dwg, float* dwu, bool freeze_up, hipStream_t s);

// kernels (decode.hip)
bool decode_eligible(int64_t n, int64_t d, int64_t f, int dtype);
size_t decode_down_workspace_bytes(int64_t n, int64_t d);
hipError_t decode_gateup(int64_t n, const int32_t* pos, int64_t n_tokens, int64_t d, int64_t f,
                         const void* x, const void* wg, const void* wu, const void* rows,
                         int64_t n_rows, const int32_t* row_index, void* h, void* g_out,
                         void* u_out, hipStream_t s, int* err, bool packed, bool up,
                         const void* table = nullptr, int64_t vocab = 0, int64_t table_ld = 0,
                         const RowCopyJob* job = nullptr);
bool decode_copy_plan(int64_t rows, int64_t f, bool up, int* per, int* seg);
hipError_t decode_down(int64_t n, int64_t d, int64_t f, const void* h, const void* wd, void* y,
                       int out_dtype, void* ws, hipStream_t s, bool packed);
hipError_t decode_pack(int64_t d, int64_t f, const void* wg, const void* wu, const void* wd,
                       void* packed_gu, void* packed_down, hipStream_t s);

// kernels (optim.hip)
AdamWConsts adamw_consts(float lr, float beta1, float beta2, float eps, float weight_decay,
                         int64_t step);
hipError_t launch_adamw_rows(void* table, int dtype, float* m, float* v, int64_t vocab, int64_t d_ff,
                             const int32_t* rows, const int32_t* n_rows, int64_t max_rows,
                             const float* grad, const AdamWConsts& c, hipStream_t s, int* err);
void host_adamw_rows(void* table, int dtype, float* m, float* v, int64_t d_ff, const int32_t* rows,
                     int64_t n_rows, const float* grad, const AdamWConsts& c, int n_threads);
hipError_t launch_cache_refresh(const void* table, int64_t vocab, const int32_t* uniq,
                                const int32_t* code, const int32_t* n_unique, int64_t max_unique,
                                int64_t row_bytes, void* cache_rows, int64_t capacity, hipStream_t s,
                                int* err, unsigned max_workgroups);

// ---------------------------------------------------------------------------
// Per-device error word
// ---------------------------------------------------------------------------
__device__ int g_staple_error = 0;

static std::mutex g_err_mu;
static std::vector<int*> g_err_ptr;  // indexed by device ordinal

int* device_error_word() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
  std::lock_guard<std::mutex> lk(g_err_mu);
  if (static_cast<size_t>(dev) >= g_err_ptr.size()) g_err_ptr.resize(dev + 1, nullptr);
  if (g_err_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_staple_error)) != hipSuccess) return nullptr;
    g_err_ptr[dev] = static_cast<int*>(p);
  }
  return g_err_ptr[dev];
}

// Fixed device scratch of staple_ffn_fwd_packed_noalloc: h (when the caller
// keeps none) and the split-K partial sums of the decode down-projection.
// Every GPU the library runs on holds its own copy until the process ends.
// In host code `scratch` only names the symbol: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

static std::mutex g_scratch_mu;
static std::vector<void*> g_scratch_ptr;  // indexed by device ordinal

static void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (static_cast<size_t>(dev) >= g_scratch_ptr.size()) g_scratch_ptr.resize(dev + 1, nullptr);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

static inline int elem_bytes(int32_t dt) { return dt == STAPLE_BF16 ? 2 : 4; }
static inline bool valid_dtype(int32_t dt) { return dt == STAPLE_BF16 || dt == STAPLE_F32; }
static inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// True when kernels can address `p`: device memory, or pinned (registered or
// hipHostMalloc'd) host memory.  Pageable host memory is refused on the host
// instead of faulting in a kernel.  A failed query leaves no error behind.
static bool device_addressable(const void* p) {
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeHost ||
         attr.type == hipMemoryTypeManaged;
}
// Pinned host memory (a row copy from it reads over PCIe).
static bool host_memory(const void* p) {
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return attr.type == hipMemoryTypeHost;
}
// Workgroups of a row copy that reads host memory: enough loads in flight for
// PCIe (64 x 16 KB), few enough to leave room beside a concurrent kernel.
constexpr unsigned kHostCopyWorkgroups = 64;
static unsigned copy_workgroups(const void* src) { return host_memory(src) ? kHostCopyWorkgroups : 0; }

static inline hipStream_t S(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace staple

using namespace staple;

#define REQUIRE(cond)                                   \
  do {                                                  \
    if (!(cond)) return STAPLE_ERR_INVALID_ARGUMENT;    \
  } while (0)

#define HIPCALL(expr)                                   \
  do {                                                  \
    if ((expr) != hipSuccess) return STAPLE_ERR_HIP;    \
  } while (0)

#define GET_ERR(var)                                    \
  int* var = device_error_word();                       \
  if (var == nullptr) return STAPLE_ERR_HIP

extern "C" {

const char* staple_status_string(staple_status_t st) {
  switch (st) {
    case STAPLE_OK: return "ok";
    case STAPLE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case STAPLE_ERR_UNSUPPORTED: return "unsupported dtype or shape";
    case STAPLE_ERR_WORKSPACE: return "workspace too small";
    case STAPLE_ERR_HIP: return "HIP runtime error";
    case STAPLE_ERR_INDEX_RANGE: return "out-of-range token ID or row index met on the device";
    case STAPLE_ERR_HOST: return "host-side failure";
    case STAPLE_ERR_SCRATCH_LIMIT:
      return "problem larger than the fixed device scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

const char* staple_version(void) { return "libstaple 0.1 (gfx950)"; }

staple_status_t staple_get_device_error(void* stream) {
  GET_ERR(err);
  int v = 0;
  HIPCALL(hipMemcpyAsync(&v, err, sizeof(int), hipMemcpyDeviceToHost, S(stream)));
  HIPCALL(hipStreamSynchronize(S(stream)));
  if (v != 0) {
    int zero = 0;
    HIPCALL(hipMemcpyAsync(err, &zero, sizeof(int), hipMemcpyHostToDevice, S(stream)));
    HIPCALL(hipStreamSynchronize(S(stream)));
    return STAPLE_ERR_INDEX_RANGE;
  }
  return STAPLE_OK;
}

// ------------------------------------------------------------------ dedup
size_t staple_dedup_workspace_bytes(int64_t n_tokens) {
  return n_tokens < 0 ? 0 : dedup_workspace_bytes(n_tokens);
}

staple_status_t staple_dedup(const int32_t* ids, int64_t n, int64_t vocab, int32_t* uniq,
                             int32_t* inv, int32_t* sorted_pos, int32_t* seg_start,
                             int32_t* n_unique, void* ws, size_t ws_bytes, void* stream) {
  REQUIRE(n >= 0 && n <= 0x7fffffffll && vocab >= 1 && vocab <= 0x7fffffffll);
  REQUIRE(seg_start && n_unique);
  REQUIRE(n == 0 || (ids && uniq && inv && sorted_pos));
  if (ws_bytes < dedup_workspace_bytes(n)) return STAPLE_ERR_WORKSPACE;
  REQUIRE(dedup_workspace_bytes(n) == 0 || ws != nullptr);
  GET_ERR(err);
  HIPCALL(launch_dedup(ids, n, vocab, uniq, inv, sorted_pos, seg_start, n_unique, ws, S(stream), err));
  return STAPLE_OK;
}

// ------------------------------------------------------------------ cache
staple_status_t staple_cache_count(const int32_t* ids, int64_t n, int64_t vocab, int64_t* counts,
                                   void* stream) {
  REQUIRE(n >= 0 && vocab >= 1 && vocab <= 0x7fffffffll && counts);
  REQUIRE(n == 0 || ids);
  GET_ERR(err);
  HIPCALL(launch_cache_count(ids, n, vocab, counts, S(stream), err));
  return STAPLE_OK;
}

size_t staple_cache_build_workspace_bytes(int64_t vocab) {
  return vocab < 1 ? 0 : cache_build_workspace_bytes(vocab);
}

staple_status_t staple_cache_build(const int64_t* counts, int64_t vocab, int64_t capacity,
                                   int32_t* id_to_slot, int32_t* slot_to_id, void* ws,
                                   size_t ws_bytes, void* stream) {
  REQUIRE(vocab >= 1 && vocab <= 0x7fffffffll && capacity >= 0 && capacity <= vocab);
  REQUIRE(counts && id_to_slot && ws && (capacity == 0 || slot_to_id));
  if (ws_bytes < cache_build_workspace_bytes(vocab)) return STAPLE_ERR_WORKSPACE;
  GET_ERR(err);
  HIPCALL(launch_cache_build(counts, vocab, capacity, id_to_slot, slot_to_id, ws, S(stream), err));
  return STAPLE_OK;
}

staple_status_t staple_cache_fill(const void* table, int64_t vocab, int64_t d_ff, int32_t dtype,
                                  const int32_t* slot_to_id, int64_t capacity, void* slot_rows,
                                  void* stream) {
  REQUIRE(valid_dtype(dtype) && vocab >= 1 && d_ff > 0 && capacity >= 0 && capacity <= vocab);
  REQUIRE((d_ff * elem_bytes(dtype)) % 16 == 0);
  REQUIRE(capacity == 0 || (table && slot_to_id && slot_rows));
  REQUIRE(capacity == 0 || (aligned16(table) && aligned16(slot_rows)));
  REQUIRE(capacity == 0 || (device_addressable(table) && device_addressable(slot_rows)));
  GET_ERR(err);
  HIPCALL(launch_gather_rows(table, vocab, slot_to_id, nullptr, capacity, d_ff * elem_bytes(dtype),
                             slot_rows, S(stream), err, copy_workgroups(table)));
  return STAPLE_OK;
}

staple_status_t staple_cache_lookup(const int32_t* uniq, const int32_t* n_unique,
                                    int64_t max_unique, const int32_t* id_to_slot, int64_t vocab,
                                    int32_t* code, int32_t* miss_uidx, int32_t* miss_ids,
                                    int32_t* n_miss, void* stream) {
  REQUIRE(max_unique >= 0 && max_unique <= 0x7fffffffll && vocab >= 1);
  REQUIRE(n_unique && id_to_slot && n_miss);
  REQUIRE(max_unique == 0 || (uniq && code && miss_uidx));
  GET_ERR(err);
  HIPCALL(launch_cache_lookup(uniq, n_unique, max_unique, id_to_slot, vocab, code, miss_uidx,
                              miss_ids, n_miss, S(stream), err));
  return STAPLE_OK;
}

staple_status_t staple_split_tokens(const int32_t* inv, int64_t n_tokens, const int32_t* code,
                                   const int32_t* n_unique, int64_t max_unique, int32_t* hit_pos,
                                   int32_t* miss_pos, int32_t* tok_row, int32_t* counts,
                                   void* stream) {
  REQUIRE(n_tokens >= 0 && n_tokens <= 0x7fffffffll && max_unique >= 0 && max_unique <= n_tokens);
  REQUIRE(n_unique && counts);
  REQUIRE(n_tokens == 0 || (inv && code && hit_pos && miss_pos && tok_row));
  GET_ERR(err);
  HIPCALL(launch_split_tokens(inv, n_tokens, code, n_unique, max_unique, hit_pos, miss_pos, tok_row,
                              counts, S(stream), err));
  return STAPLE_OK;
}

staple_status_t staple_stage_misses(const void* host_table, int64_t vocab, int64_t d_ff,
                                    int32_t dtype, const int32_t* host_miss_ids, int32_t n_miss,
                                    void* host_staging, void* dev_miss_rows, void* stream) {
  REQUIRE(valid_dtype(dtype) && vocab >= 1 && d_ff > 0 && n_miss >= 0);
  if (n_miss == 0) return STAPLE_OK;
  REQUIRE(host_table && host_miss_ids && host_staging && dev_miss_rows);
  const size_t row_bytes = static_cast<size_t>(d_ff) * elem_bytes(dtype);
  for (int32_t m = 0; m < n_miss; ++m)
    if (host_miss_ids[m] < 0 || host_miss_ids[m] >= vocab) return STAPLE_ERR_HOST;
  const char* src = static_cast<const char*>(host_table);
  char* dst = static_cast<char*>(host_staging);
  const size_t total = row_bytes * static_cast<size_t>(n_miss);
  // rows packed by the library's persistent host threads (one per 2 MB)
  auto pack = [&](int64_t lo, int64_t hi) {
    for (int64_t m = lo; m < hi; ++m)
      std::memcpy(dst + m * row_bytes, src + static_cast<size_t>(host_miss_ids[m]) * row_bytes,
                  row_bytes);
  };
  host_parallel_for(n_miss, host_pool_parts(static_cast<int64_t>(total), 16), pack);
  HIPCALL(hipMemcpyAsync(dev_miss_rows, host_staging, total, hipMemcpyHostToDevice, S(stream)));
  return STAPLE_OK;
}

// One DMA copier per device for the staging below, set up on first use and
// kept until the process ends; calls on one device take turns.
namespace {
struct DmaStaging {
  std::mutex mu;
  bool tried = false;
  SdmaCopier copier;
};
constexpr int kDmaDevices = 64;
DmaStaging g_dma[kDmaDevices];
}  // namespace

staple_status_t staple_stage_misses_dma(int64_t n_layers, const void* const* host_tables,
                                        int64_t table_stride, int64_t vocab, int64_t d_ff,
                                        int32_t dtype, const int32_t* host_miss_ids,
                                        int32_t n_miss, void* host_staging,
                                        void* const* dev_miss_rows) {
  REQUIRE(valid_dtype(dtype) && vocab >= 1 && d_ff > 0 && n_miss >= 0);
  REQUIRE(n_layers >= 1 && n_layers <= 4096 && (table_stride == 0 || table_stride >= d_ff));
  if (n_miss == 0) return STAPLE_OK;
  REQUIRE(host_tables && host_miss_ids && host_staging && dev_miss_rows);
  for (int64_t l = 0; l < n_layers; ++l) REQUIRE(host_tables[l] && dev_miss_rows[l]);
  for (int32_t m = 0; m < n_miss; ++m)
    if (host_miss_ids[m] < 0 || host_miss_ids[m] >= vocab) return STAPLE_ERR_HOST;
  REQUIRE(host_memory(host_staging));
  for (int64_t l = 0; l < n_layers; ++l) REQUIRE(device_addressable(dev_miss_rows[l]));
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess || device < 0 || device >= kDmaDevices) return STAPLE_ERR_HIP;
  DmaStaging& ds = g_dma[device];
  std::lock_guard<std::mutex> lock(ds.mu);
  if (!ds.tried) {
    ds.tried = true;
    ds.copier.init(device, SdmaCopier::kMaxSignals);
  }
  if (!ds.copier.ready) return STAPLE_ERR_UNSUPPORTED;
  const size_t row_bytes = static_cast<size_t>(d_ff) * elem_bytes(dtype);
  const size_t src_stride = static_cast<size_t>(table_stride ? table_stride : d_ff) * elem_bytes(dtype);
  const size_t block = row_bytes * static_cast<size_t>(n_miss);
  constexpr int kSig = SdmaCopier::kMaxSignals;
  char* staging = static_cast<char*>(host_staging);
  // layer l's rows are packed while layer l - 1's block is on the DMA engine
  bool ok = true;
  int64_t started = 0;
  for (int64_t l = 0; l < n_layers && ok; ++l) {
    const char* src = static_cast<const char*>(host_tables[l]);
    char* dst = staging + static_cast<size_t>(l) * block;
    auto pack = [&](int64_t lo, int64_t hi) {
      for (int64_t m = lo; m < hi; ++m)
        std::memcpy(dst + m * row_bytes, src + static_cast<size_t>(host_miss_ids[m]) * src_stride,
                    row_bytes);
    };
    host_parallel_for(n_miss, host_pool_parts(static_cast<int64_t>(block), 16), pack);
    const int sig = static_cast<int>(l % kSig);
    if (l >= kSig) ok = ds.copier.wait(sig);     // the copy that last used this signal
    ok = ok && ds.copier.start_h2d(sig, dev_miss_rows[l], dst, block);
    if (ok) started = l + 1;
  }
  for (int64_t l = std::max<int64_t>(0, started - kSig); l < started; ++l)
    ok = ds.copier.wait(static_cast<int>(l % kSig)) && ok;
  return ok ? STAPLE_OK : STAPLE_ERR_HIP;
}

staple_status_t staple_assemble_rows(const void* cache_rows, int64_t capacity,
                                     const void* miss_rows, int64_t max_miss, const int32_t* code,
                                     const int32_t* n_unique, int64_t max_unique, int64_t d_ff,
                                     int32_t dtype, void* rows, void* stream) {
  REQUIRE(valid_dtype(dtype) && d_ff > 0 && capacity >= 0 && max_miss >= 0 && max_unique >= 0);
  REQUIRE((d_ff * elem_bytes(dtype)) % 16 == 0);
  REQUIRE(n_unique && (max_unique == 0 || (code && rows)));
  REQUIRE(capacity == 0 || cache_rows);
  REQUIRE(max_miss == 0 || miss_rows);
  GET_ERR(err);
  HIPCALL(launch_assemble_rows(cache_rows, capacity, miss_rows, max_miss, code, n_unique,
                               max_unique, d_ff * elem_bytes(dtype), rows, S(stream), err));
  return STAPLE_OK;
}

staple_status_t staple_assemble_rows_from_table(const void* cache_rows, int64_t capacity,
                                                const void* table, int64_t vocab,
                                                const int32_t* uniq, const int32_t* code,
                                                const int32_t* n_unique, int64_t max_unique,
                                                int64_t d_ff, int32_t dtype, void* rows,
                                                void* stream) {
  REQUIRE(valid_dtype(dtype) && d_ff > 0 && capacity >= 0 && vocab >= 1 && max_unique >= 0);
  REQUIRE((d_ff * elem_bytes(dtype)) % 16 == 0);
  REQUIRE(n_unique && table && (max_unique == 0 || (uniq && code && rows)));
  REQUIRE(capacity == 0 || cache_rows);
  REQUIRE(aligned16(table) && (capacity == 0 || aligned16(cache_rows)) &&
          (max_unique == 0 || aligned16(rows)));
  REQUIRE(device_addressable(table) && (max_unique == 0 || device_addressable(rows)));
  GET_ERR(err);
  HIPCALL(launch_assemble_rows_table(cache_rows, capacity, table, vocab, uniq, code, n_unique,
                                     max_unique, d_ff * elem_bytes(dtype), rows, S(stream), err,
                                     copy_workgroups(table)));
  return STAPLE_OK;
}

staple_status_t staple_gather_rows(const void* src, int64_t src_rows, const int32_t* index,
                                   const int32_t* n_rows, int64_t max_rows, int64_t d_ff,
                                   int32_t dtype, void* dst, void* stream) {
  REQUIRE(valid_dtype(dtype) && d_ff > 0 && src_rows >= 1 && max_rows >= 0);
  REQUIRE((d_ff * elem_bytes(dtype)) % 16 == 0);
  REQUIRE(max_rows == 0 || (src && index && dst));
  REQUIRE(max_rows == 0 || (aligned16(src) && aligned16(dst)));
  REQUIRE(max_rows == 0 || (device_addressable(src) && device_addressable(dst)));
  GET_ERR(err);
  HIPCALL(launch_gather_rows(src, src_rows, index, n_rows, max_rows, d_ff * elem_bytes(dtype), dst,
                             S(stream), err,
                             copy_workgroups(src)));
  return STAPLE_OK;
}

// ------------------------------------------------------------------ FFN
static bool ffn_shape_ok(int64_t n, int64_t d, int64_t f, int32_t dtype) {
  return n >= 0 && n <= 0x7fffffffll && d > 0 && f > 0 && d % 64 == 0 && f % 64 == 0 &&
         d <= (1ll << 20) && f <= (1ll << 20) && valid_dtype(dtype);
}

size_t staple_ffn_down_workspace_bytes(int64_t n, int64_t d, int64_t f, int32_t dtype) {
  if (!ffn_shape_ok(n, d, f, dtype)) return 0;
  return decode_eligible(n, d, f, dtype) ? align_up(decode_down_workspace_bytes(n, d), 256) : 0;
}

// workspace of staple_ffn_fwd: [h when not saved][down partials]
size_t staple_ffn_fwd_workspace_bytes(int64_t n, int64_t d, int64_t f, int32_t dtype) {
  if (!ffn_shape_ok(n, d, f, dtype)) return 0;
  return align_up(static_cast<size_t>(n) * f * elem_bytes(dtype), 256) +
         staple_ffn_down_workspace_bytes(n, d, f, dtype);
}

static staple_status_t gate_up_impl(int64_t n_sel, const int32_t* pos, int64_t n_tokens,
                                    int64_t d, int64_t f, int32_t dtype, const void* x,
                                    const void* w_gate, const void* w_up, const void* rows,
                                    int64_t n_rows, const int32_t* row_index, void* h,
                                    void* save_g, void* save_u, hipStream_t s) {
  GET_ERR(err);
  if (decode_eligible(n_sel, d, f, dtype))
    HIPCALL(decode_gateup(n_sel, pos, n_tokens, d, f, x, w_gate, w_up, rows, n_rows, row_index, h,
                          save_g, save_u, s, err, false, w_up != nullptr));
  else if (dtype == STAPLE_BF16)
    HIPCALL(gateup_fwd<bf16_t>(n_sel, pos, n_tokens, d, f, x, w_gate, w_up, rows, n_rows,
                               row_index, h, save_g, save_u, s, err));
  else
    HIPCALL(gateup_fwd<float>(n_sel, pos, n_tokens, d, f, x, w_gate, w_up, rows, n_rows, row_index,
                              h, save_g, save_u, s, err));
  return STAPLE_OK;
}

static staple_status_t down_impl(int64_t n, int64_t d, int64_t f, int32_t dtype, int32_t out_dtype,
                                 const void* h, const void* w_down, void* y, void* ws,
                                 hipStream_t s) {
  if (decode_eligible(n, d, f, dtype)) HIPCALL(decode_down(n, d, f, h, w_down, y, out_dtype, ws, s, false));
  else if (dtype == STAPLE_BF16) HIPCALL(down_fwd<bf16_t>(n, d, f, h, w_down, y, out_dtype, s));
  else HIPCALL(down_fwd<float>(n, d, f, h, w_down, y, out_dtype, s));
  return STAPLE_OK;
}

staple_status_t staple_ffn_gate_up(int64_t n, int64_t d, int64_t f, int32_t dtype, const void* x,
                                   const void* w_gate, const void* w_up, const void* rows,
                                   int64_t n_rows, const int32_t* row_index, void* h,
                                   void* save_g, void* save_u, void* stream) {
  if (!ffn_shape_ok(n, d, f, dtype)) return STAPLE_ERR_UNSUPPORTED;
  REQUIRE(w_gate && rows && n_rows >= 1);
  REQUIRE(aligned16(w_gate) && (!w_up || aligned16(w_up)) && aligned16(rows));
  if (n == 0) return STAPLE_OK;
  REQUIRE(x && row_index && h && aligned16(x) && aligned16(h));
  REQUIRE((!save_g || aligned16(save_g)) && (!save_u || aligned16(save_u)));
  return gate_up_impl(n, nullptr, n, d, f, dtype, x, w_gate, w_up, rows, n_rows, row_index, h,
                      save_g, save_u, S(stream));
}

staple_status_t staple_ffn_gate_up_tokens(int64_t n_sel, const int32_t* token_pos, int64_t n_tokens,
                                          int64_t d, int64_t f, int32_t dtype, const void* x,
                                          const void* w_gate, const void* w_up, const void* rows,
                                          int64_t n_rows, const int32_t* row_index, void* h,
                                          void* save_g, void* save_u, void* stream) {
  if (!ffn_shape_ok(n_tokens, d, f, dtype)) return STAPLE_ERR_UNSUPPORTED;
  REQUIRE(n_sel >= 0 && n_sel <= n_tokens);
  REQUIRE(w_gate && rows && n_rows >= 1);
  REQUIRE(aligned16(w_gate) && (!w_up || aligned16(w_up)) && aligned16(rows));
  if (n_sel == 0) return STAPLE_OK;
  REQUIRE(token_pos && x && row_index && h && aligned16(x) && aligned16(h));
  REQUIRE((!save_g || aligned16(save_g)) && (!save_u || aligned16(save_u)));
  return gate_up_impl(n_sel, token_pos, n_tokens, d, f, dtype, x, w_gate, w_up, rows, n_rows,
                      row_index, h, save_g, save_u, S(stream));
}

staple_status_t staple_ffn_down(int64_t n, int64_t d, int64_t f, int32_t dtype, int32_t out_dtype,
                                const void* h, const void* w_down, void* y, void* ws,
                                size_t ws_bytes, void* stream) {
  if (!valid_dtype(out_dtype) || !ffn_shape_ok(n, d, f, dtype)) return STAPLE_ERR_UNSUPPORTED;
  REQUIRE(w_down && aligned16(w_down));
  if (n == 0) return STAPLE_OK;
  REQUIRE(h && y && aligned16(h) && aligned16(y));
  const size_t need = staple_ffn_down_workspace_bytes(n, d, f, dtype);
  if (ws_bytes < need) return STAPLE_ERR_WORKSPACE;
  REQUIRE(need == 0 || (ws && aligned16(ws)));
  return down_impl(n, d, f, dtype, out_dtype, h, w_down, y, ws, S(stream));
}

staple_status_t staple_ffn_fwd(int64_t n, int64_t d, int64_t f, int32_t dtype, int32_t out_dtype,
                               const void* x, const void* w_gate, const void* w_up,
                               const void* w_down, const void* rows, int64_t n_rows,
                               const int32_t* row_index, void* y, void* save_g, void* save_u,
                               void* save_h, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return STAPLE_ERR_UNSUPPORTED;
  if (!ffn_shape_ok(n, d, f, dtype)) return STAPLE_ERR_UNSUPPORTED;
  REQUIRE(w_gate && w_down && rows && n_rows >= 1);
  REQUIRE(aligned16(w_gate) && (!w_up || aligned16(w_up)) && aligned16(w_down) && aligned16(rows));
  if (n == 0) return STAPLE_OK;
  REQUIRE(x && row_index && y && aligned16(x) && aligned16(y));
  REQUIRE((!save_g || aligned16(save_g)) && (!save_u || aligned16(save_u)) &&
          (!save_h || aligned16(save_h)));
  if (ws_bytes < staple_ffn_fwd_workspace_bytes(n, d, f, dtype)) return STAPLE_ERR_WORKSPACE;
  REQUIRE(ws && aligned16(ws));
  void* h = save_h ? save_h : ws;
  void* down_ws = static_cast<char*>(ws) + align_up(static_cast<size_t>(n) * f * elem_bytes(dtype), 256);
  hipStream_t s = S(stream);
  staple_status_t st = gate_up_impl(n, nullptr, n, d, f, dtype, x, w_gate, w_up, rows, n_rows,
                                    row_index, h, save_g, save_u, s);
  if (st != STAPLE_OK) return st;
  return down_impl(n, d, f, dtype, out_dtype, h, w_down, y, down_ws, s);
}

staple_status_t staple_decode_pack_weights(int64_t d, int64_t f, int32_t dtype, const void* w_gate,
                                           const void* w_up, const void* w_down,
                                           void* packed_gate_up, void* packed_down, void* stream) {
  if (dtype != STAPLE_BF16 || !ffn_shape_ok(1, d, f, dtype)) return STAPLE_ERR_UNSUPPORTED;
  REQUIRE(packed_gate_up || packed_down);
  REQUIRE(!packed_gate_up || (w_gate && aligned16(w_gate) && (!w_up || aligned16(w_up)) &&
                              aligned16(packed_gate_up)));
  REQUIRE(!packed_down || (w_down && aligned16(w_down) && aligned16(packed_down)));
  HIPCALL(decode_pack(d, f, w_gate, w_up, w_down, packed_gate_up, packed_down, S(stream)));
  return STAPLE_OK;
}

staple_status_t staple_ffn_gate_up_packed(int64_t n, int64_t d, int64_t f, int32_t dtype,
                                          const void* x, const void* packed_gate_up,
                                          int32_t up_proj, const void* rows, int64_t n_rows,
                                          const int32_t* row_index, void* h, void* save_g,
                                          void* save_u, void* stream) {
  if (dtype != STAPLE_BF16 || !ffn_shape_ok(n, d, f, dtype)) return STAPLE_ERR_UNSUPPORTED;
  if (n > 0 && !decode_eligible(n, d, f, dtype)) return STAPLE_ERR_UNSUPPORTED;
  REQUIRE(packed_gate_up && rows && n_rows >= 1);
  REQUIRE(aligned16(packed_gate_up) && aligned16(rows));
  if (n == 0) return STAPLE_OK;
  REQUIRE(x && row_index && h && aligned16(x) && aligned16(h));
  REQUIRE((!save_g || aligned16(save_g)) && (!save_u || aligned16(save_u)));
  GET_ERR(err);
  HIPCALL(decode_gateup(n, nullptr, n, d, f, x, packed_gate_up, nullptr, rows, n_rows, row_index, h,
                        save_g, save_u, S(stream), err, true, up_proj != 0));
  return STAPLE_OK;
}

staple_status_t staple_ffn_down_packed(int64_t n, int64_t d, int64_t f, int32_t dtype,
                                       int32_t out_dtype, const void* h, const void* packed_down,
                                       void* y, void* ws, size_t ws_bytes, void* stream) {
  if (dtype != STAPLE_BF16 || !valid_dtype(out_dtype) || !ffn_shape_ok(n, d, f, dtype))
    return STAPLE_ERR_UNSUPPORTED;
  if (n > 0 && !decode_eligible(n, d, f, dtype)) return STAPLE_ERR_UNSUPPORTED;
  REQUIRE(packed_down && aligned16(packed_down));
  if (n == 0) return STAPLE_OK;
  REQUIRE(h && y && aligned16(h) && aligned16(y));
  if (ws_bytes < staple_ffn_down_workspace_bytes(n, d, f, dtype)) return STAPLE_ERR_WORKSPACE;
  REQUIRE(ws && aligned16(ws));
  HIPCALL(decode_down(n, d, f, h, packed_down, y, out_dtype, ws, S(stream), true));
  return STAPLE_OK;
}

staple_status_t staple_ffn_fwd_packed(int64_t n, int64_t d, int64_t f, int32_t dtype,
                                      int32_t out_dtype, const void* x,
                                      const void* packed_gate_up, int32_t up_proj,
                                      const void* packed_down, const void* rows, int64_t n_rows,
                                      const int32_t* row_index, void* y, void* save_g,
                                      void* save_u, void* save_h, void* ws, size_t ws_bytes,
                                      void* stream) {
  if (dtype != STAPLE_BF16 || !valid_dtype(out_dtype)) return STAPLE_ERR_UNSUPPORTED;
  if (!ffn_shape_ok(n, d, f, dtype)) return STAPLE_ERR_UNSUPPORTED;
  if (n > 0 && !decode_eligible(n, d, f, dtype)) return STAPLE_ERR_UNSUPPORTED;
  REQUIRE(packed_gate_up && packed_down && rows && n_rows >= 1);
  REQUIRE(aligned16(packed_gate_up) && aligned16(packed_down) && aligned16(rows));
  if (n == 0) return STAPLE_OK;
  REQUIRE(x && row_index && y && aligned16(x) && aligned16(y));
  REQUIRE((!save_g || aligned16(save_g)) && (!save_u || aligned16(save_u)) &&
          (!save_h || aligned16(save_h)));
  if (ws_bytes < staple_ffn_fwd_workspace_bytes(n, d, f, dtype)) return STAPLE_ERR_WORKSPACE;
  REQUIRE(ws && aligned16(ws));
  void* h = save_h ? save_h : ws;
  void* down_ws = static_cast<char*>(ws) + align_up(static_cast<size_t>(n) * f * elem_bytes(dtype), 256);
  hipStream_t s = S(stream);
  GET_ERR(err);
  HIPCALL(decode_gateup(n, nullptr, n, d, f, x, packed_gate_up, nullptr, rows, n_rows, row_index, h,
                        save_g, save_u, s, err, true, up_proj != 0));
  HIPCALL(decode_down(n, d, f, h, packed_down, y, out_dtype, down_ws, s, true));
  return STAPLE_OK;
}

staple_status_t staple_ffn_fwd_packed_noalloc(int64_t n, int64_t d, int64_t f, int32_t dtype,
                                              int32_t out_dtype, const void* x,
                                              const void* packed_gate_up, int32_t up_proj,
                                              const void* packed_down, const void* rows,
                                              int64_t n_rows, const int32_t* row_index, void* y,
                                              void* save_g, void* save_u, void* save_h,
                                              void* stream) {
  if (dtype != STAPLE_BF16 || !valid_dtype(out_dtype)) return STAPLE_ERR_UNSUPPORTED;
  if (!ffn_shape_ok(n, d, f, dtype)) return STAPLE_ERR_UNSUPPORTED;
  if (n > 0 && !decode_eligible(n, d, f, dtype)) return STAPLE_ERR_UNSUPPORTED;
  REQUIRE(packed_gate_up && packed_down && rows && n_rows >= 1);
  REQUIRE(aligned16(packed_gate_up) && aligned16(packed_down) && aligned16(rows));
  if (n == 0) return STAPLE_OK;
  REQUIRE(x && row_index && y && aligned16(x) && aligned16(y));
  REQUIRE((!save_g || aligned16(save_g)) && (!save_u || aligned16(save_u)) &&
          (!save_h || aligned16(save_h)));
  // the same layout as staple_ffn_fwd_packed's workspace, in the fixed scratch
  if (staple_ffn_fwd_workspace_bytes(n, d, f, dtype) > kNoAllocScratchBytes)
    return STAPLE_ERR_SCRATCH_LIMIT;
  void* ws = device_scratch();
  if (ws == nullptr) return STAPLE_ERR_HIP;
  void* h = save_h ? save_h : ws;
  void* down_ws = static_cast<char*>(ws) + align_up(static_cast<size_t>(n) * f * elem_bytes(dtype), 256);
  hipStream_t s = S(stream);
  GET_ERR(err);
  HIPCALL(decode_gateup(n, nullptr, n, d, f, x, packed_gate_up, nullptr, rows, n_rows, row_index, h,
                        save_g, save_u, s, err, true, up_proj != 0));
  HIPCALL(decode_down(n, d, f, h, packed_down, y, out_dtype, down_ws, s, true));
  return STAPLE_OK;
}

// ------------------------------------------------------------------ decode step driver
// workspace of the decode step driver: [dedup][per-token row sources][h][down partials]
size_t staple_decode_step_workspace_bytes(int64_t n, int64_t d, int64_t f) {
  if (!decode_eligible(n, d, f, STAPLE_BF16) || !ffn_shape_ok(n, d, f, STAPLE_BF16)) return 0;
  return align_up(dedup_workspace_bytes(n), 256) + align_up(static_cast<size_t>(n) * sizeof(int32_t), 256) +
         staple_ffn_fwd_workspace_bytes(n, d, f, STAPLE_BF16);
}

staple_status_t staple_decode_step_cached(
    int64_t n_layers, const staple_decode_layer_t* layers, int64_t n, int64_t d, int64_t f,
    int32_t up_proj, int32_t out_dtype, const int32_t* ids, int64_t vocab,
    const int32_t* id_to_slot, int64_t capacity, int32_t group, int32_t* uniq, int32_t* inv,
    int32_t* sorted_pos, int32_t* seg_start, int32_t* n_unique, int32_t* code, int32_t* miss_uidx,
    int32_t* n_miss, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_dtype(out_dtype) || !ffn_shape_ok(n, d, f, STAPLE_BF16) ||
      !decode_eligible(n, d, f, STAPLE_BF16))
    return STAPLE_ERR_UNSUPPORTED;
  REQUIRE(n_layers >= 1 && n_layers <= 4096 && layers);
  REQUIRE(vocab >= 1 && vocab <= 0x7fffffffll && capacity >= 0);
  REQUIRE(group >= 0 && group <= kCopyJobLayers);
  REQUIRE(ids && id_to_slot && uniq && inv && sorted_pos && seg_start && n_unique && code &&
          miss_uidx && n_miss);
  const size_t need = staple_decode_step_workspace_bytes(n, d, f);
  if (ws_bytes < need) return STAPLE_ERR_WORKSPACE;
  REQUIRE(ws && aligned16(ws));
  bool any_direct = false;
  for (int64_t l = 0; l < n_layers; ++l) {
    const staple_decode_layer_t& L = layers[l];
    REQUIRE(L.x && L.packed_gate_up && L.packed_down && L.table && L.y);
    REQUIRE(capacity == 0 || L.cache_rows);
    REQUIRE(aligned16(L.x) && aligned16(L.packed_gate_up) && aligned16(L.packed_down) &&
            aligned16(L.table) && (!L.rows || aligned16(L.rows)) && aligned16(L.y) &&
            (capacity == 0 || aligned16(L.cache_rows)));
    REQUIRE(L.table_stride == 0 || (L.table_stride >= f && L.table_stride % 8 == 0));
    REQUIRE(device_addressable(L.table));
    REQUIRE(group == 0 || L.rows);   // carried copies fill compact rows
    any_direct = any_direct || !L.rows;
  }
  REQUIRE(capacity <= 0x7fffffffll);
  GET_ERR(err);
  hipStream_t s = S(stream);
  const int64_t row_bytes = f * 2;
  auto table_ld = [&](const staple_decode_layer_t& L) -> int64_t {
    return (L.table_stride ? L.table_stride : f) * 2;
  };
  void* dedup_ws = ws;
  int32_t* row_src = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + align_up(dedup_workspace_bytes(n), 256));
  void* fwd_ws = reinterpret_cast<char*>(row_src) + align_up(static_cast<size_t>(n) * sizeof(int32_t), 256);
  void* h = fwd_ws;
  void* down_ws = static_cast<char*>(fwd_ws) + align_up(static_cast<size_t>(n) * f * 2, 256);
  // a decode batch (at most 64 tokens): dedup and cache probe in one wave
  (void)dedup_ws;
  HIPCALL(launch_dedup_lookup_wave(ids, n, vocab, id_to_slot, uniq, inv, sorted_pos, seg_start,
                                   n_unique, code, miss_uidx, n_miss,
                                   any_direct ? row_src : nullptr, s, err));
  // Which layers' rows are copied by the gate/up launches of the group before
  // (group > 0): group k + 1's rows, split in `group` parts over group k's
  // launches, when a part fits the copy waves of one launch.  The others
  // (group 0, and all of them when group == 0) are assembled here, before the
  // first layer, one launch per slice of layers.
  const int64_t G = group;
  const int64_t n_groups = G > 0 ? (n_layers + G - 1) / G : 0;
  // a part of group g's rows: unique rows part, part + G, ... (at most
  // ceil(n / G) of them) of each of its layers
  auto plan = [&](int64_t g, int* per, int* seg) -> bool {
    const int64_t layers_in = std::min<int64_t>(G, n_layers - g * G);
    return decode_copy_plan((n + G - 1) / G * layers_in, f, up_proj != 0, per, seg);
  };
  auto carried = [&](int64_t g) -> bool {   // group g's rows ride group g - 1's launches
    int per = 0, seg = 0;
    return G > 0 && g > 0 && g < n_groups && plan(g, &per, &seg);
  };
  LayerRowSources src{};
  int cnt = 0;
  for (int64_t l = 0; l < n_layers; ++l) {
    const staple_decode_layer_t& L = layers[l];
    if (!L.rows || (G > 0 && carried(l / G))) continue;
    src.cache_rows[cnt] = L.cache_rows;
    src.table[cnt] = L.table;
    src.table_ld[cnt] = table_ld(L);
    src.rows[cnt] = L.rows;
    if (++cnt == kMaxAssembleLayers) {
      HIPCALL(launch_assemble_rows_layers(src, cnt, capacity, vocab, uniq, code, n_unique, n,
                                          row_bytes, s, err));
      cnt = 0;
    }
  }
  if (cnt > 0)
    HIPCALL(launch_assemble_rows_layers(src, cnt, capacity, vocab, uniq, code, n_unique, n,
                                        row_bytes, s, err));
  for (int64_t l = 0; l < n_layers; ++l) {
    const staple_decode_layer_t& L = layers[l];
    RowCopyJob job{};
    bool with_job = false;
    if (G > 0 && carried(l / G + 1)) {
      const int64_t first = (l / G + 1) * G;
      job.n_layers = static_cast<int>(std::min<int64_t>(G, n_layers - first));
      for (int j = 0; j < job.n_layers; ++j) {
        const staple_decode_layer_t& M = layers[first + j];
        job.cache_rows[j] = M.cache_rows;
        job.table[j] = M.table;
        job.table_ld[j] = table_ld(M);
        job.rows[j] = M.rows;
      }
      job.uniq = uniq;
      job.code = code;
      job.n_unique = n_unique;
      job.max_unique = n;
      job.capacity = capacity;
      job.vocab = vocab;
      job.row_bytes = row_bytes;
      job.part = static_cast<int>(l % G);
      job.parts = static_cast<int>(G);
      job.rows_max = static_cast<int>((n + G - 1) / G * job.n_layers);
      plan(l / G + 1, &job.per, &job.seg);
      with_job = true;
    }
    if (L.rows)
      HIPCALL(decode_gateup(n, nullptr, n, d, f, L.x, L.packed_gate_up, nullptr, L.rows, n, inv, h,
                            nullptr, nullptr, s, err, true, up_proj != 0, nullptr, 0, 0,
                            with_job ? &job : nullptr));
    else   // each token's row read in place: its cache slot, or its row of the table
      HIPCALL(decode_gateup(n, nullptr, n, d, f, L.x, L.packed_gate_up, nullptr, L.cache_rows,
                            capacity, row_src, h, nullptr, nullptr, s, err, true, up_proj != 0,
                            L.table, vocab, L.table_stride ? L.table_stride : f));
    HIPCALL(decode_down(n, d, f, h, L.packed_down, L.y, out_dtype, down_ws, s, true));
  }
  return STAPLE_OK;
}

// ------------------------------------------------------------------ prefill chunk rows
size_t staple_prefill_rows_workspace_bytes(int64_t n) {
  return n < 1 || n > 0x7fffffffll ? 0 : align_up(dedup_workspace_bytes(n), 256);
}

staple_status_t staple_prefill_rows_cached(
    int64_t n_layers, const staple_row_source_t* layers, int64_t n, int64_t d_ff, int32_t dtype,
    const int32_t* ids, int64_t vocab, const int32_t* id_to_slot, int64_t capacity,
    int32_t lookup, int32_t max_workgroups, int32_t* uniq, int32_t* inv, int32_t* sorted_pos,
    int32_t* seg_start, int32_t* n_unique, int32_t* code, int32_t* miss_uidx, int32_t* n_miss,
    void* ws, size_t ws_bytes, void* stream) {
  REQUIRE(valid_dtype(dtype) && d_ff > 0 && (d_ff * elem_bytes(dtype)) % 16 == 0);
  REQUIRE(n >= 1 && n <= 0x7fffffffll && vocab >= 1 && vocab <= 0x7fffffffll);
  REQUIRE(capacity >= 0 && capacity <= 0x7fffffffll && max_workgroups >= 0);
  REQUIRE(lookup == 0 || lookup == 1);
  REQUIRE(n_layers >= 1 && n_layers <= 4096 && layers);
  REQUIRE(ids && id_to_slot && uniq && inv && sorted_pos && seg_start && n_unique && code &&
          miss_uidx && n_miss);
  const size_t need = staple_prefill_rows_workspace_bytes(n);
  if (ws_bytes < need) return STAPLE_ERR_WORKSPACE;
  REQUIRE(need == 0 || (ws && aligned16(ws)));
  for (int64_t l = 0; l < n_layers; ++l) {
    const staple_row_source_t& L = layers[l];
    REQUIRE(L.table && L.rows && (capacity == 0 || L.cache_rows));
    REQUIRE(aligned16(L.table) && aligned16(L.rows) && (capacity == 0 || aligned16(L.cache_rows)));
    REQUIRE(L.table_stride == 0 ||
            (L.table_stride >= d_ff && (L.table_stride * elem_bytes(dtype)) % 16 == 0));
    REQUIRE(device_addressable(L.table) && device_addressable(L.rows));
  }
  GET_ERR(err);
  hipStream_t s = S(stream);
  const int64_t row_bytes = d_ff * elem_bytes(dtype);
  if (lookup) {
    HIPCALL(launch_dedup(ids, n, vocab, uniq, inv, sorted_pos, seg_start, n_unique, ws, s, err));
    HIPCALL(launch_cache_lookup(uniq, n_unique, n, id_to_slot, vocab, code, miss_uidx, nullptr,
                                n_miss, s, err));
  }
  const unsigned wgs = max_workgroups > 0 ? static_cast<unsigned>(max_workgroups) : kLayerRowWorkgroups;
  LayerRowSources src{};
  int cnt = 0;
  for (int64_t l = 0; l < n_layers; ++l) {
    const staple_row_source_t& L = layers[l];
    src.cache_rows[cnt] = L.cache_rows;
    src.table[cnt] = L.table;
    src.table_ld[cnt] = (L.table_stride ? L.table_stride : d_ff) * elem_bytes(dtype);
    src.rows[cnt] = L.rows;
    if (++cnt == kMaxAssembleLayers || l + 1 == n_layers) {
      HIPCALL(launch_assemble_rows_layers(src, cnt, capacity, vocab, uniq, code, n_unique, n,
                                          row_bytes, s, err, wgs));
      cnt = 0;
    }
  }
  return STAPLE_OK;
}

staple_status_t staple_group_tables_host(const void* const* tables, int64_t n_tables,
                                         int64_t vocab, int64_t d_ff, int32_t dtype,
                                         void* grouped) {
  REQUIRE(valid_dtype(dtype) && n_tables >= 1 && n_tables <= 64 && vocab >= 1 && d_ff > 0);
  REQUIRE(tables && grouped);
  for (int64_t j = 0; j < n_tables; ++j) REQUIRE(tables[j]);
  const size_t row = static_cast<size_t>(d_ff) * elem_bytes(dtype);
  char* dst = static_cast<char*>(grouped);
  auto body = [&](int64_t lo, int64_t hi) {
    for (int64_t t = lo; t < hi; ++t)
      for (int64_t j = 0; j < n_tables; ++j)
        std::memcpy(dst + (t * n_tables + j) * row,
                    static_cast<const char*>(tables[j]) + t * row, row);
  };
  host_parallel_for(vocab, host_pool_parts(static_cast<int64_t>(vocab * n_tables * row), 16), body);
  return STAPLE_OK;
}

// ------------------------------------------------------------------ low-rank table
static bool lowrank_shape_ok(int64_t max_rows, int64_t r, int64_t f, int32_t dtype) {
  return valid_dtype(dtype) && max_rows >= 0 && max_rows <= 0x7fffffffll && r > 0 && f > 0 &&
         r % 64 == 0 && f % 64 == 0 && r <= (1ll << 20) && f <= (1ll << 20);
}

staple_status_t staple_lowrank_expand(const void* rows_r, const int32_t* n_rows, int64_t max_rows,
                                      int64_t r, int64_t d_ff, int32_t dtype, const void* proj,
                                      void* z, void* stream) {
  if (!lowrank_shape_ok(max_rows, r, d_ff, dtype)) return STAPLE_ERR_UNSUPPORTED;
  REQUIRE(n_rows && proj && aligned16(proj));
  if (max_rows == 0) return STAPLE_OK;
  REQUIRE(rows_r && z && aligned16(rows_r) && aligned16(z));
  if (dtype == STAPLE_BF16)
    HIPCALL(lowrank_expand<bf16_t>(max_rows, n_rows, r, d_ff, rows_r, proj, z, S(stream)));
  else
    HIPCALL(lowrank_expand<float>(max_rows, n_rows, r, d_ff, rows_r, proj, z, S(stream)));
  return STAPLE_OK;
}

size_t staple_lowrank_bwd_workspace_bytes(int64_t max_rows, int64_t d_ff, int32_t dtype) {
  if (max_rows < 0 || d_ff <= 0 || !valid_dtype(dtype)) return 0;
  return dtype == STAPLE_BF16 ? align_up(static_cast<size_t>(max_rows) * d_ff * 2, 256) : 0;
}

staple_status_t staple_lowrank_bwd(const float* d_rows, const void* rows_r, const int32_t* n_rows,
                                   int64_t max_rows, int64_t r, int64_t d_ff, int32_t dtype,
                                   const void* proj, float* d_rows_r, float* d_proj, void* ws,
                                   size_t ws_bytes, void* stream) {
  if (!lowrank_shape_ok(max_rows, r, d_ff, dtype)) return STAPLE_ERR_UNSUPPORTED;
  REQUIRE(n_rows && proj && d_proj && aligned16(proj) && aligned16(d_proj));
  if (max_rows > 0) {
    REQUIRE(d_rows && rows_r && d_rows_r);
    REQUIRE(aligned16(d_rows) && aligned16(rows_r) && aligned16(d_rows_r));
    const size_t need = staple_lowrank_bwd_workspace_bytes(max_rows, d_ff, dtype);
    if (ws_bytes < need) return STAPLE_ERR_WORKSPACE;
    REQUIRE(need == 0 || (ws && aligned16(ws)));
  }
  // max_rows == 0 still writes dP (all zeros: the K range is empty)
  if (dtype == STAPLE_BF16)
    HIPCALL(lowrank_bwd<bf16_t>(max_rows, n_rows, r, d_ff, d_rows, rows_r, proj, d_rows_r, d_proj,
                                ws, S(stream)));
  else
    HIPCALL(lowrank_bwd<float>(max_rows, n_rows, r, d_ff, d_rows, rows_r, proj, d_rows_r, d_proj,
                               ws, S(stream)));
  return STAPLE_OK;
}

// ------------------------------------------------------------------ AdamW
static bool adamw_hparams_ok(float lr, float beta1, float beta2, float eps, float weight_decay,
                             int64_t step) {
  return step >= 1 && std::isfinite(lr) && lr >= 0.0f && beta1 >= 0.0f && beta1 < 1.0f &&
         beta2 >= 0.0f && beta2 < 1.0f && std::isfinite(eps) && eps >= 0.0f &&
         std::isfinite(weight_decay) && weight_decay >= 0.0f;
}

staple_status_t staple_adamw_rows(void* table, float* m, float* v, int64_t vocab, int64_t d_ff,
                                  int32_t dtype, const int32_t* rows, const int32_t* n_rows,
                                  int64_t max_rows, const float* grad, float lr, float beta1,
                                  float beta2, float eps, float weight_decay, int64_t step,
                                  void* stream) {
  REQUIRE(valid_dtype(dtype) && vocab >= 1 && d_ff > 0 && d_ff % 8 == 0 && max_rows >= 0);
  REQUIRE(adamw_hparams_ok(lr, beta1, beta2, eps, weight_decay, step));
  if (max_rows == 0) return STAPLE_OK;
  REQUIRE(table && m && v && rows && grad);
  REQUIRE(aligned16(table) && aligned16(m) && aligned16(v) && aligned16(grad));
  GET_ERR(err);
  const AdamWConsts c = adamw_consts(lr, beta1, beta2, eps, weight_decay, step);
  HIPCALL(launch_adamw_rows(table, dtype, m, v, vocab, d_ff, rows, n_rows, max_rows, grad, c,
                            S(stream), err));
  return STAPLE_OK;
}

staple_status_t staple_adamw_rows_host(void* table, float* m, float* v, int64_t vocab, int64_t d_ff,
                                       int32_t dtype, const int32_t* rows, int64_t n_rows,
                                       const float* grad, float lr, float beta1, float beta2,
                                       float eps, float weight_decay, int64_t step,
                                       int32_t n_threads) {
  REQUIRE(valid_dtype(dtype) && vocab >= 1 && d_ff > 0 && n_rows >= 0);
  REQUIRE(adamw_hparams_ok(lr, beta1, beta2, eps, weight_decay, step));
  if (n_rows == 0) return STAPLE_OK;
  REQUIRE(table && m && v && rows && grad);
  for (int64_t k = 0; k < n_rows; ++k)
    if (rows[k] < 0 || rows[k] >= vocab) return STAPLE_ERR_HOST;
  const int hw = static_cast<int>(std::max(1u, std::thread::hardware_concurrency()));
  const int nt = n_threads > 0 ? n_threads : std::min(hw, 16);
  const AdamWConsts c = adamw_consts(lr, beta1, beta2, eps, weight_decay, step);
  host_adamw_rows(table, dtype, m, v, d_ff, rows, n_rows, grad, c, nt);
  return STAPLE_OK;
}

staple_status_t staple_cache_refresh(const void* table, int64_t vocab, int64_t d_ff, int32_t dtype,
                                     const int32_t* uniq, const int32_t* code,
                                     const int32_t* n_unique, int64_t max_unique, void* cache_rows,
                                     int64_t capacity, void* stream) {
  REQUIRE(valid_dtype(dtype) && vocab >= 1 && d_ff > 0 && capacity >= 0 && max_unique >= 0);
  REQUIRE((d_ff * elem_bytes(dtype)) % 16 == 0);
  if (max_unique == 0 || capacity == 0) return STAPLE_OK;
  REQUIRE(table && uniq && code && n_unique && cache_rows);
  REQUIRE(aligned16(table) && aligned16(cache_rows));
  REQUIRE(device_addressable(table) && device_addressable(cache_rows));
  GET_ERR(err);
  HIPCALL(launch_cache_refresh(table, vocab, uniq, code, n_unique, max_unique,
                               d_ff * elem_bytes(dtype), cache_rows, capacity, S(stream), err,
                               copy_workgroups(table)));
  return STAPLE_OK;
}

// workspace of the backward: [dg | du] (n x 2f, dtype), an n x f fp32 region
// (h when it is recomputed), the segment-sum partials, then (bf16) the
// K-major copies
static size_t bwd_dgu_bytes(int64_t n, int64_t f, int32_t dtype) {
  return align_up(static_cast<size_t>(n) * 2 * f * elem_bytes(dtype), 256);
}
static size_t bwd_aux_bytes(int64_t n, int64_t f) {
  return align_up(static_cast<size_t>(n) * f * sizeof(float), 256);
}
// bf16: the K-major copies W_down^T [f x d], [W_gate^T | W_up^T] [d x 2f] and
// dy^T [d x n64] (n64 = n rounded up to whole 64-token k stages, zero-padded)
static int64_t round64(int64_t v) { return (v + 63) / 64 * 64; }
static size_t bwd_kt_bytes(int64_t n, int64_t d, int64_t f, int32_t dtype) {
  if (dtype != STAPLE_BF16 || n == 0) return 0;
  return align_up(static_cast<size_t>(f) * d * 2, 256) + align_up(static_cast<size_t>(d) * 2 * f * 2, 256) +
         align_up(static_cast<size_t>(d) * round64(n) * 2, 256);
}

size_t staple_ffn_bwd_workspace_bytes(int64_t n, int64_t d, int64_t f, int32_t dtype) {
  if (!ffn_shape_ok(n, d, f, dtype)) return 0;
  return bwd_dgu_bytes(n, f, dtype) + bwd_aux_bytes(n, f) +
         align_up(segment_sum_workspace_bytes(n, f), 256) + bwd_kt_bytes(n, d, f, dtype);
}

}  // extern "C"

template <typename T>
static staple_status_t bwd_impl(int64_t n, int64_t d, int64_t f, int32_t dtype, int32_t out_dtype,
                                const void* dy, const void* x, const void* w_gate, const void* w_up,
                                const void* w_down, const void* saved_g, const void* saved_u,
                                const void* saved_h, const int32_t* sorted_pos, const int32_t* inv,
                                const int32_t* seg_start, const int32_t* n_unique,
                                int64_t max_unique, float* d_rows, void* dx, float* dw_gate,
                                float* dw_up, float* dw_down, bool fz, void* ws,
                                hipEvent_t rows_event, hipStream_t s, int* err) {
  void* dgu = ws;
  char* aux = n > 0 ? static_cast<char*>(ws) + bwd_dgu_bytes(n, f, dtype) : nullptr;
  char* seg_ws = n > 0 ? aux + bwd_aux_bytes(n, f) : nullptr;
  // bf16: K-major copies of W_down, [W_gate; W_up], dy and x, so that dh and
  // dx read both operands K-major and the weight gradients one (the same
  // products in the same order: the outputs are the same bits as with
  // MN-major operands); dh runs over the tokens in sorted order and its
  // epilogue does the table-row segment sum's chunk pass on the fp32 du.
  // fp32: the du half of [dg | du] is fp32 and the segment sum reads it.
  const bool kt = dtype == STAPLE_BF16 && n > 0;
  char* wd_t = kt ? seg_ws + align_up(segment_sum_workspace_bytes(n, f), 256) : nullptr;
  char* w_t = kt ? wd_t + align_up(static_cast<size_t>(f) * d * 2, 256) : nullptr;
  char* dy_t = kt ? w_t + align_up(static_cast<size_t>(d) * 2 * f * 2, 256) : nullptr;
  const int64_t k_dx = w_up ? 2 * f : f;    // dx contracts over [dg | du], or dg alone (STEM)
  if (kt) {
    HIPCALL(transpose_bf16(w_down, d, f, f, wd_t, d, d, s));
    HIPCALL(transpose_bf16(w_gate, f, d, d, w_t, f, k_dx, s));
    if (w_up) HIPCALL(transpose_bf16(w_up, f, d, d, w_t + f * 2, f, k_dx, s));
    HIPCALL(transpose_bf16(dy, n, d, d, dy_t, round64(n), round64(n), s));
    if (max_unique > 0) {
      const int64_t chunks = (n + kSegChunk - 1) / kSegChunk;
      float* first = reinterpret_cast<float*>(seg_ws);
      HIPCALL(dh_seg_kt(n, d, f, dy, wd_t, saved_g, saved_u, dgu, sorted_pos, inv, seg_start,
                        n_unique, max_unique, d_rows, first, first + chunks * f, s, err));
      HIPCALL(launch_segment_sum_fixup(n, f, sorted_pos, inv, seg_start, n_unique, max_unique,
                                       d_rows, seg_ws, s, err));
    } else {
      HIPCALL(dh_act_kt(n, d, f, dy, wd_t, saved_g, saved_u, dgu, nullptr, s));
    }
  } else {
    HIPCALL(dh_act<T>(n, d, f, dy, w_down, saved_g, saved_u, dgu, nullptr, s));
    if (n > 0)
      HIPCALL(launch_segment_sum(dtype, dgu, 2 * f, f, n, f, sorted_pos, inv, seg_start, n_unique,
                                 max_unique, d_rows, seg_ws, s, err));
  }
  if (rows_event) HIPCALL(hipEventRecord(rows_event, s));   // d_rows complete
  // h for dW_down: the forward's, or recomputed from the saved g and u into
  // the n x f fp32 region of the workspace
  const void* h = saved_h;
  if (!h && n > 0) {
    HIPCALL(recompute_h<T>(n, f, saved_g, saved_u, aux, s));
    h = aux;
  }
  if (kt) {
    HIPCALL(dwdown_bwd_kt(n, d, f, dy_t, round64(n), h, dw_down, s));
    // x^T into dy^T's buffer (dW_down has read it, in stream order); the
    // weight gradients come out of x^T [dg | du] transposed
    HIPCALL(transpose_bf16(x, n, d, d, dy_t, round64(n), round64(n), s));
    HIPCALL(dwgu_bwd_kt(n, d, f, dy_t, round64(n), dgu, dw_gate, dw_up, fz, s));
  } else {
    HIPCALL(dwdown_bwd<T>(n, d, f, dy, h, dw_down, s));
    HIPCALL(dwgu_bwd<T>(n, d, f, dgu, x, dw_gate, dw_up, fz, s));
  }
  if (kt) HIPCALL(dx_bwd_kt(n, d, k_dx, dgu, 2 * f, w_t, dx, out_dtype, s));
  else HIPCALL(dx_bwd<T>(n, d, f, dgu, w_gate, w_up, dx, out_dtype, s));
  return STAPLE_OK;
}

extern "C" {

staple_status_t staple_ffn_bwd_table_grad(
    int64_t n, int64_t d, int64_t f, int32_t dtype, int32_t out_dtype, const void* dy,
    const void* x, const void* w_gate, const void* w_up, const void* w_down, const void* saved_g,
    const void* saved_u, const void* saved_h, const int32_t* sorted_pos, const int32_t* inv,
    const int32_t* seg_start,
    const int32_t* n_unique, int64_t max_unique, float* d_rows, void* dx, float* dw_gate,
    float* dw_up, float* dw_down, int32_t freeze_up, void* ws, size_t ws_bytes, void* rows_event,
    void* stream) {
  if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return STAPLE_ERR_UNSUPPORTED;
  if (!ffn_shape_ok(n, d, f, dtype)) return STAPLE_ERR_UNSUPPORTED;
  // w_up null: the STEM layer (no up-projection, so no dw_up either)
  const bool fz = freeze_up != 0 || !w_up;
  REQUIRE(w_gate && w_down && dw_gate && dw_down && (fz || dw_up));
  REQUIRE(seg_start && n_unique && max_unique >= 0 && max_unique <= n);
  REQUIRE(aligned16(w_gate) && (!w_up || aligned16(w_up)) && aligned16(w_down) &&
          aligned16(dw_gate) && aligned16(dw_down) && (fz || aligned16(dw_up)));
  if (n > 0) {
    REQUIRE(dy && x && saved_g && saved_u && sorted_pos && inv && d_rows && dx);
    REQUIRE(aligned16(dy) && aligned16(x) && aligned16(saved_g) && aligned16(saved_u) &&
            (!saved_h || aligned16(saved_h)) && aligned16(dx) && aligned16(d_rows));
    if (ws_bytes < staple_ffn_bwd_workspace_bytes(n, d, f, dtype)) return STAPLE_ERR_WORKSPACE;
    REQUIRE(ws && aligned16(ws));
  }
  GET_ERR(err);
  hipStream_t s = S(stream);
  if (dtype == STAPLE_BF16)
    return bwd_impl<bf16_t>(n, d, f, dtype, out_dtype, dy, x, w_gate, w_up, w_down, saved_g,
                            saved_u, saved_h, sorted_pos, inv, seg_start, n_unique, max_unique,
                            d_rows, dx, dw_gate, dw_up, dw_down, fz, ws,
                            static_cast<hipEvent_t>(rows_event), s, err);
  return bwd_impl<float>(n, d, f, dtype, out_dtype, dy, x, w_gate, w_up, w_down, saved_g, saved_u,
                         saved_h, sorted_pos, inv, seg_start, n_unique, max_unique, d_rows, dx,
                         dw_gate, dw_up, dw_down, fz, ws, static_cast<hipEvent_t>(rows_event), s,
                         err);
}

}  // extern "C"
