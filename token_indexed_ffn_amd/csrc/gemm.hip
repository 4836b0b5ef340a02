// MFMA GEMM for the three dense contractions of the augmented FFN and their
// gradients, with the layer's elementwise work fused into the epilogues.
//
//   C[m, n] = sum_k A[m, k] * B[k, n]      (fp32 accumulation)
//
// Operands are either "K-major" (each row of the operand is contiguous along
// k, e.g. x [N x d] or W_gate [f x d]) or "MN-major" (contiguous along m or n,
// e.g. dy^T when contracting over tokens).  Tiles of 128 bytes of k per row
// are staged in LDS in K-major order with a 16-byte-chunk XOR swizzle, so the
// MFMA fragment reads are one 16-byte LDS read per lane either way; MN-major
// tiles are transposed in registers (4 k x 8 elements) on their way to LDS.
//
// bf16 uses v_mfma_f32_32x32x16_bf16 (8 bf16 of k per lane).  fp32 uses
// v_mfma_f32_32x32x2f32 eight times over the same 8-element fragments: lane
// half h supplies k = 8h + j to the j-th instruction, for A and B alike, so
// the contraction covers all 16 k of the group.
//
// Epilogues:
//   Store   - C to fp32 or bf16 (optionally split by rows into two buffers).
//   GateUp  - the B rows interleave W_gate and W_up in 32-row groups, so one
//             wave holds g and a = W_up x for the same (token, feature); the
//             epilogue reads the token's table row, forms u = a + E[t] and
//             h = silu(g) * u (STAPLE abstract: the up-projection is kept and
//             the embedding added as a residual path) and stores h (and g, u
//             for the backward when requested).
//   DhAct   - C is dh = dy W_down; the epilogue reads saved g, u and writes
//             dg = dh * u * silu'(g) and du = dh * silu(g) side by side.
#include <type_traits>

#include "common.h"

namespace staple {

enum EpiKind { kEpiStore = 0, kEpiGateUp = 1, kEpiDhAct = 2 };

struct GemmArgs {
  int64_t M, N, K;
  // A operand.  K-major: A(m,k) = a0[row(m) * lda + k], row(m) = a_rows ? a_rows[m] : m.
  // MN-major: A(m,k) = (k < a_split ? a0 + k*lda : a1 + (k-a_split)*lda)[m].
  const void* a0;
  const void* a1;
  int64_t lda;
  int64_t a_split;
  const int32_t* a_rows;
  // B operand.  K-major: B(k,n) = (n < b_split ? b0 + n*ldb : b1 + (n-b_split)*ldb)[k].
  // MN-major: B(k,n) = (k < b_split ? b0 + k*ldb : b1 + (k-b_split)*ldb)[n].
  // GateUp: K-major with n in 64-row groups: rows 0-31 of a group are W_gate
  // rows, rows 32-63 the W_up rows of the same 32 features.
  const void* b0;
  const void* b1;
  int64_t ldb;
  int64_t b_split;
  // Store: C(m,n) -> (m < c_split ? c0 + m*ldc : c1 + (m-c_split)*ldc)[n]
  void* c0;
  void* c1;
  int64_t ldc;
  int64_t c_split;
  // GateUp
  const void* rows;
  const int32_t* row_index;
  int64_t n_rows;
  int64_t d_ff;
  void* h_out;
  void* g_out;
  void* u_out;
  // DhAct
  const void* g_in;
  const void* u_in;
  void* dgu_out;
  int* err;
};

constexpr int kGemmThreads = 256;
constexpr int kRowBytes = 128;  // bytes of k per LDS tile row and stage

__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ (row & 7)) << 4); }

// ---------------------------------------------------------------------------
// Tile loaders: global -> registers -> LDS
// ---------------------------------------------------------------------------
// K-major operand tile of R rows x 128 bytes.  Thread t moves 16-byte chunk
// (t & 7) of rows (t >> 3) + 32 i.
template <int R>
struct KMajorTile {
  static constexpr int kPer = R * 8 / kGemmThreads;
  const char* row_ptr[kPer];
  uint4 reg[kPer];

  __device__ __forceinline__ void load(int64_t k_byte) {
    const int c = threadIdx.x & 7;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      reg[i] = *reinterpret_cast<const uint4*>(row_ptr[i] + k_byte + c * 16);
  }
  __device__ __forceinline__ void store(char* lds) const {
    const int c = threadIdx.x & 7;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int r = (threadIdx.x >> 3) + 32 * i;
      *reinterpret_cast<uint4*>(lds + swz(r, c)) = reg[i];
    }
  }
  __device__ __forceinline__ static int row_of(int i) { return (threadIdx.x >> 3) + 32 * i; }
};

// MN-major operand tile: BK k-rows x R contiguous elements.  A unit is 4
// consecutive k x one 16-byte vector; it is transposed in registers into
// K-major pieces (8 bytes per row for bf16, 16 bytes for fp32).
template <typename T, int R>
struct MNMajorTile {
  static constexpr int kVec = 16 / sizeof(T);                 // elements per 16-byte vector
  static constexpr int kBK = kRowBytes / sizeof(T);           // k per stage
  static constexpr int kChunks = R / kVec;                    // vectors per k-row
  static constexpr int kUnits = (kBK / 4) * kChunks;
  static constexpr int kPer = (kUnits + kGemmThreads - 1) / kGemmThreads;
  uint4 reg[kPer][4];

  // base(k) returns the element pointer of k-row k (already offset to the
  // tile's first column) or nullptr when the row lies outside the operand;
  // `cols` is the number of valid columns in the tile.
  template <typename BaseFn>
  __device__ __forceinline__ void load(int64_t k0, BaseFn base, int64_t cols) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = threadIdx.x + kGemmThreads * i;
      const int rc = q % kChunks;
      const int kq = q / kChunks;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const T* rowp = (q < kUnits) ? base(k0 + kq * 4 + kk) : nullptr;
        if (rowp != nullptr && static_cast<int64_t>(rc) * kVec < cols)
          reg[i][kk] = *reinterpret_cast<const uint4*>(rowp + rc * kVec);
        else
          reg[i][kk] = make_uint4(0, 0, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = threadIdx.x + kGemmThreads * i;
      if (q >= kUnits) continue;
      const int rc = q % kChunks;
      const int kq = q / kChunks;
      if constexpr (sizeof(T) == 2) {
        const uint32_t* v0 = reinterpret_cast<const uint32_t*>(&reg[i][0]);
        const uint32_t* v1 = reinterpret_cast<const uint32_t*>(&reg[i][1]);
        const uint32_t* v2 = reinterpret_cast<const uint32_t*>(&reg[i][2]);
        const uint32_t* v3 = reinterpret_cast<const uint32_t*>(&reg[i][3]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // elements 2j (low halves) and 2j+1 (high halves) of the four k-rows
          uint2 lo, hi;
          lo.x = (v0[j] & 0xffffu) | (v1[j] << 16);
          lo.y = (v2[j] & 0xffffu) | (v3[j] << 16);
          hi.x = (v0[j] >> 16) | (v1[j] & 0xffff0000u);
          hi.y = (v2[j] >> 16) | (v3[j] & 0xffff0000u);
          const int r0 = rc * 8 + 2 * j;
          const int r1 = r0 + 1;
          *reinterpret_cast<uint2*>(lds + swz(r0, kq >> 1) + (kq & 1) * 8) = lo;
          *reinterpret_cast<uint2*>(lds + swz(r1, kq >> 1) + (kq & 1) * 8) = hi;
        }
      } else {
        const uint32_t* v0 = reinterpret_cast<const uint32_t*>(&reg[i][0]);
        const uint32_t* v1 = reinterpret_cast<const uint32_t*>(&reg[i][1]);
        const uint32_t* v2 = reinterpret_cast<const uint32_t*>(&reg[i][2]);
        const uint32_t* v3 = reinterpret_cast<const uint32_t*>(&reg[i][3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint4 w = make_uint4(v0[e], v1[e], v2[e], v3[e]);
          *reinterpret_cast<uint4*>(lds + swz(rc * 4 + e, kq)) = w;
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// MFMA step over one 16-wide k group
// ---------------------------------------------------------------------------
template <typename T, int TM, int TN>
struct Mma;

template <int TM, int TN>
struct Mma<bf16_t, TM, TN> {
  static constexpr int kGroups = 4;  // 64 bf16 of k per stage
  __device__ __forceinline__ static void step(const char* As, const char* Bs, int a_row0, int b_row0,
                                              int kg, f32x16_t (&acc)[TM][TN]) {
    const int lane = threadIdx.x & 63;
    const int chunk = kg * 2 + (lane >> 5);
    bf16x8_t a[TM], b[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = a_row0 + i * 32 + (lane & 31);
      a[i] = *reinterpret_cast<const bf16x8_t*>(As + swz(r, chunk));
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = b_row0 + j * 32 + (lane & 31);
      b[j] = *reinterpret_cast<const bf16x8_t*>(Bs + swz(r, chunk));
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
};

template <int TM, int TN>
struct Mma<float, TM, TN> {
  static constexpr int kGroups = 2;  // 32 fp32 of k per stage
  __device__ __forceinline__ static void step(const char* As, const char* Bs, int a_row0, int b_row0,
                                              int kg, f32x16_t (&acc)[TM][TN]) {
    const int lane = threadIdx.x & 63;
    const int chunk = kg * 4 + (lane >> 5) * 2;
    float4 a[TM][2], b[TN][2];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = a_row0 + i * 32 + (lane & 31);
      a[i][0] = *reinterpret_cast<const float4*>(As + swz(r, chunk));
      a[i][1] = *reinterpret_cast<const float4*>(As + swz(r, chunk + 1));
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = b_row0 + j * 32 + (lane & 31);
      b[j][0] = *reinterpret_cast<const float4*>(Bs + swz(r, chunk));
      b[j][1] = *reinterpret_cast<const float4*>(Bs + swz(r, chunk + 1));
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const float av[8] = {a[i][0].x, a[i][0].y, a[i][0].z, a[i][0].w,
                             a[i][1].x, a[i][1].y, a[i][1].z, a[i][1].w};
        const float bv[8] = {b[j][0].x, b[j][0].y, b[j][0].z, b[j][0].w,
                             b[j][1].x, b[j][1].y, b[j][1].z, b[j][1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[e], bv[e], acc[i][j], 0, 0, 0);
      }
  }
};

// Row of output element r (0..15) of a 32x32 MFMA tile for this lane.
__device__ __forceinline__ int mfma_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, bool AK, bool BK, int EPI, typename OutT>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(GemmArgs p) {
  constexpr int WM = BM / 2, WN = BN / 2;   // 2 x 2 waves
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int kBK = kRowBytes / sizeof(T);
  static_assert(EPI != kEpiGateUp || WN % 64 == 0, "gate/up pairing needs 64-column wave tiles");

  __shared__ __attribute__((aligned(16))) char smem[2 * (BM + BN) * kRowBytes];
  char* As0 = smem;
  char* Bs0 = smem + BM * kRowBytes;
  constexpr int kStage = (BM + BN) * kRowBytes;

  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * BM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.y) * BN;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  // ---- operand addressing ----
  using ATile = typename std::conditional<AK, KMajorTile<BM>, MNMajorTile<T, BM>>::type;
  using BTile = typename std::conditional<BK, KMajorTile<BN>, MNMajorTile<T, BN>>::type;
  ATile at;
  BTile bt;
  if constexpr (AK) {
#pragma unroll
    for (int i = 0; i < ATile::kPer; ++i) {
      int64_t m = m0 + ATile::row_of(i);
      if (m > p.M - 1) m = p.M - 1;
      const int64_t row = p.a_rows ? static_cast<int64_t>(p.a_rows[m]) : m;
      at.row_ptr[i] = static_cast<const char*>(p.a0) + row * p.lda * sizeof(T);
    }
  }
  if constexpr (BK) {
#pragma unroll
    for (int i = 0; i < BTile::kPer; ++i) {
      int64_t n = n0 + BTile::row_of(i);
      if (n > p.N - 1) n = p.N - 1;
      const char* base;
      if constexpr (EPI == kEpiGateUp) {
        const int64_t feat = (n >> 6) * 32 + (n & 31);
        base = static_cast<const char*>((n & 32) ? p.b1 : p.b0) + feat * p.ldb * sizeof(T);
      } else {
        base = n < p.b_split ? static_cast<const char*>(p.b0) + n * p.ldb * sizeof(T)
                             : static_cast<const char*>(p.b1) + (n - p.b_split) * p.ldb * sizeof(T);
      }
      bt.row_ptr[i] = base;
    }
  }
  const int64_t a_cols = p.M - m0;  // valid m in this tile (MN-major A)
  const int64_t b_cols = p.N - n0;  // valid n in this tile (MN-major B)
  auto a_base = [&](int64_t k) -> const T* {
    if (k >= p.K) return nullptr;
    const T* b = k < p.a_split ? static_cast<const T*>(p.a0) + k * p.lda
                               : static_cast<const T*>(p.a1) + (k - p.a_split) * p.lda;
    return b + m0;
  };
  auto b_base = [&](int64_t k) -> const T* {
    if (k >= p.K) return nullptr;
    const T* b = k < p.b_split ? static_cast<const T*>(p.b0) + k * p.ldb
                               : static_cast<const T*>(p.b1) + (k - p.b_split) * p.ldb;
    return b + n0;
  };
  auto load_tiles = [&](int64_t kt) {
    const int64_t k0 = kt * kBK;
    if constexpr (AK) at.load(k0 * static_cast<int64_t>(sizeof(T)));
    else at.load(k0, a_base, a_cols);
    if constexpr (BK) bt.load(k0 * static_cast<int64_t>(sizeof(T)));
    else bt.load(k0, b_base, b_cols);
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int64_t nk = (p.K + kBK - 1) / kBK;
  load_tiles(0);
  at.store(As0);
  bt.store(Bs0);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = static_cast<int>(kt & 1);
    if (kt + 1 < nk) load_tiles(kt + 1);
    const char* As = As0 + cur * kStage;
    const char* Bs = Bs0 + cur * kStage;
#pragma unroll
    for (int kg = 0; kg < Mma<T, TM, TN>::kGroups; ++kg)
      Mma<T, TM, TN>::step(As, Bs, wm * WM, wn * WN, kg, acc);
    if (kt + 1 < nk) {
      at.store(As0 + (cur ^ 1) * kStage);
      bt.store(Bs0 + (cur ^ 1) * kStage);
    }
    __syncthreads();
  }

  // ---- epilogues ----
  const int col_in = lane & 31;
  if constexpr (EPI == kEpiStore) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + wn * WN + j * 32 + col_in;
        if (n >= p.N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = m0 + wm * WM + i * 32 + mfma_row(r, lane);
          if (m >= p.M) continue;
          void* cb = m < p.c_split ? p.c0 : p.c1;
          const int64_t mm = m < p.c_split ? m : m - p.c_split;
          Elem<OutT>::store(cb, mm * p.ldc + n, acc[i][j][r]);
        }
      }
  } else if constexpr (EPI == kEpiGateUp) {
    const int64_t f = p.d_ff;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < TN / 2; ++q) {
        const int64_t feat = (n0 + wn * WN + q * 64) / 2 + col_in;
        if (feat >= f) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = m0 + wm * WM + i * 32 + mfma_row(r, lane);
          if (m >= p.M) continue;
          const int64_t tok = p.a_rows ? static_cast<int64_t>(p.a_rows[m]) : m;
          const int64_t ri = p.row_index[tok];
          float e = 0.0f;
          if (ri >= 0 && ri < p.n_rows) e = Elem<T>::load(p.rows, ri * f + feat);
          else flag_index_error(p.err);
          const float g = acc[i][2 * q][r];
          const float u = acc[i][2 * q + 1][r] + e;
          const float h = g * sigmoidf_(g) * u;
          const int64_t o = tok * f + feat;
          Elem<T>::store(p.h_out, o, h);
          if (p.g_out) Elem<T>::store(p.g_out, o, g);
          if (p.u_out) Elem<T>::store(p.u_out, o, u);
        }
      }
  } else {  // kEpiDhAct: C = dh (M = tokens, N = d_ff)
    const int64_t f = p.N;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + wn * WN + j * 32 + col_in;
        if (n >= f) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = m0 + wm * WM + i * 32 + mfma_row(r, lane);
          if (m >= p.M) continue;
          const float dh = acc[i][j][r];
          const float g = Elem<T>::load(p.g_in, m * f + n);
          const float u = Elem<T>::load(p.u_in, m * f + n);
          const float s = sigmoidf_(g);
          const float du = dh * g * s;
          const float dg = dh * u * s * (1.0f + g * (1.0f - s));
          Elem<T>::store(p.dgu_out, m * 2 * f + n, dg);
          Elem<T>::store(p.dgu_out, m * 2 * f + f + n, du);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, bool AK, bool BK, int EPI, typename OutT>
static hipError_t run(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>((a.M + BM - 1) / BM), static_cast<unsigned>((a.N + BN - 1) / BN));
  gemm_kernel<T, BM, BN, AK, BK, EPI, OutT><<<grid, dim3(kGemmThreads), 0, s>>>(a);
  return hipGetLastError();
}

template <typename T>
static GemmArgs blank() {
  GemmArgs a{};
  a.a_split = a.b_split = a.c_split = INT64_MAX;
  return a;
}

// h = silu(x W_gate^T) * (x W_up^T + rows[row_index]); optional saves of g, u.
template <typename T>
hipError_t gateup_fwd(int64_t n, int64_t d, int64_t f, const void* x, const void* wg,
                      const void* wu, const void* rows, int64_t n_rows, const int32_t* row_index,
                      void* h, void* g_out, void* u_out, hipStream_t s, int* err) {
  GemmArgs a = blank<T>();
  a.M = n; a.N = 2 * f; a.K = d;
  a.a0 = x; a.lda = d;
  a.b0 = wg; a.b1 = wu; a.ldb = d;
  a.rows = rows; a.row_index = row_index; a.n_rows = n_rows; a.d_ff = f;
  a.h_out = h; a.g_out = g_out; a.u_out = u_out; a.err = err;
  return run<T, 128, 128, true, true, kEpiGateUp, T>(a, s);
}

// y = h W_down^T
template <typename T>
hipError_t down_fwd(int64_t n, int64_t d, int64_t f, const void* h, const void* wd, void* y,
                    int out_dtype, hipStream_t s) {
  GemmArgs a = blank<T>();
  a.M = n; a.N = d; a.K = f;
  a.a0 = h; a.lda = f;
  a.b0 = wd; a.ldb = f;
  a.c0 = y; a.ldc = d;
  if (out_dtype == STAPLE_F32) return run<T, 128, 128, true, true, kEpiStore, float>(a, s);
  return run<T, 128, 128, true, true, kEpiStore, bf16_t>(a, s);
}

// dh = dy W_down; dgu[:, :f] = dg, dgu[:, f:] = du
template <typename T>
hipError_t dh_act(int64_t n, int64_t d, int64_t f, const void* dy, const void* wd, const void* g,
                  const void* u, void* dgu, hipStream_t s) {
  GemmArgs a = blank<T>();
  a.M = n; a.N = f; a.K = d;
  a.a0 = dy; a.lda = d;
  a.b0 = wd; a.ldb = f;          // B(k=j, n) = W_down[j, n]
  a.g_in = g; a.u_in = u; a.dgu_out = dgu;
  return run<T, 128, 128, true, false, kEpiDhAct, T>(a, s);
}

// dx = dg W_gate + du W_up  (K = 2f over the concatenated [dg | du])
template <typename T>
hipError_t dx_bwd(int64_t n, int64_t d, int64_t f, const void* dgu, const void* wg,
                  const void* wu, void* dx, int out_dtype, hipStream_t s) {
  GemmArgs a = blank<T>();
  a.M = n; a.N = d; a.K = 2 * f;
  a.a0 = dgu; a.lda = 2 * f;
  a.b0 = wg; a.b1 = wu; a.ldb = d; a.b_split = f;
  a.c0 = dx; a.ldc = d;
  if (out_dtype == STAPLE_F32) return run<T, 128, 128, true, false, kEpiStore, float>(a, s);
  return run<T, 128, 128, true, false, kEpiStore, bf16_t>(a, s);
}

// dw_down = dy^T h   (M = d, N = f, K = tokens)
template <typename T>
hipError_t dwdown_bwd(int64_t n, int64_t d, int64_t f, const void* dy, const void* h, float* dwd,
                      hipStream_t s) {
  GemmArgs a = blank<T>();
  a.M = d; a.N = f; a.K = n;
  a.a0 = dy; a.lda = d;
  a.b0 = h; a.ldb = f;
  a.c0 = dwd; a.ldc = f;
  return run<T, 128, 128, false, false, kEpiStore, float>(a, s);
}

// [dw_gate; dw_up] = [dg | du]^T x   (M = 2f, or f when the up-projection is frozen)
template <typename T>
hipError_t dwgu_bwd(int64_t n, int64_t d, int64_t f, const void* dgu, const void* x, float* dwg,
                    float* dwu, bool freeze_up, hipStream_t s) {
  GemmArgs a = blank<T>();
  a.M = freeze_up ? f : 2 * f; a.N = d; a.K = n;
  a.a0 = dgu; a.lda = 2 * f;
  a.b0 = x; a.ldb = d;
  a.c0 = dwg; a.c1 = dwu; a.ldc = d; a.c_split = f;
  return run<T, 128, 128, false, false, kEpiStore, float>(a, s);
}

#define STAPLE_INST(T)                                                                          \
  template hipError_t gateup_fwd<T>(int64_t, int64_t, int64_t, const void*, const void*,       \
                                    const void*, const void*, int64_t, const int32_t*, void*,   \
                                    void*, void*, hipStream_t, int*);                           \
  template hipError_t down_fwd<T>(int64_t, int64_t, int64_t, const void*, const void*, void*,  \
                                  int, hipStream_t);                                            \
  template hipError_t dh_act<T>(int64_t, int64_t, int64_t, const void*, const void*,           \
                                const void*, const void*, void*, hipStream_t);                  \
  template hipError_t dx_bwd<T>(int64_t, int64_t, int64_t, const void*, const void*,           \
                                const void*, void*, int, hipStream_t);                          \
  template hipError_t dwdown_bwd<T>(int64_t, int64_t, int64_t, const void*, const void*,       \
                                    float*, hipStream_t);                                       \
  template hipError_t dwgu_bwd<T>(int64_t, int64_t, int64_t, const void*, const void*, float*, \
                                  float*, bool, hipStream_t);

STAPLE_INST(bf16_t)
STAPLE_INST(float)

}  // namespace staple
