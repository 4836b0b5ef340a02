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
// Epilogues stage each wave's accumulators through LDS, 32 rows at a time,
// so every global access of the epilogue is a 16-byte vector along a row:
//   Store   - C to fp32 or bf16 (optionally split by rows into two buffers).
//   StoreT  - C^T: element (m, n) to row n, column m (optionally split by
//             columns n into two buffers), 8 consecutive m per store.
//   GateUp  - the B rows interleave W_gate and W_up in 32-row groups, so one
//             wave holds g and a = W_up x for the same (token, feature); the
//             epilogue reads the token's table row, forms u = a + E[t] and
//             h = silu(g) * u (STAPLE abstract: the up-projection is kept and
//             the embedding added as a residual path) and stores h (and g, u
//             for the backward when requested).
//   GateStem- C is g = W_gate x alone (the STEM layer, which has no
//             up-projection: the token's table row takes its place, STAPLE
//             abstract and Table 1); the epilogue reads the table row e and
//             stores h = silu(g) * e (and g, u = e when requested).
//   DhAct   - C is dh = dy W_down; the epilogue reads saved g, u and writes
//             dg = dh * u * silu'(g) and du = dh * silu(g) side by side, and
//             optionally du once more in fp32, unrounded, for the table-row
//             segment sum.
//   DhSeg   - DhAct over the tokens in sorted order (row p of the tile is
//             sorted position p, token sorted_pos[p]): g, u and [dg | du]
//             are addressed by token, and the epilogue also sums the fp32 du
//             over each run of equal IDs inside every 32-position chunk, in
//             position order, writing a segment whole to its table-row
//             gradient and a segment that crosses a chunk boundary to the
//             chunk's first / last partial (the segment sum's chunk pass,
//             done without the fp32 du ever leaving the CU).
#include <type_traits>

#include "common.h"

namespace staple {

enum EpiKind { kEpiStore = 0, kEpiGateUp = 1, kEpiDhAct = 2, kEpiGateStem = 3, kEpiStoreT = 4,
               kEpiDhSeg = 5 };

struct GemmArgs {
  int64_t M, N, K;
  // A operand.  K-major: A(m,k) = a0[row(m) * lda + k], row(m) = a_rows ? a_rows[m] : m
  // (a_rows entries outside [0, a_rows_bound) set the error word; row 0 is read
  // instead and the gate/up epilogue stores nothing for them).
  // MN-major: A(m,k) = (k < a_split ? a0 + k*lda : a1 + (k-a_split)*lda)[m].
  const void* a0;
  const void* a1;
  int64_t lda;
  int64_t a_split;
  const int32_t* a_rows;
  int64_t a_rows_bound;
  // B operand.  K-major: B(k,n) = (n < b_split ? b0 + n*ldb : b1 + (n-b_split)*ldb)[k].
  // MN-major: B(k,n) = (k < b_split ? b0 + k*ldb : b1 + (k-b_split)*ldb)[n].
  // GateUp: K-major with n in 64-row groups: rows 0-31 of a group are W_gate
  // rows, rows 32-63 the W_up rows of the same 32 features.
  const void* b0;
  const void* b1;
  int64_t ldb;
  int64_t b_split;
  // Store: C(m,n) -> (m < c_split ? c0 + m*ldc : c1 + (m-c_split)*ldc)[n]
  // StoreT: C(m,n) -> (n < c_split ? c0 + n*ldc : c1 + (n-c_split)*ldc)[m]  (M a multiple of 8)
  void* c0;
  void* c1;
  int64_t ldc;
  int64_t c_split;
  // GateUp, GateStem (GateStem: B is W_gate alone, N = d_ff)
  const void* rows;
  const int32_t* row_index;
  int64_t n_rows;
  int64_t d_ff;
  void* h_out;
  void* g_out;
  void* u_out;
  // DhAct (du32_out: optional fp32 copy of du, [M x N] row-major)
  const void* g_in;
  const void* u_in;
  void* dgu_out;
  float* du32_out;
  int* err;
  // Optional device-side limits (counts known only on the device, e.g. the
  // batch's unique IDs): M and K become min(M, *m_dev) and min(K, *k_dev);
  // the grid is sized for the host M and the tiles past the device M leave.
  // k_dev is only used with MN-major operands (rows past K read zeros).
  const int32_t* m_dev;
  const int32_t* k_dev;
  // DhSeg: sorted positions (also the A operand's rows), the inverse map,
  // the segment offsets [U + 1], the device unique count and the row buffer
  // bound, the table-row gradient [max_unique x N] and the chunk partials
  // first / last [chunks of 32 positions x N]
  const int32_t* seg_inv;
  const int32_t* seg_start;
  const int32_t* seg_nu;
  int64_t seg_max_unique;
  float* seg_rows;
  float* seg_first;
  float* seg_last;
};

constexpr int kRowBytes = 128;  // bytes of k per LDS tile row and stage
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;

// One 16-byte-per-lane global -> LDS load (global_load_lds_dwordx4: lane l
// writes LDS bytes [dst + 16 l, +16), dst wave-uniform, passed in M0).  It is
// issued from inline asm so that the compiler does not count it among the
// LDS-counter events: with such a load in flight it would otherwise wait for
// every outstanding LDS read (lgkmcnt(0)) before each MFMA group instead of
// only the ones the group needs.  The asm has no register outputs (the data
// goes to LDS); its completion is waited for by hand (vmcnt) before the
// barrier that publishes the stage, as for the builtin form.
__device__ __forceinline__ void dma16(const void* src, lds_void* dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst)));
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

// K-major LDS tile rows hold RB bytes of k: 128 (8 chunks of 16 bytes) or 64
// (4 chunks).  The chunk index is XORed with a function of the row so that the
// MFMA fragment reads (consecutive rows, one chunk) spread over the LDS banks:
// with 128-byte rows, bits 0-2 and 3-5 of the row (which also spreads the
// transposed stores of register-staged MN-major tiles, rows 8 apart); with
// 64-byte rows, bits 2-3 (four rows share a 256-byte bank window).
template <int RB>
__device__ __forceinline__ int row_swizzle(int row) {
  if constexpr (RB == 128) return (row & 7) ^ ((row >> 3) & 7);
  else return (row >> 2) & 3;
}
template <int RB = kRowBytes>
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * RB + ((chunk ^ row_swizzle<RB>(row)) << 4);
}

// ---------------------------------------------------------------------------
// Tile loaders: global -> registers -> LDS
// ---------------------------------------------------------------------------
// K-major operand tile of R rows x RB bytes of k.
template <int R, int NT, int RB>
struct KMajorTile {
  // Direct global -> LDS loads: the i-th 16-byte load instruction of wave w
  // fills the 1 KB of LDS rows [RPI (i NW + w), RPI (i NW + w) + RPI) of the
  // tile (RPI = 1024 / RB rows; lane l at byte 16 l), so lane l fetches row
  // RPI (i NW + w) + l / LPR (LPR = RB / 16 lanes per row) and, for the
  // swizzled position (l % LPR), the logical chunk (l % LPR) ^ swizzle(row).
  static constexpr int kNW = NT / 64;
  static constexpr int kLPR = RB / 16;
  static constexpr int kRPI = 1024 / RB;
  static constexpr int kPer = R / (kRPI * kNW);
  static_assert(kPer * kRPI * kNW == R, "tile shape");
  const char* row_ptr[kPer];   // row start, then (init_chunks) plus the lane's chunk offset

  __device__ __forceinline__ static int row_of(int i) {
    return kRPI * (i * kNW + (threadIdx.x >> 6)) + (threadIdx.x & 63) / kLPR;
  }
  __device__ __forceinline__ void init_chunks() {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int row = row_of(i);
      const int phys = threadIdx.x % kLPR;
      row_ptr[i] += (phys ^ row_swizzle<RB>(row)) << 4;
    }
  }
  // `lds` is the tile's LDS buffer (local address space).
  __device__ __forceinline__ void load(int64_t k_byte, lds_char* lds) const {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      dma16(static_cast<const void*>(row_ptr[i] + k_byte),
            static_cast<lds_void*>(lds + (i * kNW + w) * 1024));
  }
  // Register-staged form of the same loads: load_regs fetches the 16-byte
  // pieces into reg[], store_piece(i) writes piece i where load() would have.
  u32x4_t reg[kPer];
  __device__ __forceinline__ void load_regs(int64_t k_byte) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) reg[i] = *reinterpret_cast<const u32x4_t*>(row_ptr[i] + k_byte);
  }
  __device__ __forceinline__ void store_piece(lds_char* lds, int i) const {
    *reinterpret_cast<lds_u32x4_t*>(lds + (i * kNW + (threadIdx.x >> 6)) * 1024 + (threadIdx.x & 63) * 16) = reg[i];
  }
};

// MN-major operand tile: BK k-rows x R contiguous elements.  A unit is 4
// consecutive k x one 16-byte vector; it is transposed in registers into
// K-major pieces (8 bytes per row for bf16, 16 bytes for fp32).
template <typename T, int R, int NT>
struct MNMajorTile {
  static constexpr int kVec = 16 / sizeof(T);                 // elements per 16-byte vector
  static constexpr int kBK = kRowBytes / sizeof(T);           // k per stage
  static constexpr int kChunks = R / kVec;                    // vectors per k-row
  static constexpr int kUnits = (kBK / 4) * kChunks;
  static constexpr int kPer = (kUnits + NT - 1) / NT;
  uint4 reg[2][kPer][4];

  // base(k) returns the element pointer of k-row k (already offset to the
  // tile's first column) or nullptr when the row lies outside the operand;
  // `cols` is the number of valid columns in the tile.
  template <int S, typename BaseFn>
  __device__ __forceinline__ void load(int64_t k0, BaseFn base, int64_t cols) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = threadIdx.x + NT * i;
      const int rc = q % kChunks;
      const int kq = q / kChunks;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const T* rowp = (q < kUnits) ? base(k0 + kq * 4 + kk) : nullptr;
        if (rowp != nullptr && static_cast<int64_t>(rc) * kVec < cols)
          reg[S][i][kk] = *reinterpret_cast<const uint4*>(rowp + rc * kVec);
        else
          reg[S][i][kk] = make_uint4(0, 0, 0, 0);
      }
    }
  }

  template <int S>
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = threadIdx.x + NT * i;
      if (q >= kUnits) continue;
      const int rc = q % kChunks;
      const int kq = q / kChunks;
      const uint32_t* v0 = reinterpret_cast<const uint32_t*>(&reg[S][i][0]);
      const uint32_t* v1 = reinterpret_cast<const uint32_t*>(&reg[S][i][1]);
      const uint32_t* v2 = reinterpret_cast<const uint32_t*>(&reg[S][i][2]);
      const uint32_t* v3 = reinterpret_cast<const uint32_t*>(&reg[S][i][3]);
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // elements 2j (low halves) and 2j+1 (high halves) of the four k-rows
          uint2 lo, hi;
          lo.x = (v0[j] & 0xffffu) | (v1[j] << 16);
          lo.y = (v2[j] & 0xffffu) | (v3[j] << 16);
          hi.x = (v0[j] >> 16) | (v1[j] & 0xffff0000u);
          hi.y = (v2[j] >> 16) | (v3[j] & 0xffff0000u);
          const int r0 = rc * 8 + 2 * j;
          *reinterpret_cast<uint2*>(lds + swz(r0, kq >> 1) + (kq & 1) * 8) = lo;
          *reinterpret_cast<uint2*>(lds + swz(r0 + 1, kq >> 1) + (kq & 1) * 8) = hi;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint4 w = make_uint4(v0[e], v1[e], v2[e], v3[e]);
          *reinterpret_cast<uint4*>(lds + swz(rc * 4 + e, kq)) = w;
        }
      }
    }
  }
};

// bf16 MN-major operand tile loaded straight into LDS without a transpose:
// LDS keeps the operand's own layout, [KR k-rows][R elements], in 32-byte
// chunks whose index is XORed with swz_mn(k); the MFMA fragments are then read
// with the transposing LDS load (ds_read_b64_tr_b16).  The i-th load
// instruction of wave w fills 1 KB = 1024 / (2 R) k-rows; lane l covers 16
// bytes of it.  k-rows past K read a zero page so they add nothing.
__device__ const uint4 g_gemm_zero_page[1] = {};

__device__ __forceinline__ int swz_mn(int k) { return ((k & 3) << 1) | ((k >> 3) & 1); }

template <int R, int NT, int KR>
struct MNDirectTile {
  static constexpr int kNW = NT / 64;
  static constexpr int kRB = R * 2;                 // bytes per k-row
  static constexpr int kRowsPerInst = 1024 / kRB;   // k-rows per 1 KB instruction
  static constexpr int kPer = KR / kRowsPerInst / kNW;
  static_assert(kPer * kRowsPerInst * kNW == KR, "tile shape");
  int krow[kPer];        // k-row (0..KR-1) this lane fills with instruction i
  int elem[kPer];        // element offset along the row (logical, 8 elements)

  __device__ __forceinline__ void init() {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int byte = (i * kNW + w) * 1024 + l * 16;   // LDS byte in the tile
      const int k = byte / kRB;
      const int in_row = byte % kRB;
      const int phys32 = in_row >> 5, half = (in_row >> 4) & 1;
      const int c32 = phys32 ^ swz_mn(k);
      krow[i] = k;
      elem[i] = c32 * 16 + half * 8;
    }
  }
  // base(k) returns the element pointer of global k-row k offset to the tile's
  // first column, or nullptr past the end of K; `cols` is the number of valid
  // columns in the tile (a multiple of 8, so a 16-byte piece is all in or out).
  template <typename BaseFn>
  __device__ __forceinline__ const void* src(int64_t k0, BaseFn base, int64_t cols, int i) const {
    const uint16_t* rowp = base(k0 + krow[i]);
    return (rowp != nullptr && elem[i] < cols) ? static_cast<const void*>(rowp + elem[i])
                                               : static_cast<const void*>(g_gemm_zero_page);
  }
  template <typename BaseFn>
  __device__ __forceinline__ void load(int64_t k0, BaseFn base, int64_t cols, lds_char* lds) const {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      dma16(src(k0, base, cols, i), static_cast<lds_void*>(lds + (i * kNW + w) * 1024));
  }
  // Register-staged form (see KMajorTile).
  u32x4_t reg[kPer];
  template <typename BaseFn>
  __device__ __forceinline__ void load_regs(int64_t k0, BaseFn base, int64_t cols) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) reg[i] = *reinterpret_cast<const u32x4_t*>(src(k0, base, cols, i));
  }
  __device__ __forceinline__ void store_piece(lds_char* lds, int i) const {
    *reinterpret_cast<lds_u32x4_t*>(lds + (i * kNW + (threadIdx.x >> 6)) * 1024 + (threadIdx.x & 63) * 16) = reg[i];
  }
};

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s;

// 8 bf16 of k (kg*16 + 8*octet .. +7) for column `col` of an MN-major LDS tile
// with row bytes RB, read by the 16-lane group of this lane (lane & 15 = i16):
// two transposing reads, each giving 4 consecutive k of column col0 + i16.
template <int RB>
__device__ __forceinline__ bf16x8_t read_tr_frag(const lds_char* tile, int kbase, int col0) {
  const int i16 = threadIdx.x & 15;
  bf16x8_t out;
  v4s_t lo, hi;
  {
    const int k = kbase + (i16 >> 2), c = col0 + 4 * (i16 & 3);
    const lds_char* p = tile + k * RB + (((c >> 4) ^ swz_mn(k)) << 5) + (c & 15) * 2;
    lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p);
  }
  {
    const int k = kbase + 4 + (i16 >> 2), c = col0 + 4 * (i16 & 3);
    const lds_char* p = tile + k * RB + (((c >> 4) ^ swz_mn(k)) << 5) + (c & 15) * 2;
    hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p);
  }
  typedef short v8s_t __attribute__((ext_vector_type(8)));
  const v8s_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  out = __builtin_bit_cast(bf16x8_t, v);
  return out;
}

// ---------------------------------------------------------------------------
// MFMA step over one 16-wide k group
// ---------------------------------------------------------------------------
template <typename T, int TM, int TN, bool AK, bool BK, int BM, int BN, int RB>
struct Mma;

typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8;

// bf16: K-major tiles are read with one 16-byte LDS read per fragment,
// MN-major tiles (kept in the operand's own layout) with two transposing reads.
template <int TM, int TN, bool AK, bool BK, int BM, int BN, int RB>
struct Mma<bf16_t, TM, TN, AK, BK, BM, BN, RB> {
  static constexpr int kGroups = RB / 32;  // 16 bf16 of k per group
  struct Frags {
    bf16x8_t a[TM], b[TN];
  };
  // Fragment piece q of group kg: q < TM is A fragment q, else B fragment q - TM.
  __device__ __forceinline__ static void read_piece(const lds_char* As, const lds_char* Bs,
                                                    int a_row0, int b_row0, int kg, int q,
                                                    Frags& fr) {
    const int lane = threadIdx.x & 63;
    const int chunk = kg * 2 + (lane >> 5);
    const int kbase = kg * 16 + 8 * (lane >> 5);
    const int half16 = 16 * ((lane >> 4) & 1);
    if (q < TM) {
      const int i = q;
      if constexpr (AK) {
        const int r = a_row0 + i * 32 + (lane & 31);
        fr.a[i] = *reinterpret_cast<const lds_bf16x8*>(As + swz<RB>(r, chunk));
      } else {
        fr.a[i] = read_tr_frag<BM * 2>(As, kbase, a_row0 + i * 32 + half16);
      }
    } else {
      const int j = q - TM;
      if constexpr (BK) {
        const int r = b_row0 + j * 32 + (lane & 31);
        fr.b[j] = *reinterpret_cast<const lds_bf16x8*>(Bs + swz<RB>(r, chunk));
      } else {
        fr.b[j] = read_tr_frag<BN * 2>(Bs, kbase, b_row0 + j * 32 + half16);
      }
    }
  }
  __device__ __forceinline__ static void read(const lds_char* As, const lds_char* Bs, int a_row0,
                                              int b_row0, int kg, Frags& fr) {
#pragma unroll
    for (int q = 0; q < TM + TN; ++q) read_piece(As, Bs, a_row0, b_row0, kg, q, fr);
  }
  // The MFMAs of one group, after(m) called after MFMA m (in this order).
  template <typename AfterFn>
  __device__ __forceinline__ static void mma_each(const Frags& fr, f32x16_t (&acc)[TM][TN],
                                                  AfterFn after) {
#pragma unroll
    for (int m = 0; m < TM * TN; ++m) {
      const int i = m / TN, j = m % TN;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.a[i], fr.b[j], acc[i][j], 0, 0, 0);
      after(m);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // The MFMAs of one group with the TM + TN fragment reads of the next group
  // issued one after each of the first TM + TN MFMAs, in this order (each
  // next-group MFMA then finds its fragments read several MFMAs earlier).
  template <typename ReadFn>
  __device__ __forceinline__ static void mma_interleaved(const Frags& fr, f32x16_t (&acc)[TM][TN],
                                                         ReadFn read_next) {
    static_assert(TM + TN <= TM * TN, "reads spread over the MFMAs");
#pragma unroll
    for (int m = 0; m < TM * TN; ++m) {
      const int i = m / TN, j = m % TN;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.a[i], fr.b[j], acc[i][j], 0, 0, 0);
      if (m < TM + TN) read_next(m);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __device__ __forceinline__ static void mma(const Frags& fr, f32x16_t (&acc)[TM][TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.a[i], fr.b[j], acc[i][j], 0, 0, 0);
  }
  // One stage: the fragments of group kg + 1 are read while group kg's MFMAs run.
  __device__ __forceinline__ static void stage(const lds_char* As, const lds_char* Bs, int a_row0,
                                               int b_row0, f32x16_t (&acc)[TM][TN]) {
    Frags fr[2];
    read(As, Bs, a_row0, b_row0, 0, fr[0]);
#pragma unroll
    for (int kg = 0; kg < kGroups; ++kg) {
      if (kg + 1 < kGroups) read(As, Bs, a_row0, b_row0, kg + 1, fr[(kg + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the MFMAs
      mma(fr[kg & 1], acc);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

template <int TM, int TN, bool AK, bool BK, int BM, int BN, int RB>
struct Mma<float, TM, TN, AK, BK, BM, BN, RB> {
  static_assert(RB == kRowBytes, "fp32 tiles use 128-byte rows");
  static constexpr int kGroups = 2;  // 32 fp32 of k per stage
  __device__ __forceinline__ static void step(const lds_char* As, const lds_char* Bs, int a_row0,
                                              int b_row0, int kg, f32x16_t (&acc)[TM][TN]) {
    const int lane = threadIdx.x & 63;
    const int chunk = kg * 4 + (lane >> 5) * 2;
    const char* Ag = (const char*)As;
    const char* Bg = (const char*)Bs;
    float4 a[TM][2], b[TN][2];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = a_row0 + i * 32 + (lane & 31);
      a[i][0] = *reinterpret_cast<const float4*>(Ag + swz(r, chunk));
      a[i][1] = *reinterpret_cast<const float4*>(Ag + swz(r, chunk + 1));
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = b_row0 + j * 32 + (lane & 31);
      b[j][0] = *reinterpret_cast<const float4*>(Bg + swz(r, chunk));
      b[j][1] = *reinterpret_cast<const float4*>(Bg + swz(r, chunk + 1));
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
  __device__ __forceinline__ static void stage(const lds_char* As, const lds_char* Bs, int a_row0,
                                               int b_row0, f32x16_t (&acc)[TM][TN]) {
#pragma unroll
    for (int kg = 0; kg < kGroups; ++kg) step(As, Bs, a_row0, b_row0, kg, acc);
  }
};

// Output tile of this workgroup.  Workgroups are dispatched round-robin over
// the 8 XCDs, each with its own L2: the linear index is first remapped so that
// every XCD owns one contiguous range of tiles, then tiles are ordered in
// groups of 8 M-tiles that sweep the N-tiles, so the workgroups running side
// by side on one XCD share a few A and B panels in that XCD's L2.
__device__ __forceinline__ void tile_coords(int64_t tiles_m, int64_t tiles_n, int64_t& mt,
                                            int64_t& nt) {
  const int64_t total = tiles_m * tiles_n;
  int64_t b = blockIdx.x;
  if (total % 8 == 0) b = (b % 8) * (total / 8) + b / 8;
  constexpr int64_t G = 8;
  const int64_t group = b / (G * tiles_n);
  const int64_t first_m = group * G;
  const int64_t gsize = (tiles_m - first_m) < G ? (tiles_m - first_m) : G;
  const int64_t in = b - group * G * tiles_n;
  mt = first_m + in % gsize;
  nt = in / gsize;
}

// Row of output element r (0..15) of a 32x32 MFMA tile for this lane.
__device__ __forceinline__ int mfma_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// ---------------------------------------------------------------------------
// Epilogue staging: one wave's 32-row block of accumulators as fp32 rows of
// WN values in LDS (row stride WN + 4 floats against bank conflicts).
// ---------------------------------------------------------------------------
template <int TN>
__device__ __forceinline__ void stage_rows(float* region, const f32x16_t (&acc)[TN]) {
  constexpr int WN = TN * 32, LD = WN + 4;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) region[mfma_row(r, lane) * LD + j * 32 + (lane & 31)] = acc[j][r];
}

__device__ __forceinline__ void read8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Eight elements of T kept as loaded (bf16: one 16-byte vector), so that a
// load can be issued well before its values are used.
template <typename T>
struct Raw8 {
  uint4 q[sizeof(T) / 2];
};

template <typename T>
__device__ __forceinline__ Raw8<T> raw_load8(const void* base, int64_t idx) {
  Raw8<T> r;
  const uint4* src = reinterpret_cast<const uint4*>(static_cast<const T*>(base) + idx);
#pragma unroll
  for (int i = 0; i < static_cast<int>(sizeof(T) / 2); ++i) r.q[i] = src[i];
  return r;
}

template <typename T>
__device__ __forceinline__ void raw_unpack8(const Raw8<T>& r, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t w[4] = {r.q[0].x, r.q[0].y, r.q[0].z, r.q[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const uint32_t w[8] = {r.q[0].x, r.q[0].y, r.q[0].z, r.q[0].w, r.q[1].x, r.q[1].y, r.q[1].z, r.q[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
  }
}

template <typename T>
__device__ __forceinline__ void load8g(const void* base, int64_t idx, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    read8(static_cast<const float*>(base) + idx, v);
  }
}

template <typename T>
__device__ __forceinline__ void store8g(void* base, int64_t idx, const float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    uint4 q;
    q.x = pack_bf16x2(v[0], v[1]);
    q.y = pack_bf16x2(v[2], v[3]);
    q.z = pack_bf16x2(v[4], v[5]);
    q.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + idx) = q;
  } else {
    float* p = static_cast<float*>(base) + idx;
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// ---------------------------------------------------------------------------
// The kernel: BM x BN tile, WGM x WGN waves, NS LDS stages of RB bytes of k.
// PIPE 0: operands loaded straight into LDS NS - 1 stages ahead, one barrier
// per stage at its start, fragments read one group ahead within the stage.
// PIPE 2 (bf16): operands staged through registers, fragment reads one group
// ahead across stage boundaries and interleaved with the MFMAs (see the loop).
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int WGM, int WGN, bool AK, bool BK, int EPI, typename OutT,
          int RB, int NS, int PIPE = 0>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_kernel(GemmArgs p) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int kBK = RB / sizeof(T);
  static_assert(EPI != kEpiGateUp || WN % 64 == 0, "gate/up pairing needs 64-column wave tiles");
  static_assert((32 * (WN + 4) * 4) * WGM * WGN <= NS * (BM + BN) * RB, "epilogue staging");

  extern __shared__ __attribute__((aligned(16))) char smem[];   // NS stages x (BM + BN) rows
  char* smem_lds = smem;
  char* As0 = smem;
  char* Bs0 = smem + BM * RB;
  constexpr int kStage = (BM + BN) * RB;

  // A device-side M shrinks the tile grid: the first tiles_m x tiles_n
  // workgroups take the live tiles (spread over every XCD by tile_coords),
  // the rest leave at once (the same decision for the whole workgroup).
  if (p.m_dev) {
    const int64_t md = *p.m_dev;
    p.M = md < p.M ? (md > 0 ? md : 0) : p.M;
    if (static_cast<int64_t>(blockIdx.x) >= ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN)) return;
  }
  int64_t mt, nt;
  tile_coords((p.M + BM - 1) / BM, (p.N + BN - 1) / BN, mt, nt);
  if (p.k_dev) {
    const int64_t kd = *p.k_dev;
    p.K = kd < p.K ? (kd > 0 ? kd : 0) : p.K;
  }
  const int64_t m0 = mt * BM;
  const int64_t n0 = nt * BN;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int wm = wid / WGN, wn = wid % WGN;

  // ---- operand addressing ----
  // bf16 MN-major operands load straight into LDS (transposed on the read);
  // fp32 MN-major operands are transposed in registers.
  constexpr bool kMNDirect = sizeof(T) == 2;
  static_assert(kMNDirect || (RB == kRowBytes && NS == 2),
                "fp32 MN-major tiles pass through registers: 128-byte rows, two stages");
  using AMN = typename std::conditional<kMNDirect, MNDirectTile<BM, NT, kBK>, MNMajorTile<T, BM, NT>>::type;
  using BMN = typename std::conditional<kMNDirect, MNDirectTile<BN, NT, kBK>, MNMajorTile<T, BN, NT>>::type;
  using ATile = typename std::conditional<AK, KMajorTile<BM, NT, RB>, AMN>::type;
  using BTile = typename std::conditional<BK, KMajorTile<BN, NT, RB>, BMN>::type;
  ATile at;
  BTile bt;
  if constexpr (AK) {
#pragma unroll
    for (int i = 0; i < ATile::kPer; ++i) {
      int64_t m = m0 + ATile::row_of(i);
      if (m > p.M - 1) m = p.M - 1;
      int64_t row = m;
      if (p.a_rows) {
        row = p.a_rows[m];
        if (row < 0 || row >= p.a_rows_bound) {
          flag_index_error(p.err);
          row = 0;
        }
      }
      at.row_ptr[i] = static_cast<const char*>(p.a0) + row * p.lda * sizeof(T);
    }
    at.init_chunks();
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
    bt.init_chunks();
  }
  if constexpr (!AK && kMNDirect) at.init();
  if constexpr (!BK && kMNDirect) bt.init();
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

  // Gate epilogues: the token and table-row index of every row of the tile
  // are loaded here and kept in LDS past the stage buffers ([BM] tokens,
  // then [BM] row indices; -1 for a token outside the batch), so that the
  // epilogue can issue all of its table-row gathers at once.  They are
  // written to LDS after the first stage's loads are issued, whose wait
  // covers them.
  // DhSeg keeps each row's token and segment (-1 when invalid) the same way.
  constexpr bool kGate = EPI == kEpiGateUp || EPI == kEpiGateStem;
  constexpr bool kSeg = EPI == kEpiDhSeg;
  static_assert(!kSeg || WN == 64, "the segment pass gives each lane one column");
  int* idx_lds = reinterpret_cast<int*>(smem + NS * kStage);
  constexpr int kIdxPer = (BM + NT - 1) / NT;
  int pro_tok[kGate || kSeg ? kIdxPer : 1], pro_ri[kGate || kSeg ? kIdxPer : 1];
  // DhSeg: the batch's unique count; past the row buffer nothing is written
  const int64_t seg_nu = kSeg ? static_cast<int64_t>(*p.seg_nu) : 0;
  const bool seg_ok = !kSeg || (seg_nu >= 0 && seg_nu <= p.seg_max_unique);
  if constexpr (kGate || kSeg) {
#pragma unroll
    for (int j = 0; j < kIdxPer; ++j) {
      const int t = static_cast<int>(threadIdx.x) + j * NT;
      int64_t m = m0 + t;
      if (m > p.M - 1) m = p.M - 1;
      int64_t tok = p.a_rows ? static_cast<int64_t>(p.a_rows[m]) : m;
      if (tok < 0 || tok >= p.a_rows_bound) tok = -1;   // flagged with the A operand's rows
      pro_tok[j] = static_cast<int>(tok);
      if constexpr (kGate) {
        pro_ri[j] = tok < 0 ? -1 : p.row_index[tok];
      } else {
        int64_t sg = tok < 0 ? -1 : p.seg_inv[tok];
        if (sg < 0 || sg >= seg_nu) {
          if (tok >= 0 && seg_ok) flag_index_error(p.err);
          sg = -1;
        }
        pro_ri[j] = static_cast<int>(sg);
      }
    }
  }
  auto stash_idx = [&]() {
    if constexpr (kGate || kSeg) {
#pragma unroll
      for (int j = 0; j < kIdxPer; ++j) {
        const int t = static_cast<int>(threadIdx.x) + j * NT;
        if (t < BM) {
          idx_lds[t] = pro_tok[j];
          idx_lds[BM + t] = pro_ri[j];
        }
      }
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Operands go straight from global memory into the LDS buffer of a later
  // stage (NS - 1 stages ahead), except fp32 MN-major ones, which pass through
  // registers (for the transpose) and are written after the current stage's
  // MFMAs (NS = 2).
  lds_char* lds = (lds_char*)(smem_lds);   // address-space cast of the dynamic LDS block
  auto a_base16 = [&](int64_t k) { return reinterpret_cast<const uint16_t*>(a_base(k)); };
  auto b_base16 = [&](int64_t k) { return reinterpret_cast<const uint16_t*>(b_base(k)); };
  auto issue_loads = [&](int64_t kt, int buf) {
    const int64_t k0 = kt * kBK;
    lds_char* la = lds + buf * kStage;
    lds_char* lb = la + BM * RB;
    if constexpr (AK) at.load(k0 * static_cast<int64_t>(sizeof(T)), la);
    else if constexpr (kMNDirect) at.load(k0, a_base16, a_cols, la);
    else at.template load<0>(k0, a_base, a_cols);
    if constexpr (BK) bt.load(k0 * static_cast<int64_t>(sizeof(T)), lb);
    else if constexpr (kMNDirect) bt.load(k0, b_base16, b_cols, lb);
    else bt.template load<0>(k0, b_base, b_cols);
  };
  auto store_regs = [&](int buf) {
    if constexpr (!AK && !kMNDirect) at.template store<0>(As0 + buf * kStage);
    if constexpr (!BK && !kMNDirect) bt.template store<0>(Bs0 + buf * kStage);
  };
  using MmaT = Mma<T, TM, TN, AK, BK, BM, BN, RB>;
  auto compute = [&](int buf) {
    const lds_char* As = lds + buf * kStage;
    const lds_char* Bs = As + BM * RB;
    MmaT::stage(As, Bs, wm * WM, wn * WN, acc);
  };

  // Pipeline: stage kt is computed while stages kt+1 .. kt+NS-1 are in
  // flight.  Every stage issues the same number of load instructions per
  // thread (kLoads), so "stage kt has landed" is a vmcnt of kLoads times the
  // number of younger stages; the barrier after it also tells every wave that
  // the buffer about to be refilled has been read by all.
  constexpr int kLoads = (AK || kMNDirect ? ATile::kPer : 0) + (BK || kMNDirect ? BTile::kPer : 0);
  const int64_t nk = (p.K + kBK - 1) / kBK;
  if constexpr (PIPE == 2) {
    // Register-staged pipeline, two LDS stages of 64 k (four groups).  In
    // stage s: groups 0-2 read the next group's fragments during their
    // MFMAs; group 2 also writes stage s + 1 (in registers since stage s - 1)
    // into the other LDS buffer, one 16-byte piece per MFMA; barrier B_{s+1}
    // (this wave's LDS writes and reads done, then s_barrier) publishes it;
    // group 3 reads stage s + 1's first group and issues the global loads of
    // stage s + 2 into the registers.  The other buffer held stage s - 1,
    // whose last reads came before B_s.  Past the end of K the writes go to
    // the idle buffer and the loads re-read the last stage, so every stage
    // runs the same instruction sequence.
    static_assert(kMNDirect && RB == 128 && NS == 2 && ATile::kPer + BTile::kPer <= TM * TN,
                  "register-staged pipeline");
    constexpr int NA = ATile::kPer, NP = ATile::kPer + BTile::kPer;
    using Fr = typename MmaT::Frags;
    Fr fr[2];
    const int a_row0 = wm * WM, b_row0 = wn * WN;
    auto load_regs = [&](int64_t kt) {
      const int64_t k0 = kt * kBK;
      if constexpr (AK) at.load_regs(k0 * static_cast<int64_t>(sizeof(T)));
      else at.load_regs(k0, a_base16, a_cols);
      if constexpr (BK) bt.load_regs(k0 * static_cast<int64_t>(sizeof(T)));
      else bt.load_regs(k0, b_base16, b_cols);
    };
    auto store_piece = [&](int buf, int q) {
      lds_char* la = lds + buf * kStage;
      if (q < NA) at.store_piece(la, q);
      else bt.store_piece(la + BM * RB, q - NA);
    };
    if (nk > 0) {
      load_regs(0);
      stash_idx();
#pragma unroll
      for (int q = 0; q < NP; ++q) store_piece(0, q);
      load_regs(nk > 1 ? 1 : 0);
      lds_barrier();                                        // B_0
      MmaT::read(lds, lds + BM * RB, a_row0, b_row0, 0, fr[0]);
    } else {
      stash_idx();
    }
    for (int64_t st = 0; st < nk; ++st) {
      const int cur = static_cast<int>(st & 1);
      const lds_char* As = lds + cur * kStage;
      const lds_char* Bs = As + BM * RB;
      MmaT::mma_interleaved(fr[0], acc, [&](int q) { MmaT::read_piece(As, Bs, a_row0, b_row0, 1, q, fr[1]); });
      MmaT::mma_interleaved(fr[1], acc, [&](int q) { MmaT::read_piece(As, Bs, a_row0, b_row0, 2, q, fr[0]); });
      MmaT::mma_each(fr[0], acc, [&](int m) {
        if (m < TM + TN) MmaT::read_piece(As, Bs, a_row0, b_row0, 3, m, fr[1]);
        if (m < NP) store_piece(cur ^ 1, m);
      });
      lds_barrier();                                        // B_{st+1}
      const bool more = st + 1 < nk;
      const lds_char* An = more ? lds + (cur ^ 1) * kStage : As;
      const lds_char* Bn = An + BM * RB;
      const int64_t next = st + 2 < nk ? st + 2 : nk - 1;
      MmaT::mma_each(fr[1], acc, [&](int m) {
        if (m < TM + TN) MmaT::read_piece(An, Bn, a_row0, b_row0, 0, m, fr[0]);
        if (m == TM + TN) load_regs(next);
      });
    }
  } else {
#pragma unroll
  for (int st = 0; st < NS - 1; ++st) {
    if (st < nk) {
      issue_loads(st, st);
      store_regs(st);
    }
  }
  stash_idx();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int64_t younger = (nk - 1 - kt) < (NS - 2) ? (nk - 1 - kt) : (NS - 2);
    static_assert(NS >= 2 && NS <= 5 && (NS - 2) * kLoads < 64, "stages");
    if (younger >= 3) wait_vmcnt<(NS >= 5 ? 3 * kLoads : 0)>();
    else if (younger == 2) wait_vmcnt<(NS >= 4 ? 2 * kLoads : 0)>();
    else if (younger == 1) wait_vmcnt<(NS >= 3 ? kLoads : 0)>();
    else wait_vmcnt<0>();
    if constexpr (kMNDirect) lds_barrier();
    else __syncthreads();   // register-staged tiles were written with ds_write
    if (kt + NS - 1 < nk) issue_loads(kt + NS - 1, static_cast<int>((kt + NS - 1) % NS));
    compute(static_cast<int>(kt % NS));
    if (kt + NS - 1 < nk) store_regs(static_cast<int>((kt + NS - 1) % NS));
  }
  }
  __syncthreads();   // the epilogue reuses the stage buffers

  // ---- epilogue: per 32-row block, stage through this wave's LDS region ----
  constexpr int LD = WN + 4;
  float* region = reinterpret_cast<float*>(smem) + wid * 32 * LD;
  constexpr int kChunks = 32 * WN / 8;          // 8-column chunks per 32-row block
  // Gate epilogues: chunk q = lane + 64 c of block i is row q / kCpr of the
  // block and 8 features from (q % kCpr) 8 of the wave's features (gate/up:
  // wave columns are pairs of [32 gate | 32 up] for the same 32 features).
  // Every block's table rows are fetched before the first block is formed:
  // one gather latency per tile instead of two dependent ones per block.
  constexpr int kCpr = EPI == kEpiGateUp ? WN / 16 : WN / 8;
  constexpr int kGateChunks = 32 * kCpr;
  constexpr int kGatePer = (kGateChunks + 63) / 64;
  const int64_t wave_feat0 = EPI == kEpiGateUp ? (n0 + wn * WN) / 2 : n0 + wn * WN;
  Raw8<T> epre[kGate ? TM : 1][kGate ? kGatePer : 1];
  if constexpr (kGate) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int c = 0; c < kGatePer; ++c) {
        const int q = lane + 64 * c;
        const int row = wm * WM + i * 32 + q / kCpr;
        const int64_t feat = wave_feat0 + (q % kCpr) * 8;
        const int64_t ri = idx_lds[BM + row];
        const bool ok = q < kGateChunks && ri >= 0 && ri < p.n_rows && feat < p.d_ff;
        epre[i][c] = raw_load8<T>(p.rows, ok ? ri * p.d_ff + feat : 0);
      }
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    stage_rows<TN>(region, acc[i]);
    __syncthreads();
    const int64_t mrow0 = m0 + wm * WM + i * 32;
    if constexpr (EPI == kEpiStore) {
#pragma unroll
      for (int q = lane; q < kChunks; q += 64) {
        const int rr = q / (WN / 8), cc = (q % (WN / 8)) * 8;
        const int64_t m = mrow0 + rr;
        const int64_t n = n0 + wn * WN + cc;
        if (m < p.M && n < p.N) {
          float v[8];
          read8(region + rr * LD + cc, v);
          void* cb = m < p.c_split ? p.c0 : p.c1;
          const int64_t mm = m < p.c_split ? m : m - p.c_split;
          store8g<OutT>(cb, mm * p.ldc + n, v);
        }
      }
    } else if constexpr (EPI == kEpiStoreT) {
      // lane q % WN owns column n, 8 rows from (q / WN) 8 per store
#pragma unroll
      for (int q = lane; q < WN * 4; q += 64) {
        const int cc = q % WN, rg = (q / WN) * 8;
        const int64_t m = mrow0 + rg;
        const int64_t n = n0 + wn * WN + cc;
        if (m < p.M && n < p.N) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = region[(rg + e) * LD + cc];
          void* cb = n < p.c_split ? p.c0 : p.c1;
          const int64_t nn = n < p.c_split ? n : n - p.c_split;
          store8g<OutT>(cb, nn * p.ldc + m, v);
        }
      }
    } else if constexpr (EPI == kEpiGateUp) {
      // h, g, u from the staged [gate | up] pairs and the prefetched rows
      const int64_t f = p.d_ff;
#pragma unroll
      for (int c = 0; c < kGatePer; ++c) {
        const int q = lane + 64 * c;
        if (q >= kGateChunks) continue;
        const int rr = q / kCpr;
        const int fc = (q % kCpr) * 8;
        const int pair = fc / 32, fin = fc % 32;
        const int row = wm * WM + i * 32 + rr;
        const int64_t m = mrow0 + rr;
        const int64_t feat = wave_feat0 + fc;
        const int64_t tok = idx_lds[row], ri = idx_lds[BM + row];
        if (m < p.M && feat < f && tok >= 0) {
          float g[8], a[8], e[8];
          read8(region + rr * LD + pair * 64 + fin, g);
          read8(region + rr * LD + pair * 64 + 32 + fin, a);
          raw_unpack8<T>(epre[i][c], e);
          if (!(ri >= 0 && ri < p.n_rows)) {
            flag_index_error(p.err);
#pragma unroll
            for (int k = 0; k < 8; ++k) e[k] = 0.0f;
          }
          float u[8], h[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            u[k] = a[k] + e[k];
            h[k] = g[k] * sigmoidf_(g[k]) * u[k];
          }
          const int64_t o = tok * f + feat;
          store8g<T>(p.h_out, o, h);
          if (p.g_out) store8g<T>(p.g_out, o, g);
          if (p.u_out) store8g<T>(p.u_out, o, u);
        }
      }
    } else if constexpr (EPI == kEpiGateStem) {
      // C = g (M = tokens, N = d_ff); u is the table row
      const int64_t f = p.d_ff;
#pragma unroll
      for (int c = 0; c < kGatePer; ++c) {
        const int q = lane + 64 * c;
        if (q >= kGateChunks) continue;
        const int rr = q / kCpr, cc = (q % kCpr) * 8;
        const int row = wm * WM + i * 32 + rr;
        const int64_t m = mrow0 + rr;
        const int64_t n = wave_feat0 + cc;
        const int64_t tok = idx_lds[row], ri = idx_lds[BM + row];
        if (m < p.M && n < f && tok >= 0) {
          float g[8], h[8], e[8];
          read8(region + rr * LD + cc, g);
          raw_unpack8<T>(epre[i][c], e);
          if (!(ri >= 0 && ri < p.n_rows)) {
            flag_index_error(p.err);
#pragma unroll
            for (int k = 0; k < 8; ++k) e[k] = 0.0f;
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) h[k] = g[k] * sigmoidf_(g[k]) * e[k];
          const int64_t o = tok * f + n;
          store8g<T>(p.h_out, o, h);
          if (p.g_out) store8g<T>(p.g_out, o, g);
          if (p.u_out) store8g<T>(p.u_out, o, e);
        }
      }
    } else if constexpr (EPI == kEpiDhSeg) {
      // rows are sorted positions; g, u and [dg | du] live at the row's token
      const int64_t f = p.N;
      constexpr int kPerLane = (kChunks + 63) / 64;
      float gv[kPerLane][8], uv[kPerLane][8];
#pragma unroll
      for (int c = 0; c < kPerLane; ++c) {
        const int q = lane + 64 * c;
        const int rr = q / (WN / 8), cc = (q % (WN / 8)) * 8;
        const int64_t m = mrow0 + rr;
        const int64_t n = n0 + wn * WN + cc;
        const int64_t tok = idx_lds[wm * WM + i * 32 + rr];
        const bool ok = q < kChunks && m < p.M && n < f && tok >= 0;
        load8g<T>(p.g_in, ok ? tok * f + n : 0, gv[c]);
        load8g<T>(p.u_in, ok ? tok * f + n : 0, uv[c]);
      }
#pragma unroll
      for (int c = 0; c < kPerLane; ++c) {
        const int q = lane + 64 * c;
        const int rr = q / (WN / 8), cc = (q % (WN / 8)) * 8;
        const int64_t m = mrow0 + rr;
        const int64_t n = n0 + wn * WN + cc;
        const int64_t tok = idx_lds[wm * WM + i * 32 + rr];
        if (q < kChunks && m < p.M) {
          float du[8];
          if (n < f && tok >= 0) {
            float dh[8], dg[8];
            read8(region + rr * LD + cc, dh);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const float s = sigmoidf_(gv[c][k]);
              du[k] = dh[k] * gv[c][k] * s;
              dg[k] = dh[k] * uv[c][k] * s * (1.0f + gv[c][k] * (1.0f - s));
            }
            store8g<T>(p.dgu_out, tok * 2 * f + n, dg);
            store8g<T>(p.dgu_out, tok * 2 * f + f + n, du);
          } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) du[k] = 0.0f;   // a flagged row adds nothing
          }
          // the fp32 du stays in this wave's staging rows for the segment pass
          *reinterpret_cast<float4*>(region + rr * LD + cc) = make_float4(du[0], du[1], du[2], du[3]);
          *reinterpret_cast<float4*>(region + rr * LD + cc + 4) = make_float4(du[4], du[5], du[6], du[7]);
        }
      }
      __syncthreads();
      // lane l walks column l of the block's 32 positions in order; a run of
      // one segment ends at a change of segment or at the block's end.  A
      // run that starts the block belongs to a segment begun in an earlier
      // chunk when position p0 - 1 has the same segment; one that ends the
      // block continues past it when position p1 has the same segment
      // (segments are contiguous in sorted order): so no segment offset is
      // loaded inside the walk.
      static_assert(kSegChunk == 32, "one chunk of the segment sum per 32-row block");
      const int64_t p0 = mrow0;
      const int64_t p1 = p0 + kSegChunk < p.M ? p0 + kSegChunk : p.M;
      if (seg_ok && p0 < p.M) {
        const int64_t chunk = p0 / kSegChunk;
        const int row0 = wm * WM + i * 32;
        const int len = static_cast<int>(p1 - p0);
        // segments of the positions just before and after the block (-2: none)
        auto seg_at = [&](int64_t pos) -> int {
          if (pos < 0 || pos >= p.M) return -2;
          if (pos >= m0 && pos < m0 + BM) return idx_lds[BM + (pos - m0)];
          const int64_t t = p.a_rows[pos];
          if (t < 0 || t >= p.a_rows_bound) return -1;
          const int64_t sg = p.seg_inv[t];
          return sg >= 0 && sg < seg_nu ? static_cast<int>(sg) : -1;
        };
        const int prev_sg = seg_at(p0 - 1), next_sg = seg_at(p1);
        // lane r: the segment of row r, and whether row r ends a run
        const int my_sg = lane < len ? idx_lds[BM + row0 + lane] : -3;
        const int nx_sg = lane + 1 < len ? idx_lds[BM + row0 + lane + 1] : -4;
        const uint64_t ends = __ballot(lane < len && (lane == len - 1 || nx_sg != my_sg));
        const int64_t col = n0 + wn * WN + lane;
        float a = 0.0f;
        int run0 = 0;
#pragma unroll
        for (int r = 0; r < kSegChunk; ++r) {
          if (r < len) {
            a += region[r * LD + lane];
            if ((ends >> r) & 1ull) {
              const int sg = __builtin_amdgcn_readlane(my_sg, r);
              if (sg >= 0 && col < f) {
                const bool before = run0 == 0 && prev_sg == sg;
                const bool after = r == len - 1 && next_sg == sg;
                float* dst = before ? p.seg_first + chunk * f + col         // began in an earlier chunk
                             : after ? p.seg_last + chunk * f + col          // continues past p1
                                     : p.seg_rows + sg * f + col;           // whole segment here
                *dst = a;
              }
              a = 0.0f;
              run0 = r + 1;
            }
          }
        }
      }
      if (!seg_ok && blockIdx.x == 0 && threadIdx.x == 0 && i == 0) flag_index_error(p.err);
    } else {  // kEpiDhAct: C = dh (M = tokens, N = d_ff)
      // g and u of all of this lane's chunks are loaded first, then dg, du
      // are formed and stored
      const int64_t f = p.N;
      constexpr int kPerLane = (kChunks + 63) / 64;
      float gv[kPerLane][8], uv[kPerLane][8];
#pragma unroll
      for (int c = 0; c < kPerLane; ++c) {
        const int q = lane + 64 * c;
        const int rr = q / (WN / 8), cc = (q % (WN / 8)) * 8;
        const int64_t m = mrow0 + rr;
        const int64_t n = n0 + wn * WN + cc;
        const bool ok = q < kChunks && m < p.M && n < f;
        load8g<T>(p.g_in, ok ? m * f + n : 0, gv[c]);
        load8g<T>(p.u_in, ok ? m * f + n : 0, uv[c]);
      }
#pragma unroll
      for (int c = 0; c < kPerLane; ++c) {
        const int q = lane + 64 * c;
        const int rr = q / (WN / 8), cc = (q % (WN / 8)) * 8;
        const int64_t m = mrow0 + rr;
        const int64_t n = n0 + wn * WN + cc;
        if (q < kChunks && m < p.M && n < f) {
          float dh[8], dg[8], du[8];
          read8(region + rr * LD + cc, dh);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float s = sigmoidf_(gv[c][k]);
            du[k] = dh[k] * gv[c][k] * s;
            dg[k] = dh[k] * uv[c][k] * s * (1.0f + gv[c][k] * (1.0f - s));
          }
          store8g<T>(p.dgu_out, m * 2 * f + n, dg);
          store8g<T>(p.dgu_out, m * 2 * f + f + n, du);
          if (p.du32_out) store8g<float>(p.du32_out, m * f + n, du);
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int WGM, int WGN, bool AK, bool BK, int EPI, typename OutT,
          int RB, int NS, int PIPE = 0>
static hipError_t run_tile(const GemmArgs& a, hipStream_t s) {
  constexpr bool kIdx = EPI == kEpiGateUp || EPI == kEpiGateStem || EPI == kEpiDhSeg;
  constexpr size_t kSmem = static_cast<size_t>(NS) * (BM + BN) * RB + (kIdx ? 2 * BM * sizeof(int) : 0);
  auto kern = &gemm_kernel<T, BM, BN, WGM, WGN, AK, BK, EPI, OutT, RB, NS, PIPE>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
      static_cast<int>(kSmem));
  if (attr != hipSuccess) return attr;
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  kern<<<dim3(static_cast<unsigned>(tiles)), dim3(64 * WGM * WGN), kSmem, s>>>(a);
  return hipGetLastError();
}

// 256x256 tiles for large bf16 problems, 256x128 tiles for plain GEMMs that
// 256x256 tiles would leave half the GPU idle on, 128x128 tiles on 4 waves
// otherwise.
template <typename T, bool AK, bool BK, int EPI, typename OutT>
static hipError_t run(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if constexpr (sizeof(T) == 2) {
    // Register-staged 8-wave pipeline: 1-3 points of MFMA peak above the
    // direct-to-LDS one on five of the six training GEMMs (level on dx).
    // Measured slower: 2x2 waves of 128x128 (half the LDS reads per MFMA)
    // with either pipeline, three to five 32 KB stages (loads three or four
    // stages ahead: the kernels are not waiting on global-load latency), and
    // (on the training shapes) 256x128 or 128x256 tiles on 4 waves with two
    // workgroups per CU.
    const int64_t tiles256 = ((a.M + 255) / 256) * ((a.N + 255) / 256);
    // Plain stores of two K-major operands with 256 x 256 tiles for at most
    // half the compute units: 256 x 128 tiles on 4 x 2 waves of 64 x 64
    // (direct-to-LDS pipeline) when they fill more than half and at most all
    // of them, one round.  Measured for N = 2048, K = 8192: M 2560-4096
    // 134-149 us against 139-158 us on 128 x 128 tiles and (M 4096) 192 us
    // on 256 x 256 ones; from M 4608 (a second round of 256 x 128 tiles) the
    // 256 x 256 tiles are faster again, 190 against 248 us.
    if constexpr (EPI == kEpiStore && AK && BK) {
      const int64_t cus = device_cus();
      const int64_t tiles_rect = ((a.M + 255) / 256) * ((a.N + 127) / 128);
      if (a.M >= 256 && 2 * tiles256 <= cus && 2 * tiles_rect > cus && tiles_rect <= cus)
        return run_tile<T, 256, 128, 4, 2, AK, BK, EPI, OutT, kRowBytes, 2>(a, s);
    }
    if (a.M >= 256 && a.N >= 256 && tiles256 >= 128)
      return run_tile<T, 256, 256, 2, 4, AK, BK, EPI, OutT, kRowBytes, 2, 2>(a, s);
  }
  return run_tile<T, 128, 128, 2, 2, AK, BK, EPI, OutT, kRowBytes, 2>(a, s);
}

template <typename T>
static GemmArgs blank() {
  GemmArgs a{};
  a.a_split = a.b_split = a.c_split = INT64_MAX;
  return a;
}

// h = silu(x W_gate^T) * (x W_up^T + rows[row_index]); optional saves of g, u.
// With wu null (the STEM layer) u = rows[row_index] and the GEMM is W_gate's
// alone.  With `pos`, only the n_sel tokens pos[0 .. n_sel) of the n_tokens
// are computed (their rows of x, h, g, u; row_index stays indexed by token).
template <typename T>
hipError_t gateup_fwd(int64_t n_sel, const int32_t* pos, int64_t n_tokens, int64_t d, int64_t f,
                      const void* x, const void* wg, const void* wu, const void* rows,
                      int64_t n_rows, const int32_t* row_index, void* h, void* g_out, void* u_out,
                      hipStream_t s, int* err) {
  GemmArgs a = blank<T>();
  a.M = n_sel; a.N = 2 * f; a.K = d;
  a.a0 = x; a.lda = d;
  a.a_rows = pos; a.a_rows_bound = n_tokens;
  a.b0 = wg; a.b1 = wu; a.ldb = d;
  a.rows = rows; a.row_index = row_index; a.n_rows = n_rows; a.d_ff = f;
  a.h_out = h; a.g_out = g_out; a.u_out = u_out; a.err = err;
  if (!wu) {
    a.N = f;
    return run<T, true, true, kEpiGateStem, T>(a, s);
  }
  return run<T, true, true, kEpiGateUp, T>(a, s);
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
  if (out_dtype == STAPLE_F32) return run<T, true, true, kEpiStore, float>(a, s);
  return run<T, true, true, kEpiStore, bf16_t>(a, s);
}

// dh = dy W_down; dgu[:, :f] = dg, dgu[:, f:] = du; du32 (nullable) = du in fp32
template <typename T>
hipError_t dh_act(int64_t n, int64_t d, int64_t f, const void* dy, const void* wd, const void* g,
                  const void* u, void* dgu, float* du32, hipStream_t s) {
  GemmArgs a = blank<T>();
  a.M = n; a.N = f; a.K = d;
  a.a0 = dy; a.lda = d;
  a.b0 = wd; a.ldb = f;          // B(k=j, n) = W_down[j, n]
  a.g_in = g; a.u_in = u; a.dgu_out = dgu; a.du32_out = du32;
  return run<T, true, false, kEpiDhAct, T>(a, s);
}

// dx = dg W_gate + du W_up  (K = 2f over the concatenated [dg | du]); with wu
// null (STEM) dx = dg W_gate (K = f, the dg half of each row)
template <typename T>
hipError_t dx_bwd(int64_t n, int64_t d, int64_t f, const void* dgu, const void* wg,
                  const void* wu, void* dx, int out_dtype, hipStream_t s) {
  GemmArgs a = blank<T>();
  a.M = n; a.N = d; a.K = wu ? 2 * f : f;
  a.a0 = dgu; a.lda = 2 * f;
  a.b0 = wg; a.b1 = wu; a.ldb = d; a.b_split = f;
  a.c0 = dx; a.ldc = d;
  if (out_dtype == STAPLE_F32) return run<T, true, false, kEpiStore, float>(a, s);
  return run<T, true, false, kEpiStore, bf16_t>(a, s);
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
  return run<T, false, false, kEpiStore, float>(a, s);
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
  return run<T, false, false, kEpiStore, float>(a, s);
}

// ---------------------------------------------------------------------------
// K-major copies for the backward (bf16).  The GEMM reads a K-major operand
// with one 16-byte LDS read per fragment and an MN-major one with two
// transposing reads; at the 1B training shapes the K-major form of dx, dh and
// dW_down is 7-20% faster than the MN-major one, for a copy that costs a few
// percent of that GEMM.
// ---------------------------------------------------------------------------
// dst[c * ld_dst + r] = src[r * ld_src + c] for r < rows, c < cols, through a
// 64 x 64 tile in LDS (16-byte loads along src rows, 16-byte stores along dst
// rows); dst entries r in [rows, dst_cols) are zeros, so a K-major operand
// can be padded to whole 64-element k stages.  cols, dst_cols, ld_src and
// ld_dst are multiples of 8.
constexpr int kTrTile = 64;
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ src,
                                                             int64_t rows, int64_t cols,
                                                             int64_t ld_src,
                                                             uint16_t* __restrict__ dst,
                                                             int64_t dst_cols, int64_t ld_dst) {
  __shared__ uint16_t t[kTrTile][kTrTile + 2];
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kTrTile;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * kTrTile;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rr = static_cast<int>(threadIdx.x) / 8 + 32 * i, vc = (threadIdx.x % 8) * 8;
    const int64_t r = r0 + rr, c = c0 + vc;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < rows && c < cols) v = *reinterpret_cast<const uint4*>(src + r * ld_src + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      t[rr][vc + 2 * j] = static_cast<uint16_t>(w[j] & 0xffffu);
      t[rr][vc + 2 * j + 1] = static_cast<uint16_t>(w[j] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int cc = static_cast<int>(threadIdx.x) / 8 + 32 * i, vr = (threadIdx.x % 8) * 8;
    const int64_t c = c0 + cc, r = r0 + vr;
    if (c >= cols || r >= dst_cols) continue;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = static_cast<uint32_t>(t[vr + 2 * j][cc]) | (static_cast<uint32_t>(t[vr + 2 * j + 1][cc]) << 16);
    *reinterpret_cast<uint4*>(dst + c * ld_dst + r) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

hipError_t transpose_bf16(const void* src, int64_t rows, int64_t cols, int64_t ld_src, void* dst,
                          int64_t dst_cols, int64_t ld_dst, hipStream_t s) {
  if (rows <= 0 || cols <= 0 || dst_cols <= 0) return hipSuccess;
  if (cols % 8 || dst_cols % 8 || ld_src % 8 || ld_dst % 8 || dst_cols < rows || ld_dst < dst_cols)
    return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>((cols + kTrTile - 1) / kTrTile),
                  static_cast<unsigned>((dst_cols + kTrTile - 1) / kTrTile));
  transpose_bf16_kernel<<<grid, dim3(256), 0, s>>>(static_cast<const uint16_t*>(src), rows, cols,
                                                   ld_src, static_cast<uint16_t*>(dst), dst_cols,
                                                   ld_dst);
  return hipGetLastError();
}

// dh with B = W_down^T [f x d] K-major (wd_t: B(k, n) = wd_t[n d + k])
hipError_t dh_act_kt(int64_t n, int64_t d, int64_t f, const void* dy, const void* wd_t,
                     const void* g, const void* u, void* dgu, float* du32, hipStream_t s) {
  GemmArgs a = blank<bf16_t>();
  a.M = n; a.N = f; a.K = d;
  a.a0 = dy; a.lda = d;
  a.b0 = wd_t; a.ldb = d;
  a.g_in = g; a.u_in = u; a.dgu_out = dgu; a.du32_out = du32;
  return run<bf16_t, true, true, kEpiDhAct, bf16_t>(a, s);
}

// dh over the tokens in sorted order with B = W_down^T K-major, [dg | du] at
// each token's row, and the table-row gradient's chunk pass in the epilogue:
// d_rows for segments inside a 32-position chunk, first / last partials for
// the others (completed by the segment sum's fixup pass)
hipError_t dh_seg_kt(int64_t n, int64_t d, int64_t f, const void* dy, const void* wd_t,
                     const void* g, const void* u, void* dgu, const int32_t* sorted_pos,
                     const int32_t* inv, const int32_t* seg_start, const int32_t* n_unique,
                     int64_t max_unique, float* d_rows, float* first, float* last, hipStream_t s,
                     int* err) {
  GemmArgs a = blank<bf16_t>();
  a.M = n; a.N = f; a.K = d;
  a.a0 = dy; a.lda = d;
  a.a_rows = sorted_pos; a.a_rows_bound = n;
  a.b0 = wd_t; a.ldb = d;
  a.g_in = g; a.u_in = u; a.dgu_out = dgu;
  a.seg_inv = inv; a.seg_start = seg_start; a.seg_nu = n_unique; a.seg_max_unique = max_unique;
  a.seg_rows = d_rows; a.seg_first = first; a.seg_last = last;
  a.err = err;
  return run<bf16_t, true, true, kEpiDhSeg, bf16_t>(a, s);
}

// dx with B = [W_gate^T | W_up^T] [d x k] K-major (k = 2f, or f for the STEM layer)
hipError_t dx_bwd_kt(int64_t n, int64_t d, int64_t k, const void* dgu, int64_t ld_dgu,
                     const void* w_t, void* dx, int out_dtype, hipStream_t s) {
  GemmArgs a = blank<bf16_t>();
  a.M = n; a.N = d; a.K = k;
  a.a0 = dgu; a.lda = ld_dgu;
  a.b0 = w_t; a.ldb = k;
  a.c0 = dx; a.ldc = d;
  if (out_dtype == STAPLE_F32) return run<bf16_t, true, true, kEpiStore, float>(a, s);
  return run<bf16_t, true, true, kEpiStore, bf16_t>(a, s);
}

// [dW_gate; dW_up] with A = x^T [d x ld_t] K-major (zero past the n tokens):
// C = x^T [dg | du] is [dW_gate; dW_up]^T, stored transposed (M = d, N = 2f,
// or f when the up-projection is frozen)
hipError_t dwgu_bwd_kt(int64_t n, int64_t d, int64_t f, const void* x_t, int64_t ld_t,
                       const void* dgu, float* dwg, float* dwu, bool freeze_up, hipStream_t s) {
  GemmArgs a = blank<bf16_t>();
  a.M = d; a.N = freeze_up ? f : 2 * f; a.K = n;
  a.a0 = x_t; a.lda = ld_t;
  a.b0 = dgu; a.ldb = 2 * f;
  a.c0 = dwg; a.c1 = dwu; a.ldc = d; a.c_split = f;
  return run<bf16_t, true, false, kEpiStoreT, float>(a, s);
}

// dW_down with A = dy^T [d x ld_t] K-major (zero past the n tokens)
hipError_t dwdown_bwd_kt(int64_t n, int64_t d, int64_t f, const void* dy_t, int64_t ld_t,
                         const void* h, float* dwd, hipStream_t s) {
  GemmArgs a = blank<bf16_t>();
  a.M = d; a.N = f; a.K = n;
  a.a0 = dy_t; a.lda = ld_t;
  a.b0 = h; a.ldb = f;
  a.c0 = dwd; a.ldc = f;
  return run<bf16_t, true, false, kEpiStore, float>(a, s);
}

// h = silu(g) * u from the saved g and u, for a backward whose caller kept no
// h: n * f elements (a multiple of 8), 16-byte vectors, grid-stride.
template <typename T>
__global__ __launch_bounds__(256) void recompute_h_kernel(const void* __restrict__ g,
                                                          const void* __restrict__ u,
                                                          void* __restrict__ h, int64_t n8) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n8;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    float gv[8], uv[8], hv[8];
    load8g<T>(g, i * 8, gv);
    load8g<T>(u, i * 8, uv);
#pragma unroll
    for (int k = 0; k < 8; ++k) hv[k] = gv[k] * sigmoidf_(gv[k]) * uv[k];
    store8g<T>(h, i * 8, hv);
  }
}

template <typename T>
hipError_t recompute_h(int64_t n, int64_t f, const void* g, const void* u, void* h, hipStream_t s) {
  const int64_t n8 = n * f / 8;
  if (n8 <= 0) return hipSuccess;
  const int64_t blocks = (n8 + 255) / 256;
  recompute_h_kernel<T><<<dim3(static_cast<unsigned>(blocks < 8192 ? blocks : 8192)), dim3(256), 0, s>>>(
      g, u, h, n8);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Low-rank table: Z = R_r P^T for the first *n of max_rows compact rows, and
// the gradients dE_r = dZ P, dP = dZ^T R_r from dZ (the layer's fp32
// table-row gradient, rounded to T as the operand of both contractions).
// ---------------------------------------------------------------------------
template <typename T>
hipError_t lowrank_expand(int64_t max_rows, const int32_t* n_dev, int64_t r, int64_t f,
                          const void* rows_r, const void* proj, void* z, hipStream_t s) {
  GemmArgs a = blank<T>();
  a.M = max_rows; a.N = f; a.K = r;
  a.a0 = rows_r; a.lda = r;        // A(u, k) = R_r[u, k]
  a.b0 = proj; a.ldb = r;          // B(k, j) = P[j, k] (K-major rows of P)
  a.c0 = z; a.ldc = f;
  a.m_dev = n_dev;
  return run<T, true, true, kEpiStore, T>(a, s);
}

template <typename T>
__global__ __launch_bounds__(256) void round_rows_kernel(const float* __restrict__ src,
                                                         void* __restrict__ dst, int64_t max_rows,
                                                         const int32_t* __restrict__ n_dev,
                                                         int64_t cols) {
  const int64_t nd = *n_dev;
  const int64_t n8 = (nd < max_rows ? (nd > 0 ? nd : 0) : max_rows) * cols / 8;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n8;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    float v[8];
    read8(src + i * 8, v);
    store8g<T>(dst, i * 8, v);
  }
}

// dZ (fp32 [max_rows x f]) -> dE_r [max_rows x r] fp32, dP [f x r] fp32;
// bf16: dZ rounded into ws ([max_rows x f] bf16) first.
template <typename T>
hipError_t lowrank_bwd(int64_t max_rows, const int32_t* n_dev, int64_t r, int64_t f,
                       const float* dz, const void* rows_r, const void* proj, float* d_rows_r,
                       float* d_proj, void* ws, hipStream_t s) {
  const void* dzo = dz;
  if constexpr (sizeof(T) == 2) {
    const int64_t blocks = (max_rows * f / 8 + 255) / 256;
    if (blocks > 0)
      round_rows_kernel<T><<<dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)), dim3(256), 0,
                           s>>>(dz, ws, max_rows, n_dev, f);
    dzo = ws;
  }
  GemmArgs a = blank<T>();         // dE_r = dZ P: M = rows, N = r, K = f
  a.M = max_rows; a.N = r; a.K = f;
  a.a0 = dzo; a.lda = f;           // A(u, j) = dZ[u, j]
  a.b0 = proj; a.ldb = r;          // B(j, n) = P[j, n] (MN-major)
  a.c0 = d_rows_r; a.ldc = r;
  a.m_dev = n_dev;
  // r is narrow (2 tiles of 256 at r = 512): 128 x 128 tiles keep every CU busy
  hipError_t e = run_tile<T, 128, 128, 2, 2, true, false, kEpiStore, float, kRowBytes, 2>(a, s);
  if (e != hipSuccess) return e;
  GemmArgs b = blank<T>();         // dP = dZ^T R_r: M = f, N = r, K = rows
  b.M = f; b.N = r; b.K = max_rows;
  b.a0 = dzo; b.lda = f;           // A(j, u) = dZ[u, j] (MN-major)
  b.b0 = rows_r; b.ldb = r;        // B(u, n) = R_r[u, n] (MN-major)
  b.c0 = d_proj; b.ldc = r;
  b.k_dev = n_dev;
  return run<T, false, false, kEpiStore, float>(b, s);
}

#define STAPLE_INST(T)                                                                          \
  template hipError_t lowrank_expand<T>(int64_t, const int32_t*, int64_t, int64_t, const void*,\
                                        const void*, void*, hipStream_t);                       \
  template hipError_t lowrank_bwd<T>(int64_t, const int32_t*, int64_t, int64_t, const float*,  \
                                     const void*, const void*, float*, float*, void*,           \
                                     hipStream_t);                                              \
  template hipError_t recompute_h<T>(int64_t, int64_t, const void*, const void*, void*,        \
                                     hipStream_t);                                              \
  template hipError_t gateup_fwd<T>(int64_t, const int32_t*, int64_t, int64_t, int64_t,        \
                                    const void*, const void*, const void*, const void*, int64_t,\
                                    const int32_t*, void*, void*, void*, hipStream_t, int*);     \
  template hipError_t down_fwd<T>(int64_t, int64_t, int64_t, const void*, const void*, void*,  \
                                  int, hipStream_t);                                            \
  template hipError_t dh_act<T>(int64_t, int64_t, int64_t, const void*, const void*,           \
                                const void*, const void*, void*, float*, hipStream_t);          \
  template hipError_t dx_bwd<T>(int64_t, int64_t, int64_t, const void*, const void*,           \
                                const void*, void*, int, hipStream_t);                          \
  template hipError_t dwdown_bwd<T>(int64_t, int64_t, int64_t, const void*, const void*,       \
                                    float*, hipStream_t);                                       \
  template hipError_t dwgu_bwd<T>(int64_t, int64_t, int64_t, const void*, const void*, float*, \
                                  float*, bool, hipStream_t);

STAPLE_INST(bf16_t)
STAPLE_INST(float)

}  // namespace staple
