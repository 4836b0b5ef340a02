// Decode-shaped (at most 64 tokens) forward kernels: the weights are streamed
// from HBM exactly once and the small activation block is re-read from L2.
//
// Both kernels put the weight matrix on the MFMA's A side (16-row blocks of
// v_mfma_f32_16x16x32_bf16) and the tokens on the B side (four 16-token
// tiles).  A 64-wide "macro step" of k is 128 bytes of every row; lane
// (r, q) = (lane % 16, lane / 16) holds bytes [16q, 16q+16) and
// [64+16q, 64+16q+16) of row r, and the j-th MFMA of the step takes the j-th
// of them.  Weights come either row-major (each load instruction reads 64
// contiguous bytes of 16 rows) or packed in exactly this order (each load
// instruction reads 1 KB of contiguous memory; see decode_pack_kernel).  The
// activation, which every workgroup reads, is loaded by dedicated loader waves
// as whole cache lines straight into LDS and read back in the fragment
// pattern, so the compute waves' load queue holds weights only.  A and B use
// the same k order, so the contraction is unchanged.
//
// Gate/up: one workgroup per 4 groups of 8 features (6 groups when d_ff has
// more than four groups per CU); each compute wave owns the gate and up rows
// of one group over a part of d_model, the parts are folded in LDS,
// and the epilogue gathers each token's table row, forms u = W_up x + E[t]
// and h = silu(W_gate x) * u (STAPLE abstract: the up-projection is retained
// and the embedding added as a residual path; retrieval-path table: row
// reconstruction fused with the FFN) and stores h with 16-byte vectors.
// The STEM layer, which has no up-projection (the table row replaces it,
// STAPLE abstract and Table 4's STEM row), runs the same kernel on W_gate
// alone: a wave owns the gate rows of 16 features and u = E[t].  When the
// rows are read in place (a row index selects a cache slot or, negative, a
// row of the table itself, e.g. in pinned host memory), one more wave per
// workgroup loads every token's slice of its row into LDS while the weights
// stream, so that no compute wave waits on those loads (STAPLE
// retrieval-path table, Decode row: misses read zero-copy).
//
// Down: d_model is too narrow to fill 256 CUs with whole-K tiles, so the K
// range (d_ff) is split over several workgroups per output block; each writes
// an fp32 partial and a second small kernel sums the partials in split order
// (deterministic) and stores y.
#include <type_traits>

#include "common.h"

namespace staple {

constexpr int kDecMaxTokens = 64;
constexpr int kDownSplitMax = 8;

// Two 16-byte loads of one 128-byte macro step: lane (r, q) = (lane % 16,
// lane / 16) reads bytes [16q, 16q + 16) and [64 + 16q, 64 + 16q + 16), so
// each load instruction covers 64 contiguous bytes of 16 rows.
struct Frag2 {
  uint4 v[2];
};

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) {
  return __builtin_bit_cast(bf16x8_t, u);
}

// acc[a * NB + b] += A_a x B_b over the step (two v_mfma_f32_16x16x32_bf16:
// the j-th takes the j-th load of every lane, i.e. k-octets 4j..4j+3).
template <int NA, int NB>
__device__ __forceinline__ void mma_step(const Frag2 (&a)[NA], const Frag2 (&b)[NB],
                                         f32x4_t (&acc)[NA * NB]) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int k = 0; k < NB; ++k)
        acc[i * NB + k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(a[i].v[j]), as_bf16x8(b[k].v[j]), acc[i * NB + k], 0, 0, 0);
}

typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;

// The activation block of one macro step in LDS: 64 tokens x 128 bytes, token
// t's 16-byte chunk c at t * 128 + ((c ^ ((t >> 1) & 7)) << 4); the XOR keeps
// every 16-lane group of the Frag2-pattern reads on distinct banks.  It is
// loaded straight from global memory into LDS by eight 1 KB instructions,
// load i covering tokens 8i .. 8i+7 as whole cache lines: lane l writes LDS
// bytes 1024 i + 16 l, i.e. token 8i + l / 8 at position l % 8, so it fetches
// the chunk that position holds, (l % 8) ^ ((t >> 1) & 7).
constexpr int kXBlock = 64 * 128;

__device__ __forceinline__ int xblock_at(int t, int c) { return t * 128 + ((c ^ ((t >> 1) & 7)) << 4); }

// Activation ring: A steps in flight, one more slot than that (A + 1 slots)
// so the slot a load lands in was read two barriers earlier.

// Roles in a decode workgroup of (G + 1) KH waves: waves 0 .. G KH - 1
// compute (row group w % G, K part w / G); wave G KH + p loads part p's
// activation.  With RW, one more wave (the last) loads the workgroup's
// table-row slices into LDS for the epilogue (it counts as a loader for the
// barriers and the fold).
struct WaveRole {
  bool loader;
  int grp, part;
  bool row;
};
template <int G, int KH, bool RW = false>
__device__ __forceinline__ WaveRole wave_role() {
  const int wid = threadIdx.x >> 6;
  if (RW && wid == (G + 1) * KH) return {true, 0, 0, true};
  if (wid >= G * KH) return {true, 0, wid - G * KH, false};
  return {false, wid % G, wid / G, false};
}

// 16-byte pieces of zeros: the source of table-row pieces that do not exist.
__device__ const uint4 g_decode_zero_rows[16] = {};

// One compute wave's 16 weight rows (pa: the lane's bytes at step 0; step s
// at pa + s * wstep and pa + s * wstep + JOFF: row-major rows have wstep 128
// and JOFF 64, packed fragments JOFF 1024) times the activation of at most 64
// tokens (act[act_row(t)]: token t's row) over macro steps [s0, s1) of its K
// part; acc[k] is token tile k.
//
// The four compute waves of a part share the part's activation, which its
// loader wave brings into a ring of A + 1 LDS slots (kXBlock per part) with
// global-to-LDS loads A steps ahead, waiting on its own load counter only.  Compute waves issue only weight loads (WD steps ahead, 8
// registers per step), so a weight wait never waits behind activation loads
// and the reverse.  One barrier per step: before barrier i the loader's step
// i + 1 has landed, and its next load targets the slot read at step i - 1.
// Every wave runs the same number of steps, `len_max` (steps past s1 re-read
// the last valid step with zeroed weights), so the barriers match; a compute
// wave with `active` false (a row group past the end of the matrix, pa still
// pointing at valid memory) runs them with zeroed weights too.
// `after_prologue` runs on compute waves once their first loads are issued.
// A row wave (role.row) runs `row_issue` (loads it does not wait for here),
// in two phases around the first barrier, and then only joins the barriers,
// so its loads, however slow, hold up no other wave; the caller waits for
// them after the stream.
template <int WD, int A, int KH, int JOFF, typename RowFn, typename Hook, typename RowIssue>
__device__ __forceinline__ void stream_act_ring(WaveRole role, bool active, const char* pa, int64_t wstep,
                                                const uint16_t* act, int64_t act_ld, RowFn act_row,
                                                int n, lds_char* xl, int64_t s0, int64_t s1,
                                                int64_t len_max, f32x4_t (&acc)[4],
                                                Hook&& after_prologue, RowIssue&& row_issue) {
  constexpr int NB = 4, NS = A + 1;
  constexpr int U = NS % WD == 0 ? NS : NS * WD;   // unrolled steps: static slot and register indices
  constexpr int kSlot = KH * kXBlock;
  const int lane = threadIdx.x & 63;
  auto clamp = [&](int64_t s) -> int64_t { return s < s1 ? s : s1 - 1; };
#pragma unroll
  for (int k = 0; k < NB; ++k)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[k][i] = 0.0f;
  const int64_t ngroups = len_max > 0 ? (len_max + U - 1) / U : 0;
  if (role.row) {
    // row_issue(0) before the first barrier, row_issue(1) right after it, so
    // that work which must wait for loads of its own (row indices) is done
    // while the first step computes instead of before it starts
    row_issue(0);
    if (len_max > 0) {
      lds_barrier();
      row_issue(1);
      for (int64_t it = 0; it < ngroups; ++it)
#pragma unroll
        for (int j = 0; j < U; ++j) lds_barrier();
    } else {
      row_issue(1);
    }
    return;
  }
  if (len_max <= 0) {   // uniform over the workgroup
    if (!role.loader) after_prologue();
    return;
  }

  if (role.loader) {
    const char* px[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = 8 * i + (lane >> 3);
      const int chunk = (lane & 7) ^ ((t >> 1) & 7);
      px[i] = reinterpret_cast<const char*>(act + act_row(min(t, n - 1)) * act_ld) + chunk * 16;
    }
    lds_char* base = xl + role.part * kXBlock;
    auto issue = [&](int64_t s, int slot) {
      const int64_t o = clamp(s) * 128;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(px[i] + o),
                                         static_cast<lds_void*>(base + slot * kSlot + i * 1024), 16, 0, 0);
    };
#pragma unroll
    for (int j = 0; j < A; ++j) issue(s0 + j, j);
    wait_vmcnt<8 * (A - 1)>();
    lds_barrier();
    for (int64_t it = 0; it < ngroups; ++it) {
#pragma unroll
      for (int j = 0; j < U; ++j) {
        issue(s0 + it * U + j + A, (j + A) % NS);
        wait_vmcnt<8 * (A - 1)>();
        lds_barrier();
      }
    }
    return;
  }

  const int r = lane & 15, q = lane >> 4;
  auto load_w = [&](Frag2& fr, int64_t s) {
    const char* p = pa + clamp(s) * wstep;
    fr.v[0] = *reinterpret_cast<const uint4*>(p);
    fr.v[1] = *reinterpret_cast<const uint4*>(p + JOFF);
  };
  Frag2 a[WD];
#pragma unroll
  for (int j = 0; j < WD; ++j) load_w(a[j], s0 + j);
  after_prologue();
  lds_barrier();
  for (int64_t it = 0; it < ngroups; ++it) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t s = s0 + it * U + j;
      __builtin_amdgcn_sched_barrier(0);
      const lds_char* cur = xl + (j % NS) * kSlot + role.part * kXBlock;
      Frag2 b[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int t = 16 * k + r;
        b[k].v[0] = __builtin_bit_cast(uint4, *reinterpret_cast<const lds_u32x4*>(cur + xblock_at(t, q)));
        b[k].v[1] = __builtin_bit_cast(uint4, *reinterpret_cast<const lds_u32x4*>(cur + xblock_at(t, q + 4)));
      }
      const int wi = j % WD;
      const uint32_t keep = (active && s < s1) ? 0xffffffffu : 0u;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        a[wi].v[jj].x &= keep; a[wi].v[jj].y &= keep;
        a[wi].v[jj].z &= keep; a[wi].v[jj].w &= keep;
      }
      const Frag2 aa[1] = {a[wi]};
      mma_step<1, NB>(aa, b, acc);
      __builtin_amdgcn_sched_barrier(0);
      load_w(a[wi], s + WD);
      lds_barrier();
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Stages one wave's 16-row x 64-token MFMA result so that lane t can read
// row e of its token at st[e * kStageLd + t].
constexpr int kStageLd = 65;
template <bool ADD = false>
__device__ __forceinline__ void stage_wave_rows(float* st, const f32x4_t (&acc)[4]) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float& e = st[(4 * q + i) * kStageLd + 16 * k + r];
      if constexpr (ADD) e += acc[k][i];
      else e = acc[k][i];
    }
}

// Folds the KH parts of a workgroup's K range: the part-k compute waves
// (k >= 1) add their sums into the staged rows of their row group in part
// order; loader waves only join the barriers.  On return stage[grp] holds the
// full sums and only part-0 compute waves go on.  (stage: one 16-row block
// per row group.)
template <int KH>
__device__ __forceinline__ bool fold_parts(WaveRole role, float (*stage)[16 * kStageLd],
                                           const f32x4_t (&acc)[4]) {
  if (!role.loader && role.part == 0) stage_wave_rows(stage[role.grp], acc);
#pragma unroll
  for (int k = 1; k < KH; ++k) {
    __syncthreads();
    if (!role.loader && role.part == k) stage_wave_rows<true>(stage[role.grp], acc);
  }
  if constexpr (KH > 1) __syncthreads();
  return !role.loader && role.part == 0;
}

// Gate/up for at most 64 tokens, features split over the waves: one
// workgroup (G KH compute waves and KH activation loaders) per FG G features;
// compute wave w owns one 16-row MFMA block over part w / G of d_model, and
// the KH parts are folded in LDS.  With UP (the STAPLE layer, FG = 8) the
// block is the gate rows then the up rows of features 8 (w % G) .. +8 of the
// workgroup; without (the STEM layer, FG = 16) it is the gate rows of
// features 16 (w % G) .. +16 and u is the table row.  Row groups past f (in
// the last workgroup when f / FG is not a multiple of G) stream nothing and
// store nothing.
// With `pos`, the n tokens of the launch are pos[0 .. n) of the n_tokens rows
// of x, h, g, u and row_index (out-of-range positions set the error word and
// are neither read nor written).
// 16-byte pieces one copy-wave lane carries (RowCopyJob): the launcher sizes
// each job to fit grid x 64 x kCopyVecs pieces.
constexpr int kCopyVecs = 8;

template <typename P>
__device__ __forceinline__ P pick4(const P (&a)[kCopyJobLayers], int j) {
  return j == 0 ? a[0] : j == 1 ? a[1] : j == 2 ? a[2] : a[3];
}

// Source of a token's table row for the gate/up epilogue: row index v =
// row_index[token]; with `table`, a negative v = -1 - id selects row id of
// the table (e.g. pinned host memory, read in place) and a non-negative one
// row v of `rows` (e.g. the HBM cache).  (A free function of plain values:
// as a lambda over captured variables the compiler selected between the
// addresses of the two row strides and kept both in scratch memory.)
__device__ __forceinline__ const uint16_t* decode_row_src(const uint16_t* table, int64_t vocab,
                                                          int64_t table_ld, const uint16_t* rows,
                                                          int64_t n_rows, int64_t f, int64_t v,
                                                          bool& ok) {
  if (table && v < 0) {
    ok = -1 - v < vocab;
    return table + (-1 - v) * table_ld;
  }
  ok = v >= 0 && v < n_rows;
  return rows + v * f;
}

template <int WD, int A, int G, int KH, bool PACKED, bool UP, bool RW = false, bool CW = false>
__global__ __launch_bounds__(64 * ((G + 1) * KH + (RW || CW ? 1 : 0))) void decode_gateup_kernel(
    int n, const int32_t* __restrict__ pos, int64_t n_tokens, int64_t d, int64_t f,
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg,
    const uint16_t* __restrict__ wu, const uint16_t* __restrict__ rows, int64_t n_rows,
    const int32_t* __restrict__ row_index, uint16_t* __restrict__ h, uint16_t* __restrict__ g_out,
    uint16_t* __restrict__ u_out, int* err, const uint16_t* __restrict__ table, int64_t vocab,
    int64_t table_ld, RowCopyJob job) {
  static_assert(!(RW && CW), "one extra wave");
  constexpr int FG = UP ? 8 : 16;                                   // features per row group
  // RW: the workgroup's G FG features of each token's table row, token t at
  // byte t kSliceBytes, loaded by the row wave
  constexpr int kSliceBytes = G * FG * 2;
  __shared__ __attribute__((aligned(16))) char xs[(A + 1) * KH * kXBlock];
  __shared__ float stage[G][16 * kStageLd];
  __shared__ __attribute__((aligned(16))) char erows[RW ? 64 * kSliceBytes : 16];
  __shared__ __attribute__((aligned(16))) char cbuf[CW ? kCopyVecs * 1024 : 16];
  const int lane = threadIdx.x & 63;
  const WaveRole role = wave_role<G, KH, RW || CW>();
  const int grp = role.grp, part = role.part;
  const int r = lane & 15, q = lane >> 4;
  const int64_t rb = static_cast<int64_t>(blockIdx.x) * G + grp;   // this wave's row group
  const bool active = rb < f / FG;
  const int64_t rbc = active ? rb : 0;                              // valid memory for the rest
  const int64_t f0 = rbc * FG;                                      // this wave's features
  // PACKED: wg is the packed gate/up (or gate) block of this row group
  const uint16_t* wrow = !UP ? wg + (f0 + r) * d : r < 8 ? wg + (f0 + r) * d : wu + (f0 + r - 8) * d;
  const char* pa = PACKED ? reinterpret_cast<const char*>(wg) + rbc * 2048 + lane * 16
                          : reinterpret_cast<const char*>(wrow) + q * 16;
  const int64_t wstep = PACKED ? (f / FG) * 2048 : 128;
  const int64_t T = d / 64, len = (T + KH - 1) / KH;
  const int64_t s0 = part * len < T ? part * len : T, s1 = s0 + len < T ? s0 + len : T;
  f32x4_t acc[4];
  // token position of launch token t (-1 when out of range)
  auto tok_of = [&](int t) -> int64_t {
    if (!pos) return t;
    const int64_t p = pos[t];
    return p >= 0 && p < n_tokens ? p : -1;
  };
  auto act_row = [&](int t) -> int64_t {
    const int64_t p = tok_of(t);
    return p < 0 ? 0 : p;
  };
  const int64_t tok = tok_of(min(lane, n - 1));
  // the epilogue's table row of a token (row index v = row_index[token])
  auto row_of = [&](int64_t v, bool& ok) -> const uint16_t* {
    return decode_row_src(table, vocab, table_ld, rows, n_rows, f, v, ok);
  };
  // Without RW each compute wave fetches its lane's token's row (this wave's
  // features) once the stream is under way.  With RW the row wave loads the
  // slices of all tokens straight into LDS (zeros for a bad index, which it
  // flags), and no compute wave waits on those loads.
  bool erow_ok = true;
  uint4 erow[FG / 8];
  auto fetch_row = [&]() {
    if constexpr (!RW) {
      const uint16_t* src = row_of(row_index[tok < 0 ? 0 : tok], erow_ok);
#pragma unroll
      for (int c = 0; c < FG / 8; ++c)
        erow[c] = *reinterpret_cast<const uint4*>(erow_ok ? src + f0 + 8 * c : x);
    }
  };
  auto row_issue = [&](int phase) {
    if constexpr (RW) {
      if (phase != 0) return;
      constexpr int kPieces = kSliceBytes / 16;          // per token; one 1 KB load per piece
      const int64_t fbase = static_cast<int64_t>(blockIdx.x) * G * FG;
      const int64_t p = tok_of(min(lane, n - 1));
      bool ok = false;
      const uint16_t* src = p < 0 ? nullptr : row_of(row_index[p], ok);
      if (p >= 0 && !ok && lane < n) flag_index_error(err);
      const unsigned long long base =
          ok ? reinterpret_cast<unsigned long long>(src + fbase) : 0ull;
#pragma unroll
      for (int i = 0; i < kPieces; ++i) {
        const int c = i * 64 + lane, t = c / kPieces, k = c % kPieces;
        const unsigned long long b = __shfl(base, t, 64);
        const bool use = t < n && b != 0ull && fbase + 8 * k < f;
        const void* g = use ? reinterpret_cast<const void*>(b + 16ull * k)
                            : static_cast<const void*>(g_decode_zero_rows + k);
        __builtin_amdgcn_global_load_lds(g, static_cast<lds_void*>((lds_char*)(erows) + i * 1024), 16, 0, 0);
      }
    }
  };
  // CW: the extra wave carries compact-row copies of other layers (job).
  // Before the stream it fetches the row indices of its pieces (one wait),
  // then loads every piece straight into LDS (global-to-LDS, over PCIe for
  // rows of a pinned host table) with no wait in between; it joins the
  // stream's barriers without waiting for them, and after the stream waits
  // once and writes the pieces to their compact rows.  So the copies hide
  // under the weight stream and hold up no compute wave, and no piece is
  // held in registers across the stream.
  // The job's rows (unique row u, layer j) of this launch, token-major (the
  // rows of one token over the job's layers side by side: one contiguous
  // read when the tables are interleaved token-major), are cut into job.per
  // segments each; workgroup b copies segment b % per of row b / per, lane l
  // its 16-byte pieces l, l + 64, ... (the launcher sizes job.seg to fit the
  // wave).  The row's unique index does not depend on the device count, so
  // the count, the cache code and the ID are loaded together and waited for
  // once; this runs right after the stream's first barrier, beside the first
  // step's MFMAs, and the pieces' loads are then never waited for before the
  // stream ends.
  uint32_t cmask = 0;            // pieces this lane loaded
  int64_t c_dst = 0;             // byte offset of the segment in its compact-row block
  int c_j = 0;                   // its layer in the job
  auto copy_issue = [&](int phase) {
    if constexpr (CW) {
      if (phase != 1) return;
      const uint32_t per = static_cast<uint32_t>(job.per);
      const uint32_t r = blockIdx.x / per, sg = blockIdx.x - r * per;
      if (r >= static_cast<uint32_t>(job.rows_max)) return;
      const uint32_t nl = static_cast<uint32_t>(job.n_layers);
      const uint32_t i = r / nl;
      c_j = static_cast<int>(r - i * nl);
      const int64_t u = job.part + static_cast<int64_t>(job.parts) * i;
      const int64_t u_ld = u < job.max_unique ? u : job.max_unique - 1;
      const int64_t nu = *job.n_unique;
      const int32_t code = job.code[u_ld];
      const int32_t id = job.uniq[u_ld];
      if (u >= nu || u >= job.max_unique) return;
      const char* src;
      if (code >= 0) {
        if (code >= job.capacity) {
          if (lane == 0) flag_index_error(err);
          return;
        }
        src = static_cast<const char*>(pick4(job.cache_rows, c_j)) + code * job.row_bytes;
      } else {
        if (id < 0 || id >= job.vocab) {
          if (lane == 0) flag_index_error(err);
          return;
        }
        src = static_cast<const char*>(pick4(job.table, c_j)) + id * pick4(job.table_ld, c_j);
      }
      const uint32_t vecs = static_cast<uint32_t>(job.row_bytes / 16);
      const uint32_t c0 = sg * static_cast<uint32_t>(job.seg);
      const uint32_t c1 = min(c0 + static_cast<uint32_t>(job.seg), vecs);
      c_dst = u * job.row_bytes + static_cast<int64_t>(c0) * 16;
      src += static_cast<int64_t>(c0) * 16;
#pragma unroll
      for (int k = 0; k < kCopyVecs; ++k) {
        const uint32_t c = static_cast<uint32_t>(k) * 64u + lane;
        if (c0 + c < c1) {
          __builtin_amdgcn_global_load_lds(src + c * 16u,
                                           static_cast<lds_void*>((lds_char*)(cbuf) + k * 1024), 16, 0, 0);
          cmask |= 1u << k;
        }
      }
    } else {
      row_issue(phase);
    }
  };
  stream_act_ring<WD, A, KH, PACKED ? 1024 : 64>(role, active, pa, wstep, x, d, act_row, n,
                                                  (lds_char*)(xs), s0, s1, len, acc, fetch_row,
                                                  copy_issue);
  if constexpr (CW) {
    if (role.row && cmask) {
      wait_vmcnt<0>();
      char* dst = static_cast<char*>(pick4(job.rows, c_j)) + c_dst;
#pragma unroll
      for (int k = 0; k < kCopyVecs; ++k) {
        if ((cmask >> k) & 1u)
          *reinterpret_cast<uint4*>(dst + (k * 64 + lane) * 16) =
              *reinterpret_cast<const uint4*>(cbuf + k * 1024 + lane * 16);
      }
    }
  }
  if constexpr (RW) {
    if (role.row) wait_vmcnt<0>();   // its pieces are in LDS
    __syncthreads();
    if (!role.loader) {
#pragma unroll
      for (int c = 0; c < FG / 8; ++c)
        erow[c] = *reinterpret_cast<const uint4*>(erows + lane * kSliceBytes + grp * FG * 2 + c * 16);
    }
  }

  // epilogue: the row group's block staged so that lane t holds its token's
  // 16 sums (UP: 8 gate then 8 up; STEM: 16 gate)
  if (!fold_parts<KH>(role, stage, acc) || !active) return;
  const float* st = stage[grp];
  const int t = lane;
  if (t >= n) return;
  if (tok < 0) {
    flag_index_error(err);
    return;
  }
  float gv[FG], uv[FG], hv[FG], ev[FG];
  if (erow_ok) {
#pragma unroll
    for (int c = 0; c < FG / 8; ++c) {
      const uint32_t wds[4] = {erow[c].x, erow[c].y, erow[c].z, erow[c].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ev[8 * c + 2 * i] = __uint_as_float(wds[i] << 16);
        ev[8 * c + 2 * i + 1] = __uint_as_float(wds[i] & 0xffff0000u);
      }
    }
  } else {
    flag_index_error(err);
#pragma unroll
    for (int i = 0; i < FG; ++i) ev[i] = 0.0f;
  }
#pragma unroll
  for (int e = 0; e < FG; ++e) {
    gv[e] = st[e * kStageLd + t];
    uv[e] = UP ? st[(8 + e) * kStageLd + t] + ev[e] : ev[e];
    hv[e] = gv[e] * sigmoidf_(gv[e]) * uv[e];
  }
  auto pack = [](const float* v) {
    uint4 o;
    o.x = pack_bf16x2(v[0], v[1]);
    o.y = pack_bf16x2(v[2], v[3]);
    o.z = pack_bf16x2(v[4], v[5]);
    o.w = pack_bf16x2(v[6], v[7]);
    return o;
  };
  const int64_t o = tok * f + f0;
#pragma unroll
  for (int c = 0; c < FG / 8; ++c) {
    *reinterpret_cast<uint4*>(h + o + 8 * c) = pack(hv + 8 * c);
    if (g_out) *reinterpret_cast<uint4*>(g_out + o + 8 * c) = pack(gv + 8 * c);
    if (u_out) *reinterpret_cast<uint4*>(u_out + o + 8 * c) = pack(uv + 8 * c);
  }
}

// Down projection for at most 64 tokens, d_ff split KS ways over workgroups
// and KH ways inside one: workgroup (output block b of 16 G, split ks) with
// compute wave w owning outputs 16 G b + 16 (w % G) .. +16 over part w / G of
// the split's steps (plus KH activation loaders); writes partial[ks][t][n] in
// fp32.  Row groups past d_model (in the last block when d / 16 is not a
// multiple of G) stream nothing and write nothing.
template <int WD, int A, int G, int KS, int KH, bool PACKED>
__global__ __launch_bounds__(64 * (G + 1) * KH) void decode_down_kernel(int n, int64_t d, int64_t f,
                                                                       const uint16_t* __restrict__ h,
                                                                       const uint16_t* __restrict__ wd,
                                                                       float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) char xs[(A + 1) * KH * kXBlock];
  __shared__ float stage[G][16 * kStageLd];
  const int lane = threadIdx.x & 63;
  const WaveRole role = wave_role<G, KH>();
  const int grp = role.grp, part = role.part;
  const int r = lane & 15, q = lane >> 4;
  // workgroup id -> (split, output block) split-minor: consecutive ids go to
  // different XCDs, so each XCD's workgroups share few d_ff slices of h and
  // fetch only those into their L2
  const int ks = static_cast<int>(blockIdx.x % KS);
  const int64_t blk = blockIdx.x / KS;
  const int64_t rb = blk * G + grp;           // this wave's 16-output row group
  const bool active = rb < d / 16;
  const int64_t rbc = active ? rb : 0;        // valid memory for the rest
  const int64_t n0 = rbc * 16;
  const int64_t T = f / 64;
  const int64_t k0 = T * ks / KS, k1 = T * (ks + 1) / KS;
  const int64_t len = (k1 - k0 + KH - 1) / KH;
  const int64_t s0 = k0 + part * len < k1 ? k0 + part * len : k1;
  const int64_t s1 = s0 + len < k1 ? s0 + len : k1;
  // PACKED: wd is the packed down block (row block = 16 outputs)
  const char* pa =
      PACKED ? reinterpret_cast<const char*>(wd) + rbc * 2048 + lane * 16
             : reinterpret_cast<const char*>(wd + (n0 + r) * f) + q * 16;
  const int64_t wstep = PACKED ? (d / 16) * 2048 : 128;
  f32x4_t acc[4];
  stream_act_ring<WD, A, KH, PACKED ? 1024 : 64>(role, active, pa, wstep, h, f,
                                                  [](int t) -> int64_t { return t; }, n,
                                                  (lds_char*)(xs), s0, s1, len, acc, []() {},
                                                  [](int) {});
  if (!fold_parts<KH>(role, stage, acc) || !active) return;
  const float* st = stage[grp];
  const int t = lane;
  if (t >= n) return;
  float* dst = partial + (static_cast<int64_t>(ks) * n + t) * d + n0;
#pragma unroll
  for (int e0 = 0; e0 < 16; e0 += 4)
    *reinterpret_cast<float4*>(dst + e0) =
        make_float4(st[e0 * kStageLd + t], st[(e0 + 1) * kStageLd + t], st[(e0 + 2) * kStageLd + t],
                    st[(e0 + 3) * kStageLd + t]);
}

template <typename OutT>
__global__ void decode_down_reduce_kernel(int64_t count, int ksplit, const float* __restrict__ partial,
                                          OutT* __restrict__ y) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i >= count) return;
  float4 s = *reinterpret_cast<const float4*>(partial + i);
#pragma unroll
  for (int ks = 1; ks < ksplit; ++ks) {
    const float4 p = *reinterpret_cast<const float4*>(partial + ks * count + i);
    s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
  }
  if constexpr (sizeof(OutT) == 4) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + i) = s;
  } else {
    uint2 o;
    o.x = pack_bf16x2(s.x, s.y);
    o.y = pack_bf16x2(s.z, s.w);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + i) = o;
  }
}

// Packed weights for the decode kernels: a [R x K] bf16 operand becomes
// K/64 steps of R/16 row blocks, each block two 1 KB loads of 64 lanes x 16
// bytes in the Frag2 pattern: byte ((s * R/16 + rb) * 2 + j) * 1024 + 16 lane
// holds bytes [128 s + 64 j + 16 (lane / 16), +16) of block row lane % 16.
// A gate/up row block is features 8 rb .. 8 rb + 8: its rows 0-7 are those
// rows of W_gate and rows 8-15 those of W_up; a down row block is rows
// 16 rb .. 16 rb + 16 of W_down, and a gate-only block (the STEM layer) rows
// 16 rb .. 16 rb + 16 of W_gate.  Step-major order over all row blocks puts
// what the whole grid reads at one step side by side in HBM, and every load
// instruction of the decode kernels reads 1 KB of contiguous memory.
__global__ void decode_pack_kernel(int64_t total, int64_t rb_count, int64_t k, bool gate_up,
                                   const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
                                   uint4* __restrict__ out) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (c >= total) return;
  const int lane = static_cast<int>(c & 63), j = static_cast<int>((c >> 6) & 1);
  const int64_t blk = c >> 7, rb = blk % rb_count, s = blk / rb_count;
  const int r = lane & 15, q = lane >> 4;
  const uint16_t* row = gate_up ? (r < 8 ? a + (8 * rb + r) * k : b + (8 * rb + r - 8) * k) : a + (16 * rb + r) * k;
  out[c] = *reinterpret_cast<const uint4*>(row + s * 64 + j * 32 + q * 8);
}

bool decode_eligible(int64_t n, int64_t d, int64_t f, int dtype) {
  return dtype == STAPLE_BF16 && n >= 1 && n <= kDecMaxTokens && d % 64 == 0 && f % 64 == 0;
}

size_t decode_down_workspace_bytes(int64_t n, int64_t d) {
  return static_cast<size_t>(kDownSplitMax) * n * d * sizeof(float);
}

// Launch shapes of the two decode kernels (measured on MI355X, batch 64,
// d_model 2048 / d_ff 8192 and 4096 / 11008): gate/up on 8 waves (d_model in
// two parts) with two steps in flight per wave; down on 4 waves with four
// steps in flight and d_ff split over about one workgroup per CU (8 ways for
// 32 output blocks, 4 for 64, 2 from 128 on).
// Deeper prefetch, 2 or 4 steps per barrier, other split counts, and the
// earlier layouts that split d_model (or d_ff) over the waves of a workgroup
// and folded their partial sums in LDS all measured slower.
constexpr int kGateUpAhead = 2;      // weight steps in flight per compute wave
constexpr int kGateUpAheadLong = 4;  // the same for the 6-group, one-part shape (whole-d_model
                                     // streams: 64 steps per wave at d_model 4096; 31.3 us
                                     // against 31.5-32.6 us with 2 at 4096 x 11008)
constexpr int kGateUpActAhead = 3;   // activation steps in flight per loader wave
constexpr int kGateUpParts = 2;      // d_model split in two inside a 4-group gate/up workgroup
constexpr int kDownAhead = 2;
constexpr int kDownActAhead = 3;
constexpr int kDownParts = 2;

int decode_down_splits(int64_t d) {
  const int64_t blocks = d / 64;
  return blocks <= 32 ? 8 : blocks <= 64 ? 4 : 2;
}

hipError_t decode_pack(int64_t d, int64_t f, const void* wg, const void* wu, const void* wd,
                       void* packed_gu, void* packed_down, hipStream_t s) {
  auto go = [&](int64_t rbs, int64_t k, bool gu, const void* a, const void* b, void* out) {
    const int64_t total = rbs * (k / 64) * 128;
    decode_pack_kernel<<<dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s>>>(
        total, rbs, k, gu, static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b),
        static_cast<uint4*>(out));
  };
  if (packed_gu) {
    if (wu) go(f / 8, d, true, wg, wu, packed_gu);
    else go(f / 16, d, false, wg, nullptr, packed_gu);   // gate-only blocks
  }
  if (packed_down) go(d / 16, f, false, wd, nullptr, packed_down);
  return hipGetLastError();
}

// `up`: the weights hold W_up (the STAPLE layer; row-major: wu, packed: the
// interleaved blocks) or not (the STEM layer: W_gate alone, u = E[t]).
int decode_gateup_grid(int64_t f, bool up) {
  const int64_t groups = up ? f / 8 : f / 16;
  const int64_t cus = device_cus();
  const bool wide = groups > 4 * cus;
  const int per = up ? (wide ? 6 : 4)
                     : (groups <= 2 * cus ? 2 : groups <= 3 * cus ? 3 : wide ? 6 : 4);
  return static_cast<int>((groups + per - 1) / per);
}

// The segments of a gate/up launch's copy job of at most `rows` compact rows
// of d_ff f: every row gets gridDim / rows workgroups; false when a
// workgroup's segment would not fit its copy wave (64 lanes x kCopyVecs
// pieces of 16 bytes).
bool decode_copy_plan(int64_t rows, int64_t f, bool up, int* per, int* seg) {
  const int64_t grid = decode_gateup_grid(f, up);
  if (rows <= 0 || rows > grid) return false;
  const int64_t p = grid / rows, vecs = f * 2 / 16, sz = (vecs + p - 1) / p;
  if (sz > 64 * kCopyVecs) return false;
  *per = static_cast<int>(p);
  *seg = static_cast<int>(sz);
  return true;
}

hipError_t decode_gateup(int64_t n, const int32_t* pos, int64_t n_tokens, int64_t d, int64_t f,
                         const void* x, const void* wg, const void* wu, const void* rows,
                         int64_t n_rows, const int32_t* row_index, void* h, void* g_out,
                         void* u_out, hipStream_t s, int* err, bool packed, bool up,
                         const void* table, int64_t vocab, int64_t table_ld,
                         const RowCopyJob* job) {
  if (table_ld <= 0) table_ld = f;
  if (job && (table || !packed)) return hipErrorInvalidValue;   // copies ride the packed kernel only
  // STAPLE: 4 row groups (32 features) per workgroup, on two K parts, while
  // that fits one workgroup per CU; else 6 row groups on one part (d_ff
  // 11008: 230 workgroups of 7 waves instead of 344 of 10 on 256 CUs whose
  // LDS holds one 10-wave workgroup each: 32 us instead of 44 per launch at
  // d_model 4096).
  // STEM (16-feature row groups, half the bytes per feature): as many row
  // groups per workgroup as make about one workgroup per CU, 2, 3 or 4 on two
  // K parts, else 6 on one.
  const int64_t groups = up ? f / 8 : f / 16;
  const int64_t cus = device_cus();
  const bool wide = groups > 4 * cus;
  const int per = up ? (wide ? 6 : 4)
                     : (groups <= 2 * cus ? 2 : groups <= 3 * cus ? 3 : wide ? 6 : 4);
  const unsigned grid = static_cast<unsigned>((groups + per - 1) / per);
  const RowCopyJob no_job{};
  auto go = [&](auto kern, int threads) {
    if (table || job) threads += 64;   // the row wave or the copy wave
    kern<<<dim3(grid), dim3(threads), 0, s>>>(
        static_cast<int>(n), pos, n_tokens, d, f, static_cast<const uint16_t*>(x),
        static_cast<const uint16_t*>(wg),
        static_cast<const uint16_t*>(wu), static_cast<const uint16_t*>(rows), n_rows, row_index,
        static_cast<uint16_t*>(h), static_cast<uint16_t*>(g_out), static_cast<uint16_t*>(u_out), err,
        static_cast<const uint16_t*>(table), vocab, table_ld, job ? *job : no_job);
  };
  auto pick = [&](auto packed_tag, auto up_tag, auto rw_tag, auto cw_tag) {
    constexpr bool P = decltype(packed_tag)::value, U = decltype(up_tag)::value;
    constexpr bool R = decltype(rw_tag)::value, C = decltype(cw_tag)::value;
    constexpr int WD = kGateUpAhead, A = kGateUpActAhead, KH = kGateUpParts;
    if (per == 6) go(decode_gateup_kernel<kGateUpAheadLong, A, 6, 1, P, U, R, C>, 64 * 7);
    else if (per == 4) go(decode_gateup_kernel<WD, A, 4, KH, P, U, R, C>, 64 * 5 * KH);
    else if constexpr (!U) {
      if (per == 3) go(decode_gateup_kernel<WD, A, 3, KH, P, U, R, C>, 64 * 4 * KH);
      else go(decode_gateup_kernel<WD, A, 2, KH, P, U, R, C>, 64 * 3 * KH);
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  // rows read in place (a table given): packed weights only, with the row wave
  if (table && !packed) return hipErrorInvalidValue;
  if (table && up) pick(T_{}, T_{}, T_{}, F_{});
  else if (table) pick(T_{}, F_{}, T_{}, F_{});
  else if (job && up) pick(T_{}, T_{}, F_{}, T_{});
  else if (job) pick(T_{}, F_{}, F_{}, T_{});
  else if (packed && up) pick(T_{}, T_{}, F_{}, F_{});
  else if (packed) pick(T_{}, F_{}, F_{}, F_{});
  else if (up) pick(F_{}, T_{}, F_{}, F_{});
  else pick(F_{}, F_{}, F_{}, F_{});
  return hipGetLastError();
}

hipError_t decode_down(int64_t n, int64_t d, int64_t f, const void* h, const void* wd, void* y,
                       int out_dtype, void* ws, hipStream_t s, bool packed) {
  float* partial = static_cast<float*>(ws);
  const int ks = decode_down_splits(d);
  auto go = [&](auto kern) {
    kern<<<dim3(static_cast<unsigned>(d / 64 * ks)), dim3(320 * kDownParts), 0, s>>>(
        static_cast<int>(n), d, f, static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(wd),
        partial);
  };
  auto pick = [&](auto packed_tag) {
    constexpr bool P = decltype(packed_tag)::value;
    if (ks == 8) go(decode_down_kernel<kDownAhead, kDownActAhead, 4, 8, kDownParts, P>);
    else if (ks == 4) go(decode_down_kernel<kDownAhead, kDownActAhead, 4, 4, kDownParts, P>);
    else go(decode_down_kernel<kDownAhead, kDownActAhead, 4, 2, kDownParts, P>);
  };
  if (packed) pick(std::true_type{});
  else pick(std::false_type{});
  const int64_t count = n * d;
  const unsigned blocks = static_cast<unsigned>((count / 4 + 255) / 256);
  if (out_dtype == STAPLE_F32)
    decode_down_reduce_kernel<float><<<blocks, 256, 0, s>>>(count, ks, partial, static_cast<float*>(y));
  else
    decode_down_reduce_kernel<uint16_t><<<blocks, 256, 0, s>>>(count, ks, partial,
                                                               static_cast<uint16_t*>(y));
  return hipGetLastError();
}

}  // namespace staple
