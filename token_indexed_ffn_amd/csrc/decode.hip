// Decode-shaped (at most 64 tokens) forward kernels: the weights are streamed
// from HBM exactly once and the small activation block is re-read from L2.
//
// Both kernels put the weight matrix on the MFMA's A side (16-row blocks of
// v_mfma_f32_16x16x32_bf16) and the tokens on the B side (four 16-token
// tiles).  A 64-wide "macro step" of k is 128 bytes of every row; for the
// weights, lane (r, q) = (lane % 16, lane / 16) loads its bytes [16q, 16q+16)
// and [64+16q, 64+16q+16) straight into registers, so each load instruction
// reads 64 contiguous bytes of 16 rows, and the j-th MFMA of the step takes
// the j-th load of every lane.  The activation, which every workgroup reads,
// is loaded as whole cache lines and put into the same fragment pattern
// through LDS (half the cache-line requests of the fragment pattern).  A and
// B use the same k order, so the contraction is unchanged.
//
// Gate/up: one workgroup per 32 features; each of its four waves owns the
// gate and up rows of 8 features over all of d_model, the activation of each
// step is shared by the waves through LDS, and the epilogue gathers each
// token's table row, forms u = W_up x + E[t] and h = silu(W_gate x) * u
// (STAPLE abstract: the up-projection is retained and the embedding added as
// a residual path; retrieval-path table: row reconstruction fused with the
// FFN) and stores h with 16-byte vectors.
//
// Down: d_model is too narrow to fill 256 CUs with whole-K tiles, so the K
// range (d_ff) is split over several workgroups per output block (8 per 64
// outputs by default); each writes an fp32 partial and a second small kernel
// sums the partials in split order (deterministic) and stores y.
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
// t's 16-byte chunk c at t * 128 + ((c ^ ((t >> 1) & 7)) << 4).  It is loaded
// from global memory with eight 1 KB instructions that each cover 8 whole
// tokens x 128 bytes (full cache lines), written to LDS and read back in the
// Frag2 pattern; the XOR keeps every 16-lane group of both the writes and the
// reads on distinct banks.
constexpr int kXBlock = 64 * 128;

__device__ __forceinline__ int xblock_at(int t, int c) { return t * 128 + ((c ^ ((t >> 1) & 7)) << 4); }

// One wave's 16 weight rows (pa: the lane's bytes at step 0) times the
// activation of at most 64 tokens over macro steps [s0, s1).  The workgroup
// has 4 KH waves: waves w and w + 4 k (k < KH) stream the same 16 rows over
// KH parts of the K range (part k = wid / 4), and the four waves of one part
// share its activation: each step's block (64 tokens x 128 bytes, act[t]:
// token t's row) is loaded once per part as whole cache lines (two 1 KB loads
// per wave: tokens 16 (wid % 4) + l / 8 and 16 (wid % 4) + 8 + l / 8, chunk
// l % 8; act_row(t) gives the row of act that holds token t), written to one
// of two LDS slots (`xl`, 2 x KH x kXBlock bytes) and read by the part's four
// waves; one barrier per step hands a slot over.
// Every wave runs the same number of steps, `len_max` (waves with fewer read
// their last step again with zeroed weights), so the barriers match.
// Weights and activations are loaded WD steps ahead (8 + 8 registers per
// step): loads complete in issue order, so waiting for a step's activation
// also waits for every weight load issued before it.  `after_prologue` runs
// once the first steps are in flight.
// The weight bytes of step s are at pa + s * wstep and pa + s * wstep + JOFF
// (row-major rows: wstep 128, JOFF 64; packed fragments: JOFF 1024).
template <int WD, int KH, int JOFF, typename RowFn, typename Hook>
__device__ __forceinline__ void stream_shared_act(const char* pa, int64_t wstep, const uint16_t* act,
                                                  int64_t act_ld, RowFn act_row, int n, lds_char* xl,
                                                  int64_t s0, int64_t s1, int64_t len_max,
                                                  f32x4_t (&acc)[4], Hook&& after_prologue) {
  constexpr int NB = 4;
  constexpr int U = WD % 2 == 0 ? WD : 2 * WD;          // unrolled steps (even: LDS slot parity)
  constexpr int kSlot = KH * kXBlock;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int grp = wid & 3, part = wid >> 2;
  const int r = lane & 15, q = lane >> 4;
  const char* px[2];
  int wofs[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int tt = 16 * grp + 8 * i + (lane >> 3);
    px[i] = reinterpret_cast<const char*>(act + act_row(min(tt, n - 1)) * act_ld) + (lane & 7) * 16;
    wofs[i] = part * kXBlock + xblock_at(tt, lane & 7);
  }
  // steps past s1 (or an empty range) re-read a valid step: s1 - 1, or s0 - 1
  // (the previous part's last step) when the range is empty
  auto clamp = [&](int64_t s) -> int64_t { return s < s1 ? s : s1 - 1; };
  auto load_w = [&](Frag2& fr, int64_t s) {
    const char* p = pa + clamp(s) * wstep;
    fr.v[0] = *reinterpret_cast<const uint4*>(p);
    fr.v[1] = *reinterpret_cast<const uint4*>(p + JOFF);
  };
  auto load_x = [&](uint4 (&dst)[2], int64_t s) {
#pragma unroll
    for (int i = 0; i < 2; ++i) dst[i] = *reinterpret_cast<const uint4*>(px[i] + clamp(s) * 128);
  };
  auto store_x = [&](lds_char* slot, const uint4 (&src)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<lds_u32x4*>(slot + wofs[i]) = __builtin_bit_cast(u32x4_t, src[i]);
  };
#pragma unroll
  for (int k = 0; k < NB; ++k)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[k][i] = 0.0f;
  if (len_max <= 0) {   // uniform over the workgroup
    after_prologue();
    return;
  }

  // step s0 goes to slot 0 now; steps s0+1 .. s0+WD wait in xv[(s - s0) % WD]
  Frag2 a[WD];
  uint4 xv[WD][2], x0[2];
  load_x(x0, s0);
#pragma unroll
  for (int j = 0; j < WD; ++j) load_w(a[j], s0 + j);
#pragma unroll
  for (int j = 1; j <= WD; ++j) load_x(xv[j % WD], s0 + j);
  after_prologue();
  store_x(xl, x0);
  __syncthreads();

  const int64_t ngroups = (len_max + U - 1) / U;
  for (int64_t it = 0; it < ngroups; ++it) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t s = s0 + it * U + j;
      __builtin_amdgcn_sched_barrier(0);
      store_x(xl + ((j + 1) & 1) * kSlot, xv[(j + 1) % WD]);   // step s+1
      const lds_char* cur = xl + (j & 1) * kSlot + part * kXBlock;
      Frag2 b[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int t = 16 * k + r;
        b[k].v[0] = __builtin_bit_cast(uint4, *reinterpret_cast<const lds_u32x4*>(cur + xblock_at(t, q)));
        b[k].v[1] = __builtin_bit_cast(uint4, *reinterpret_cast<const lds_u32x4*>(cur + xblock_at(t, q + 4)));
      }
      const int wi = j % WD;
      const uint32_t keep = (s < s1) ? 0xffffffffu : 0u;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        a[wi].v[jj].x &= keep; a[wi].v[jj].y &= keep;
        a[wi].v[jj].z &= keep; a[wi].v[jj].w &= keep;
      }
      const Frag2 aa[1] = {a[wi]};
      mma_step<1, NB>(aa, b, acc);
      __builtin_amdgcn_sched_barrier(0);
      load_w(a[wi], s + WD);
      load_x(xv[(j + 1) % WD], s + 1 + WD);
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

// Folds the KH parts of a workgroup's K range: the part-k waves (k >= 1) add
// their sums into the staged rows of their row group in part order; on return
// stage[wid % 4] holds the full sums and only part-0 waves go on.
template <int KH>
__device__ __forceinline__ bool fold_parts(float (*stage)[16 * kStageLd], const f32x4_t (&acc)[4]) {
  const int wid = threadIdx.x >> 6;
  const int grp = wid & 3, part = wid >> 2;
  if (part == 0) stage_wave_rows(stage[grp], acc);
#pragma unroll
  for (int k = 1; k < KH; ++k) {
    __syncthreads();
    if (part == k) stage_wave_rows<true>(stage[grp], acc);
  }
  if constexpr (KH > 1) __syncthreads();
  return part == 0;
}

// Gate/up for at most 64 tokens, features split over the waves: one
// workgroup (4 KH waves) per 32 features; wave w owns the gate and up rows of
// features 8 (w % 4) .. +8 (one 16-row MFMA block: 8 gate rows, then 8 up
// rows) over part w / 4 of d_model, and the KH parts are folded in LDS.
// With `pos`, the n tokens of the launch are pos[0 .. n) of the n_tokens rows
// of x, h, g, u and row_index (out-of-range positions set the error word and
// are neither read nor written).
template <int WD, int KH, bool PACKED>
__global__ __launch_bounds__(256 * KH) void decode_gateup_kernel(
    int n, const int32_t* __restrict__ pos, int64_t n_tokens, int64_t d, int64_t f,
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg,
    const uint16_t* __restrict__ wu, const uint16_t* __restrict__ rows, int64_t n_rows,
    const int32_t* __restrict__ row_index, uint16_t* __restrict__ h, uint16_t* __restrict__ g_out,
    uint16_t* __restrict__ u_out, int* err) {
  __shared__ __attribute__((aligned(16))) char xs[2 * KH * kXBlock];
  __shared__ float stage[4][16 * kStageLd];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int grp = wid & 3, part = wid >> 2;
  const int r = lane & 15, q = lane >> 4;
  const int64_t f0 = static_cast<int64_t>(blockIdx.x) * 32 + 8 * grp;   // this wave's features
  // PACKED: wg is the packed gate/up block (row block = 8 features)
  const char* pa =
      PACKED ? reinterpret_cast<const char*>(wg) + (static_cast<int64_t>(blockIdx.x) * 4 + grp) * 2048 + lane * 16
             : reinterpret_cast<const char*>(r < 8 ? wg + (f0 + r) * d : wu + (f0 + r - 8) * d) + q * 16;
  const int64_t wstep = PACKED ? (f / 8) * 2048 : 128;
  const int64_t T = d / 64, len = (T + KH - 1) / KH;
  const int64_t s0 = part * len < T ? part * len : T, s1 = s0 + len < T ? s0 + len : T;
  f32x4_t acc[4];
  // the epilogue's table row (lane = token, this wave's 8 features), fetched
  // once the stream is under way
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
  int64_t ri;
  bool erow_ok;
  uint4 erow;
  stream_shared_act<WD, KH, PACKED ? 1024 : 64>(pa, wstep, x, d, act_row, n, (lds_char*)(xs), s0, s1,
                                                 len, acc, [&]() {
    ri = row_index[tok < 0 ? 0 : tok];
    erow_ok = ri >= 0 && ri < n_rows;
    erow = *reinterpret_cast<const uint4*>(erow_ok ? rows + ri * f + f0 : x);
  });

  // epilogue: rows 0-7 (gate) and 8-15 (up) of the row group's block, staged
  // so that lane t holds its token's 8 gate and 8 up sums
  if (!fold_parts<KH>(stage, acc)) return;
  const float* st = stage[grp];
  const int t = lane;
  if (t >= n) return;
  if (tok < 0) {
    flag_index_error(err);
    return;
  }
  float gv[8], uv[8], hv[8], ev[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    gv[e] = st[e * kStageLd + t];
    uv[e] = st[(8 + e) * kStageLd + t];
  }
  if (erow_ok) {
    const uint32_t wds[4] = {erow.x, erow.y, erow.z, erow.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ev[2 * i] = __uint_as_float(wds[i] << 16);
      ev[2 * i + 1] = __uint_as_float(wds[i] & 0xffff0000u);
    }
  } else {
    flag_index_error(err);
#pragma unroll
    for (int i = 0; i < 8; ++i) ev[i] = 0.0f;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uv[e] += ev[e];
    hv[e] = gv[e] * sigmoidf_(gv[e]) * uv[e];
  }
  auto pack = [](const float (&v)[8]) {
    uint4 o;
    o.x = static_cast<uint32_t>(f32_to_bf16(v[0])) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
    o.y = static_cast<uint32_t>(f32_to_bf16(v[2])) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
    o.z = static_cast<uint32_t>(f32_to_bf16(v[4])) | (static_cast<uint32_t>(f32_to_bf16(v[5])) << 16);
    o.w = static_cast<uint32_t>(f32_to_bf16(v[6])) | (static_cast<uint32_t>(f32_to_bf16(v[7])) << 16);
    return o;
  };
  const int64_t o = tok * f + f0;
  *reinterpret_cast<uint4*>(h + o) = pack(hv);
  if (g_out) *reinterpret_cast<uint4*>(g_out + o) = pack(gv);
  if (u_out) *reinterpret_cast<uint4*>(u_out + o) = pack(uv);
}

// Down projection for at most 64 tokens, d_ff split KS ways over workgroups
// and KH ways inside one: workgroup (output block b of 64, split ks) with
// wave w owning outputs 64 b + 16 (w % 4) .. +16 over part w / 4 of the
// split's steps; writes partial[ks][t][n] in fp32.
template <int WD, int KS, int KH, bool PACKED>
__global__ __launch_bounds__(256 * KH) void decode_down_kernel(int n, int64_t d, int64_t f,
                                                               const uint16_t* __restrict__ h,
                                                               const uint16_t* __restrict__ wd,
                                                               float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) char xs[2 * KH * kXBlock];
  __shared__ float stage[4][16 * kStageLd];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int grp = wid & 3, part = wid >> 2;
  const int r = lane & 15, q = lane >> 4;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 64 + 16 * grp;
  const int ks = blockIdx.y;
  const int64_t T = f / 64;
  const int64_t k0 = T * ks / KS, k1 = T * (ks + 1) / KS;
  const int64_t len = (k1 - k0 + KH - 1) / KH;
  const int64_t s0 = k0 + part * len < k1 ? k0 + part * len : k1;
  const int64_t s1 = s0 + len < k1 ? s0 + len : k1;
  // PACKED: wd is the packed down block (row block = 16 outputs)
  const char* pa =
      PACKED ? reinterpret_cast<const char*>(wd) + (static_cast<int64_t>(blockIdx.x) * 4 + grp) * 2048 + lane * 16
             : reinterpret_cast<const char*>(wd + (n0 + r) * f) + q * 16;
  const int64_t wstep = PACKED ? (d / 16) * 2048 : 128;
  f32x4_t acc[4];
  stream_shared_act<WD, KH, PACKED ? 1024 : 64>(pa, wstep, h, f, [](int t) -> int64_t { return t; }, n,
                                                 (lds_char*)(xs), s0, s1, len, acc, []() {});
  if (!fold_parts<KH>(stage, acc)) return;
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
    o.x = static_cast<uint32_t>(f32_to_bf16(s.x)) | (static_cast<uint32_t>(f32_to_bf16(s.y)) << 16);
    o.y = static_cast<uint32_t>(f32_to_bf16(s.z)) | (static_cast<uint32_t>(f32_to_bf16(s.w)) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + i) = o;
  }
}

// Packed weights for the decode kernels: a [R x K] bf16 operand becomes
// K/64 steps of R/16 row blocks, each block two 1 KB loads of 64 lanes x 16
// bytes in the Frag2 pattern: byte ((s * R/16 + rb) * 2 + j) * 1024 + 16 lane
// holds bytes [128 s + 64 j + 16 (lane / 16), +16) of block row lane % 16.
// A gate/up row block is features 8 rb .. 8 rb + 8: its rows 0-7 are those
// rows of W_gate and rows 8-15 those of W_up; a down row block is rows
// 16 rb .. 16 rb + 16 of W_down.  Step-major order over all row blocks puts
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

// Launch shapes of the two decode kernels.
// Launch shapes (measured on MI355X for d_model 2048 / d_ff 8192, batch 64):
// gate/up on 8 waves (d_model in two parts) with two steps in flight per
// wave, down on 4 waves with four steps in flight and d_ff split 8 ways over
// workgroups.
// Deeper prefetch, 2 or 4 steps per barrier, 4 splits, and the earlier
// layouts that split d_model (or d_ff) over the waves of a workgroup and
// folded their partial sums in LDS all measured slower.
constexpr int kGateUpAhead = 2;   // steps in flight per wave
constexpr int kDownAhead = 4;
constexpr int kDownSplit = 8;
constexpr int kGateUpParts = 2;   // d_model split in two inside a gate/up workgroup (8 waves)
constexpr int kDownParts = 1;
static_assert(kDownSplit <= kDownSplitMax, "down partials fit the workspace");

hipError_t decode_pack(int64_t d, int64_t f, const void* wg, const void* wu, const void* wd,
                       void* packed_gu, void* packed_down, hipStream_t s) {
  auto go = [&](int64_t rbs, int64_t k, bool gu, const void* a, const void* b, void* out) {
    const int64_t total = rbs * (k / 64) * 128;
    decode_pack_kernel<<<dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s>>>(
        total, rbs, k, gu, static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b),
        static_cast<uint4*>(out));
  };
  if (packed_gu) go(f / 8, d, true, wg, wu, packed_gu);
  if (packed_down) go(d / 16, f, false, wd, nullptr, packed_down);
  return hipGetLastError();
}

hipError_t decode_gateup(int64_t n, const int32_t* pos, int64_t n_tokens, int64_t d, int64_t f,
                         const void* x, const void* wg, const void* wu, const void* rows,
                         int64_t n_rows, const int32_t* row_index, void* h, void* g_out,
                         void* u_out, hipStream_t s, int* err, bool packed) {
  auto go = [&](auto kern, int threads) {
    kern<<<dim3(static_cast<unsigned>(f / 32)), dim3(threads), 0, s>>>(
        static_cast<int>(n), pos, n_tokens, d, f, static_cast<const uint16_t*>(x),
        static_cast<const uint16_t*>(wg),
        static_cast<const uint16_t*>(wu), static_cast<const uint16_t*>(rows), n_rows, row_index,
        static_cast<uint16_t*>(h), static_cast<uint16_t*>(g_out), static_cast<uint16_t*>(u_out), err);
  };
  if (packed) go(decode_gateup_kernel<kGateUpAhead, kGateUpParts, true>, 256 * kGateUpParts);
  else go(decode_gateup_kernel<kGateUpAhead, kGateUpParts, false>, 256 * kGateUpParts);
  return hipGetLastError();
}

hipError_t decode_down(int64_t n, int64_t d, int64_t f, const void* h, const void* wd, void* y,
                       int out_dtype, void* ws, hipStream_t s, bool packed) {
  float* partial = static_cast<float*>(ws);
  auto go = [&](auto kern) {
    kern<<<dim3(static_cast<unsigned>(d / 64), kDownSplit), dim3(256 * kDownParts), 0, s>>>(
        static_cast<int>(n), d, f, static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(wd),
        partial);
  };
  if (packed) go(decode_down_kernel<kDownAhead, kDownSplit, kDownParts, true>);
  else go(decode_down_kernel<kDownAhead, kDownSplit, kDownParts, false>);
  const int64_t count = n * d;
  const unsigned blocks = static_cast<unsigned>((count / 4 + 255) / 256);
  if (out_dtype == STAPLE_F32)
    decode_down_reduce_kernel<float><<<blocks, 256, 0, s>>>(count, kDownSplit, partial,
                                                            static_cast<float*>(y));
  else
    decode_down_reduce_kernel<uint16_t><<<blocks, 256, 0, s>>>(count, kDownSplit, partial,
                                                               static_cast<uint16_t*>(y));
  return hipGetLastError();
}

}  // namespace staple
