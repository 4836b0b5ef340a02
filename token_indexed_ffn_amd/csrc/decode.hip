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

__device__ __forceinline__ void load_step(Frag2& f, const char* p, int64_t off) {
  f.v[0] = *reinterpret_cast<const uint4*>(p + off);
  f.v[1] = *reinterpret_cast<const uint4*>(p + off + 64);
}

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

// Position in the LDS partials of output (row-block a, token tile b, row
// rr in 0..15, token column cc in 0..15) for `wave`, with NT = NA * NB tiles.
template <int NT>
__device__ __forceinline__ int part_at(int wave, int tile, int rr, int cc) {
  const int lane = cc + 16 * (rr >> 2);
  const int reg = rr & 3;
  return ((wave * NT + tile) * 4 + reg) * 64 + lane;
}

template <int NT>
__device__ __forceinline__ void store_partials(float* part, int slot, const f32x4_t (&acc)[NT]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[((slot * NT + t) * 4 + i) * 64 + lane] = acc[t][i];
}

template <int NT>
__device__ __forceinline__ void add_partials(const float* part, int slot, f32x4_t (&acc)[NT]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[t][i] += part[((slot * NT + t) * 4 + i) * 64 + lane];
}

typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;

// The activation block of one macro step in LDS: 64 tokens x 128 bytes, token
// t's 16-byte chunk c at t * 128 + ((c ^ ((t >> 1) & 7)) << 4).  It is loaded
// from global memory with eight 1 KB instructions that each cover 8 whole
// tokens x 128 bytes (full cache lines, lane l: token 8i + l / 8, chunk
// l % 8), written to the wave's LDS block and read back in the Frag2 pattern;
// the XOR keeps every 16-lane group of both the writes and the reads on
// distinct banks.
constexpr int kXBlock = 64 * 128;

__device__ __forceinline__ int xblock_at(int t, int c) { return t * 128 + ((c ^ ((t >> 1) & 7)) << 4); }

// Streams macro steps [s0, s1) of NA weight row-blocks (16 rows each, pa[i]
// the lane's bytes at step 0) and the activation of NB token tiles through NS
// register slots: the loads of NS steps are in flight while one step's MFMAs
// run.  The activation is loaded as full cache lines (px[i]: the 16 bytes of
// the lane's i-th load at step 0) and rearranged into MFMA fragments through
// the wave's own LDS block (kXBlock bytes at `xlds`).  Scheduling barriers
// keep each refill where it is written (otherwise the compiler sinks the
// loads next to their use); steps past s1 in the last group read the last
// step again and their weights are masked to zero, and the last group issues
// no refills.  `after_prologue` runs once the first NS steps are in flight.
template <int NA, int NB, int NS, typename Hook>
__device__ __forceinline__ void stream_k_xline(const char* const (&pa)[NA], const char* const (&px)[8],
                                               lds_char* xlds, int64_t s0, int64_t s1,
                                               f32x4_t (&acc)[NA * NB], Hook&& after_prologue) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const int64_t ngroups = (s1 - s0 + NS - 1) / NS;
  if (ngroups <= 0) {
    after_prologue();
    return;
  }
  auto off = [&](int64_t s) -> int64_t { return (s < s1 ? s : s1 - 1) * 128; };
  Frag2 a[NS][NA];
  uint4 xv[NS][8];
  int wofs[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) wofs[i] = xblock_at(8 * i + (lane >> 3), lane & 7);
  auto issue = [&](int j, int64_t s) {
#pragma unroll
    for (int i = 0; i < NA; ++i) load_step(a[j][i], pa[i], off(s));
#pragma unroll
    for (int i = 0; i < 8; ++i) xv[j][i] = *reinterpret_cast<const uint4*>(px[i] + off(s));
  };
  auto consume = [&](int j, int64_t s) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<lds_u32x4*>(xlds + wofs[i]) = __builtin_bit_cast(u32x4_t, xv[j][i]);
    Frag2 b[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int t = 16 * k + r;
      b[k].v[0] = __builtin_bit_cast(uint4, *reinterpret_cast<const lds_u32x4*>(xlds + xblock_at(t, q)));
      b[k].v[1] = __builtin_bit_cast(uint4, *reinterpret_cast<const lds_u32x4*>(xlds + xblock_at(t, q + 4)));
    }
    const uint32_t keep = (s < s1) ? 0xffffffffu : 0u;
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        a[j][i].v[jj].x &= keep; a[j][i].v[jj].y &= keep;
        a[j][i].v[jj].z &= keep; a[j][i].v[jj].w &= keep;
      }
    mma_step<NA, NB>(a[j], b, acc);
  };
#pragma unroll
  for (int j = 0; j < NS; ++j) issue(j, s0 + j);
  after_prologue();
  for (int64_t it = 0; it + 1 < ngroups; ++it) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int64_t s = s0 + it * NS + j;
      __builtin_amdgcn_sched_barrier(0);
      consume(j, s);
      __builtin_amdgcn_sched_barrier(0);
      issue(j, s + NS);
    }
  }
  // last group: nothing more to load
  const int64_t sl = s0 + (ngroups - 1) * NS;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    __builtin_amdgcn_sched_barrier(0);
    consume(j, sl + j);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Gate/up for at most 64 tokens, features split over the waves: one
// workgroup (4 waves) per 32 features; wave w owns gate and up rows of
// features 8w .. 8w+7 (one 16-row MFMA block: 8 gate rows, then 8 up rows)
// over the whole of d_model, so no partial sums cross waves.  The activation
// of SPB macro steps (64 tokens x 128 bytes each) is loaded once per
// workgroup as whole cache lines (two 1 KB loads per wave and step), written
// to one of two LDS slots and read by all four waves; one barrier per SPB
// steps hands a slot over.  Weights and activations are loaded WD steps ahead
// (8 + 8 registers per step): loads complete in issue order, so waiting for
// a step's activation also waits for every weight load issued before it.
template <int WD, int SPB>
__global__ __launch_bounds__(256) void decode_gateup_fs_kernel(
    int n, int64_t d, int64_t f, const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg,
    const uint16_t* __restrict__ wu, const uint16_t* __restrict__ rows, int64_t n_rows,
    const int32_t* __restrict__ row_index, uint16_t* __restrict__ h, uint16_t* __restrict__ g_out,
    uint16_t* __restrict__ u_out, int* err) {
  constexpr int NB = 4;
  constexpr int XS = WD / SPB;                          // slots of activation registers (super-steps)
  constexpr int U = XS % 2 == 0 ? XS : 2 * XS;          // unrolled super-steps (even: LDS slot parity)
  static_assert(WD % SPB == 0 && XS >= 1, "prefetch depth in whole super-steps");
  constexpr int kSlot = SPB * kXBlock;
  constexpr int kEpiLd = 65;                            // floats per staged row
  __shared__ __attribute__((aligned(16))) char xs[2 * kSlot];
  __shared__ float stage[4][16 * kEpiLd];
  lds_char* xl = (lds_char*)(xs);
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int64_t f0 = static_cast<int64_t>(blockIdx.x) * 32 + 8 * wid;   // this wave's features
  const int64_t T = d / 64;
  const char* pa = reinterpret_cast<const char*>(r < 8 ? wg + (f0 + r) * d : wu + (f0 + r - 8) * d) + q * 16;
  // activation loads of this wave: tokens 16 wid + l / 8 and 16 wid + 8 + l / 8, chunk l % 8
  const char* px[2];
  int wofs[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int tt = 16 * wid + 8 * i + (lane >> 3);
    px[i] = reinterpret_cast<const char*>(x + static_cast<int64_t>(min(tt, n - 1)) * d) + (lane & 7) * 16;
    wofs[i] = xblock_at(tt, lane & 7);
  }
  auto off = [&](int64_t s) -> int64_t { return (s < T ? s : T - 1) * 128; };

  Frag2 a[WD];
  uint4 xv[XS][SPB][2];
  f32x4_t acc[NB];
#pragma unroll
  for (int k = 0; k < NB; ++k)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[k][i] = 0.0f;
  auto load_x = [&](uint4 (&dst)[SPB][2], int64_t super) {
#pragma unroll
    for (int sb = 0; sb < SPB; ++sb)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        dst[sb][i] = *reinterpret_cast<const uint4*>(px[i] + off(super * SPB + sb));
  };
  auto store_x = [&](lds_char* slot, const uint4 (&src)[SPB][2]) {
#pragma unroll
    for (int sb = 0; sb < SPB; ++sb)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        *reinterpret_cast<lds_u32x4*>(slot + sb * kXBlock + wofs[i]) = __builtin_bit_cast(u32x4_t, src[sb][i]);
  };

  // super-step 0 goes to slot 0 now; super-steps 1 .. XS wait in xv[S % XS]
  uint4 x0[SPB][2];
  load_x(x0, 0);
#pragma unroll
  for (int j = 0; j < WD; ++j) load_step(a[j], pa, off(j));
#pragma unroll
  for (int j = 1; j <= XS; ++j) load_x(xv[j % XS], j);
  // the epilogue's table row (lane = token, this wave's 8 features)
  const int64_t ri = row_index[min(lane, n - 1)];
  const bool erow_ok = ri >= 0 && ri < n_rows;
  const uint4 erow = *reinterpret_cast<const uint4*>(erow_ok ? rows + ri * f + f0 : x);
  store_x(xl, x0);
  __syncthreads();

  const int64_t nsuper = (T + SPB - 1) / SPB;
  const int64_t ngroups = (nsuper + U - 1) / U;
  for (int64_t it = 0; it < ngroups; ++it) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t S = it * U + j;
      __builtin_amdgcn_sched_barrier(0);
      store_x(xl + ((j + 1) & 1) * kSlot, xv[(j + 1) % XS]);   // super-step S+1
      const lds_char* cur = xl + (j & 1) * kSlot;
#pragma unroll
      for (int sb = 0; sb < SPB; ++sb) {
        const int64_t s = S * SPB + sb;
        const int wi = (j * SPB + sb) % WD;
        Frag2 b[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
          const int t = 16 * k + r;
          b[k].v[0] = __builtin_bit_cast(uint4, *reinterpret_cast<const lds_u32x4*>(cur + sb * kXBlock + xblock_at(t, q)));
          b[k].v[1] = __builtin_bit_cast(uint4, *reinterpret_cast<const lds_u32x4*>(cur + sb * kXBlock + xblock_at(t, q + 4)));
        }
        const uint32_t keep = (s < T) ? 0xffffffffu : 0u;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          a[wi].v[jj].x &= keep; a[wi].v[jj].y &= keep;
          a[wi].v[jj].z &= keep; a[wi].v[jj].w &= keep;
        }
        const Frag2 aa[1] = {a[wi]};
        mma_step<1, NB>(aa, b, acc);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int sb = 0; sb < SPB; ++sb) {
        const int64_t s = S * SPB + sb;
        load_step(a[(j * SPB + sb) % WD], pa, off(s + WD));
      }
      load_x(xv[(j + 1) % XS], S + 1 + XS);
      lds_barrier();
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // epilogue: rows 0-7 (gate) and 8-15 (up) of this wave's block, staged so
  // that lane t holds its token's 8 gate and 8 up sums
  float* st = stage[wid];
#pragma unroll
  for (int k = 0; k < NB; ++k)
#pragma unroll
    for (int i = 0; i < 4; ++i) st[(4 * q + i) * kEpiLd + 16 * k + r] = acc[k][i];
  __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4));   // lgkmcnt(0): own stores visible to own reads
  const int t = lane;
  if (t >= n) return;
  float gv[8], uv[8], hv[8], ev[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    gv[e] = st[e * kEpiLd + t];
    uv[e] = st[(8 + e) * kEpiLd + t];
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
  const int64_t o = static_cast<int64_t>(t) * f + f0;
  *reinterpret_cast<uint4*>(h + o) = pack(hv);
  if (g_out) *reinterpret_cast<uint4*>(g_out + o) = pack(gv);
  if (u_out) *reinterpret_cast<uint4*>(u_out + o) = pack(uv);
}

// Partial y over one K split: partial[ks][t][n0 + c] (fp32) for the 16*NA
// outputs n0.. of this workgroup and split ks of KS.  (Summing the splits in
// the last workgroup to finish, behind an arrival counter, measured slower on
// MI355X than the separate reduction kernel: publishing the partials across
// XCDs costs an L2 writeback or uncached accesses per workgroup.)
template <int WAVES, int NS, int NA, int KS>
__global__ __launch_bounds__(64 * WAVES) void decode_down_partial_kernel(
    int n, int64_t d, int64_t f, const uint16_t* __restrict__ h, const uint16_t* __restrict__ wd,
    float* __restrict__ partial) {
  constexpr int NB = 4, NT = NA * NB, F = 16 * NA, FPT = F / 4;
  static_assert(NT * 4 * 64 * 4 >= kXBlock, "activation block fits in the wave's partials");
  __shared__ __attribute__((aligned(16))) float part[WAVES * NT * 4 * 64];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * F;
  const int ks = blockIdx.y;
  const int64_t T = f / 64;
  const int64_t gw = (static_cast<int64_t>(ks) * WAVES + wid + (blockIdx.x >> 3)) % (WAVES * KS);
  const int64_t s0 = T * gw / (WAVES * KS), s1 = T * (gw + 1) / (WAVES * KS);
  const char* pa[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i)
    pa[i] = reinterpret_cast<const char*>(wd + (n0 + 16 * i + r) * f) + q * 16;
  const char* px[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = min(8 * i + (lane >> 3), n - 1);
    px[i] = reinterpret_cast<const char*>(h + static_cast<int64_t>(t) * f) + (lane & 7) * 16;
  }

  f32x4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[t][i] = 0.0f;
  lds_char* xlds = (lds_char*)(reinterpret_cast<char*>(part) + wid * NT * 4 * 64 * 4);
  stream_k_xline<NA, NB, NS>(pa, px, xlds, s0, s1, acc, []() {});

  store_partials<NT>(part, wid, acc);
  __syncthreads();
  const int t = threadIdx.x >> 2;
  const int fq = (threadIdx.x & 3) * FPT;
  if (threadIdx.x < 256 && t < n) {
    float* dst = partial + (static_cast<int64_t>(ks) * n + t) * d + n0 + fq;
#pragma unroll
    for (int e0 = 0; e0 < FPT; e0 += 4) {
      float out[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int fr = fq + e0 + e;
        const int tile = (fr >> 4) * NB + (t >> 4);
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) sum += part[part_at<NT>(w, tile, fr & 15, t & 15)];
        out[e] = sum;
      }
      *reinterpret_cast<float4*>(dst + e0) = make_float4(out[0], out[1], out[2], out[3]);
    }
  }
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

bool decode_eligible(int64_t n, int64_t d, int64_t f, int dtype) {
  return dtype == STAPLE_BF16 && n >= 1 && n <= kDecMaxTokens && d % 64 == 0 && f % 64 == 0;
}

size_t decode_down_workspace_bytes(int64_t n, int64_t d) {
  return static_cast<size_t>(kDownSplitMax) * n * d * sizeof(float);
}

// Launch shapes of the two decode kernels.
// (gate/up: deeper prefetch, 2 or 4 steps per barrier and the earlier
// d_model split over the waves with a partial-sum fold all measured slower.)
struct DecodeConfig {
  int dn_shape;   // down kernel shape: 1 (32 outputs, 4 splits), 2 (64, 8), 3 (64, 4), 4 (128, 8)
};
// Measured best on MI355X for d_model 2048 / d_ff 8192, batch 64.
static DecodeConfig g_decode_cfg = {2};

void decode_set_config(int dn_shape) { g_decode_cfg = {dn_shape}; }

hipError_t decode_gateup(int64_t n, int64_t d, int64_t f, const void* x, const void* wg,
                         const void* wu, const void* rows, int64_t n_rows,
                         const int32_t* row_index, void* h, void* g_out, void* u_out,
                         hipStream_t s, int* err) {
  auto go = [&](auto kern) {
    kern<<<dim3(static_cast<unsigned>(f / 32)), dim3(256), 0, s>>>(
        static_cast<int>(n), d, f, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wg),
        static_cast<const uint16_t*>(wu), static_cast<const uint16_t*>(rows), n_rows, row_index,
        static_cast<uint16_t*>(h), static_cast<uint16_t*>(g_out), static_cast<uint16_t*>(u_out), err);
  };
  go(decode_gateup_fs_kernel<4, 1>);
  return hipGetLastError();
}

template <int NA, int KS>
static void launch_dn(int64_t n, int64_t d, int64_t f, const void* h, const void* wd, float* partial,
                      hipStream_t s) {
  decode_down_partial_kernel<4, 2, NA, KS><<<dim3(static_cast<unsigned>(d / (16 * NA)), KS),
                                             dim3(256), 0, s>>>(
      static_cast<int>(n), d, f, static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(wd),
      partial);
}

hipError_t decode_down(int64_t n, int64_t d, int64_t f, const void* h, const void* wd, void* y,
                       int out_dtype, void* ws, hipStream_t s) {
  float* partial = static_cast<float*>(ws);
  int ks = 8;
  switch (g_decode_cfg.dn_shape) {
    case 1: launch_dn<2, 4>(n, d, f, h, wd, partial, s); ks = 4; break;
    case 3: launch_dn<4, 4>(n, d, f, h, wd, partial, s); ks = 4; break;
    case 4: launch_dn<8, 8>(n, d, f, h, wd, partial, s); ks = 8; break;
    default: launch_dn<4, 8>(n, d, f, h, wd, partial, s); ks = 8; break;
  }
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
