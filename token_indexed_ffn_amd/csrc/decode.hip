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
// B use the same k order, so the contraction is unchanged.  Two steps of
// loads are kept in flight per wave.
//
// Gate/up: one workgroup per 32 features; its four waves split d_model and
// their partial sums meet in LDS, after which the epilogue gathers each
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

// Gate/up for at most 64 tokens: one workgroup (4 waves) per 32 features,
// the waves split d_model, and the wave partial sums are folded in LDS after
// the stream; the epilogue gathers each token's table row, forms
// u = W_up x + E[t] and h = silu(W_gate x) * u and stores h (and g, u when
// asked) with 16-byte vectors.
template <int NS>
__global__ __launch_bounds__(256) void decode_gateup_kernel(
    int n, int64_t d, int64_t f, const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg,
    const uint16_t* __restrict__ wu, const uint16_t* __restrict__ rows, int64_t n_rows,
    const int32_t* __restrict__ row_index, uint16_t* __restrict__ h, uint16_t* __restrict__ g_out,
    uint16_t* __restrict__ u_out, int* err) {
  constexpr int WAVES = 4, NA = 4, NB = 4, NT = NA * NB;
  constexpr int kRing = NT * 4 * 64 * 4;            // bytes of LDS per wave (partials)
  static_assert(kRing >= kXBlock, "activation block fits");
  __shared__ __attribute__((aligned(16))) char smem[WAVES * kRing];
  lds_char* lds = (lds_char*)(smem);
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int64_t f0 = static_cast<int64_t>(blockIdx.x) * 32;
  const int64_t T = d / 64;
  const int slice = (wid + static_cast<int>(blockIdx.x >> 3)) % WAVES;
  const int64_t s0 = T * slice / WAVES, s1 = T * (slice + 1) / WAVES;
  const char* pa[NA] = {reinterpret_cast<const char*>(wg + (f0 + r) * d) + q * 16,
                        reinterpret_cast<const char*>(wg + (f0 + 16 + r) * d) + q * 16,
                        reinterpret_cast<const char*>(wu + (f0 + r) * d) + q * 16,
                        reinterpret_cast<const char*>(wu + (f0 + 16 + r) * d) + q * 16};
  const char* px[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = min(8 * i + (lane >> 3), n - 1);
    px[i] = reinterpret_cast<const char*>(x + static_cast<int64_t>(t) * d) + (lane & 7) * 16;
  }

  // epilogue thread -> (token et, 8 consecutive features); its table row is
  // fetched (branch-free, from a valid address) once the first steps are in
  // flight
  const int et = threadIdx.x >> 2;
  const int efq = (threadIdx.x & 3) * 8;
  bool erow_ok;
  uint4 erow;

  f32x4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[t][i] = 0.0f;
  stream_k_xline<NA, NB, NS>(pa, px, lds + wid * kRing, s0, s1, acc, [&]() {
    const int64_t ri = row_index[min(et, n - 1)];
    erow_ok = ri >= 0 && ri < n_rows;
    const uint16_t* esrc = erow_ok ? rows + ri * f + f0 + efq : x;
    erow = *reinterpret_cast<const uint4*>(esrc);
  });

  // each wave parks its sums in its own LDS block
  float* part = reinterpret_cast<float*>(smem);
  constexpr int kRingF = kRing / 4;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[wid * kRingF + (t * 4 + i) * 64 + lane] = acc[t][i];
  __syncthreads();

  const int t = et;
  const int fq = efq;
  if (t >= n) return;
  float gv[8], av[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int fr = fq + e;
    const int tile_g = (fr >> 4) * NB + (t >> 4);
    const int tile_u = (2 + (fr >> 4)) * NB + (t >> 4);
    const int rr = fr & 15, cc = t & 15;
    const int at = cc + 16 * (rr >> 2), reg = rr & 3;
    float g = 0.0f, a = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      g += part[w * kRingF + (tile_g * 4 + reg) * 64 + at];
      a += part[w * kRingF + (tile_u * 4 + reg) * 64 + at];
    }
    gv[e] = g;
    av[e] = a;
  }
  float ev[8];
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
  uint32_t ph[4], pg[4], pu[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float hv[2], uv[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = 2 * i + k;
      uv[k] = av[e] + ev[e];
      hv[k] = gv[e] * sigmoidf_(gv[e]) * uv[k];
    }
    ph[i] = static_cast<uint32_t>(f32_to_bf16(hv[0])) | (static_cast<uint32_t>(f32_to_bf16(hv[1])) << 16);
    pg[i] = static_cast<uint32_t>(f32_to_bf16(gv[2 * i])) |
            (static_cast<uint32_t>(f32_to_bf16(gv[2 * i + 1])) << 16);
    pu[i] = static_cast<uint32_t>(f32_to_bf16(uv[0])) | (static_cast<uint32_t>(f32_to_bf16(uv[1])) << 16);
  }
  const int64_t o = static_cast<int64_t>(t) * f + f0 + fq;
  *reinterpret_cast<uint4*>(h + o) = make_uint4(ph[0], ph[1], ph[2], ph[3]);
  if (g_out) *reinterpret_cast<uint4*>(g_out + o) = make_uint4(pg[0], pg[1], pg[2], pg[3]);
  if (u_out) *reinterpret_cast<uint4*>(u_out + o) = make_uint4(pu[0], pu[1], pu[2], pu[3]);
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
struct DecodeConfig {
  int gu_slots;   // steps in flight per wave in the gate/up kernel (2 or 3)
  int dn_shape;   // down kernel shape: 1 (32 outputs, 4 splits), 2 (64, 8), 3 (64, 4), 4 (128, 8)
};
// Measured best on MI355X for d_model 2048 / d_ff 8192, batch 64.
static DecodeConfig g_decode_cfg = {2, 2};

void decode_set_config(int gu_slots, int dn_shape) { g_decode_cfg = {gu_slots, dn_shape}; }

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
  if (g_decode_cfg.gu_slots >= 3) go(decode_gateup_kernel<3>);
  else go(decode_gateup_kernel<2>);
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
