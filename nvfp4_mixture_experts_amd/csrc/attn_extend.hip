// attn_extend.hip -- extend attention over a quantised KV cache on gfx950: new query
// tokens attend to a cached prefix (16-bit, fp8 or NVFP4) and, causally, to the new
// tokens themselves, with an optional sliding window.
//
// FreeToken fork PR #84 (page 1), the bullet on the extend-attention kernel of the
// NVFP4 KV-cache step: the cache loops of the extend kernel need a quantised twin of
// their tile (the per-tensor fp8 scales go on the dot outputs, and the softmax
// normaliser sums the unscaled probabilities), while the loops over the new tokens
// stay 16-bit.  That is the structure here: one templated tile over a chunk of 64
// keys, run on the cache in its format and on the new tokens in bf16.
//
// A block of 4 waves takes 64 query rows of one kv head: row r is (token, head of the
// kv head's group) number 64 b + r in token-major order, so the query heads that
// share a kv head share every staged key and value.  Chunks alternate between two LDS
// buffers: chunk j + 1 is staged between chunk j's P V products.  Per chunk of 64 keys:
//   1. the chunk's keys and values are turned into bf16 in LDS (exact for every
//      format: an e4m3 value, or an e2m1 code times its e4m3 block scale, has at most
//      6 significant bits), keys as rows [key][dim], values transposed [dim][key];
//   2. S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (each wave 64 keys x its 16 rows, Q in
//      registers), times the key tensor scale and 1/sqrt(d) on the dot outputs, keys
//      outside a row's causal / window range masked.  In the result's layout a lane
//      holds 16 scores of ONE query row (keys 16 c + 4 (lane / 16) + r), which is the
//      operand layout of P^T for v_mfma_f32_16x16x16_bf16: P never leaves registers;
//   3. online softmax per row in fp32 (base-2 exponentials, the row spread over 4
//      lanes), relative to a reference max that moves only when a chunk exceeds it
//      by more than 2^8 (O and l are rescaled then, and only then); the normaliser
//      sums the unscaled probabilities; P times the value tensor scale as a bf16 pair
//      (hi = bf16(p), lo = bf16(p - hi): about 16 significant bits; one bf16 alone
//      costs the output about 2e-3 of relative L2);
//   4. O^T += V^T P^T on v_mfma_f32_16x16x16_bf16 (each wave d x 16 rows; the hi and
//      lo products into the same accumulator).
// At the end O / l is rounded to bf16.
#include "ftmoe_device.hpp"
#include "ftmoe_kernels.hpp"

namespace ftmoe {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 at_bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float at_f32x4;
typedef unsigned int at_u32x4 __attribute__((ext_vector_type(4)));
typedef short at_s16x4 __attribute__((ext_vector_type(4)));
typedef float at_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 at_bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kAttnWaves = 4;
constexpr int kAttnRows = 16 * kAttnWaves;  // query rows per block
constexpr int kChunk = 64;                  // keys per chunk
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct AttnLds {
  uint16_t k[kChunk][D + 16];            // keys of the chunk, bf16 (16 of padding)
  uint16_t vt[D][kChunk + 4];            // values transposed, bf16 (4 of padding)
};

__device__ __forceinline__ at_f32x4 mfma(at_u32x4 a, at_u32x4 b, at_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(at_bf16x8, a),
                                                 __builtin_bit_cast(at_bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ at_f32x4 mfma16(uint2 a, uint2 b, at_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(at_s16x4, a),
                                                   __builtin_bit_cast(at_s16x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pk(bf16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// max and sum of v over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the 16-lane rows of a
// wave), in registers: v_permlane16_swap with one register as both operands yields the
// values of lanes l and l ^ 16, v_permlane32_swap those of l and l ^ 32, in the same
// order on both lanes of a pair (so both get the same bits)
__device__ __forceinline__ float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Staging of keys [c0, c0 + 64) of one source into LDS, in two halves: fetch_chunk
// issues the global loads (into registers, so that the next chunk's loads travel
// while this chunk is multiplied) and store_chunk turns them into bf16 in LDS.  Rows
// past `end` repeat the source's last row of the range (finite values whose scores
// are masked).  Item w = tid + 256 j is key pair kp = w % 32 (keys 2 kp, 2 kp + 1) and
// dim group part = w / 32 (dims 8 part .. + 7): the 32 lanes of one dim group write
// the transposed values of 32 consecutive key pairs, 32 consecutive LDS words.
template <int D>
struct ChunkRaw {
  static constexpr int kItems = (kChunk / 2) * (D / 8) / (kAttnWaves * kWave);
  at_u32x4 k[kItems][2], v[kItems][2];  // FMT 0: 8 bf16; 1: 8 e4m3 in x, y; 2: codes x, scale y
};

template <int D, int FMT>
__device__ __forceinline__ at_u32x4 fetch8(const void* src, const uint8_t* bscale, size_t row,
                                           int part) {
  at_u32x4 r = {0u, 0u, 0u, 0u};
  if constexpr (FMT == 0) {
    r = *reinterpret_cast<const at_u32x4*>(static_cast<const uint16_t*>(src) + row * D + 8 * part);
  } else if constexpr (FMT == 1) {
    const uint2 a = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(src) + row * D + 8 * part);
    r.x = a.x;
    r.y = a.y;
  } else {
    r.x = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(src) + row * (D / 2) + 4 * part);
    r.y = bscale[row * (D / 16) + part / 2];
  }
  return r;
}

// Eight elements as bf16, exactly (an e4m3 value, or an e2m1 code times its e4m3
// block scale, has at most 6 significant bits).
template <int FMT>
__device__ __forceinline__ at_u32x4 widen8(at_u32x4 r) {
  if constexpr (FMT == 0) {
    return r;
  } else if constexpr (FMT == 1) {
    return at_u32x4{pk(e4m3x2_to_bf16<false>(r.x)), pk(e4m3x2_to_bf16<true>(r.x)),
                    pk(e4m3x2_to_bf16<false>(r.y)), pk(e4m3x2_to_bf16<true>(r.y))};
  } else {
    const uint4 v = dequant8_bf16(r.x, e4m3_to_f32(r.y));
    return at_u32x4{v.x, v.y, v.z, v.w};
  }
}

template <int D, int FMT>
__device__ __forceinline__ void fetch_chunk(ChunkRaw<D>& raw, const void* kc, const void* vc,
                                            const uint8_t* kbs, const uint8_t* vbs, int c0,
                                            int first, int end, int Hkv, int kh) {
#pragma unroll
  for (int j = 0; j < ChunkRaw<D>::kItems; ++j) {
    const int w = threadIdx.x + kAttnWaves * kWave * j;
    const int kp = w & 31, part = w >> 5;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int key = c0 + 2 * kp + e;
      const size_t row = static_cast<size_t>((key < end ? key : end - 1) - first) * Hkv + kh;
      raw.k[j][e] = fetch8<D, FMT>(kc, kbs, row, part);
      raw.v[j][e] = fetch8<D, FMT>(vc, vbs, row, part);
    }
  }
}

template <int D, int FMT>
__device__ __forceinline__ void store_chunk(AttnLds<D>& lds, const ChunkRaw<D>& raw) {
#pragma unroll
  for (int j = 0; j < ChunkRaw<D>::kItems; ++j) {
    const int w = threadIdx.x + kAttnWaves * kWave * j;
    const int kp = w & 31, part = w >> 5;
    at_u32x4 vv[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      *reinterpret_cast<at_u32x4*>(&lds.k[2 * kp + e][8 * part]) = widen8<FMT>(raw.k[j][e]);
      vv[e] = widen8<FMT>(raw.v[j][e]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // dims 8 part + 2 q (low halves) and + 1 (high halves)
      const uint32_t a = vv[0][q], b = vv[1][q];
      *reinterpret_cast<uint32_t*>(&lds.vt[8 * part + 2 * q][2 * kp]) = (a & 0xFFFFu) | (b << 16);
      *reinterpret_cast<uint32_t*>(&lds.vt[8 * part + 2 * q + 1][2 * kp]) = (a >> 16) | (b & 0xFFFF0000u);
    }
  }
}

template <int D>
struct RowState {
  float m, l;             // reference max (base 2, -inf before any visible key) of the lane's
                          // query row, and its normaliser relative to that reference
  at_f32x4 o[D / 16];     // O^T fragments: dims 16 f + 4 (lane / 16) + r of that row
  int lo, hi;             // visible key positions [lo, hi] of the row
  int all_lo, all_hi;     // keys in [all_lo, all_hi] are visible to every row of the block
};

// O and l stay relative to a row's reference max until a chunk's max exceeds it by
// more than this (base 2): probabilities are then at most 2^8, and most chunks need
// no rescaling of O at all.
constexpr float kRescaleSlack = 8.0f;

// One chunk [c0, end) (end - c0 <= 64) of one source against the wave's 16 rows.
// kscale2 = key tensor scale x 1/sqrt(d) x log2(e) (> 0); lvs = log2 of the value
// tensor scale (added to the exponent, so P comes out multiplied by the scale) and
// ivs its reciprocal (the normaliser sums the unscaled probabilities).
template <int D, int FMT, class Stage>
__device__ __forceinline__ void chunk_step(AttnLds<D>& lds, const at_u32x4 (&qf)[D / 32], int c0,
                                           int end, float kscale2, float lvs, float ivs,
                                           RowState<D>& st, Stage&& stage) {
  const int lane = threadIdx.x & (kWave - 1);
  const int i = lane & 15, g = lane >> 4;
  // S^T = K Q^T: key fragments c of 16; lane: keys 16 c + 4 g + r of query row i
  at_f32x4 s[4];
  {
    at_u32x4 kf[4][D / 32];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        kf[c][ks] = *reinterpret_cast<const at_u32x4*>(&lds.k[16 * c + i][32 * ks + 8 * g]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < 4; ++c) s[c] = at_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
      for (int c = 0; c < 4; ++c) s[c] = mfma(kf[c][ks], qf[ks], s[c]);
  }
  // the values' fragments travel while the softmax runs
  uint2 vf[D / 16][4];
#pragma unroll
  for (int f = 0; f < D / 16; ++f)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      vf[f][c] = *reinterpret_cast<const uint2*>(&lds.vt[16 * f + i][16 * c + 4 * g]);
  __builtin_amdgcn_sched_barrier(0);
  // a whole chunk inside every row's visible range needs no mask (most cache chunks);
  // the test is the same for the whole block
  const bool whole = end - c0 == kChunk && c0 >= st.all_lo && end - 1 <= st.all_hi;
  if (!whole) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kpos = c0 + 16 * c + 4 * g + r;
        const bool vis = (kpos < end) & (kpos >= st.lo) & (kpos <= st.hi);
        s[c][r] = vis ? s[c][r] : -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[c][r]);
  mx = rows_max(mx);
  mx *= kscale2;  // the chunk's max of the row's scaled scores (scaling by kscale2 > 0 keeps order)
  // first visible key (reference -inf), or the max moved past the slack: new reference
  const bool grow = mx > st.m + kRescaleSlack;
  if (__ballot(grow) != 0) {
    const float alpha = grow ? __builtin_amdgcn_exp2f(st.m - mx) : 1.0f;  // 0 from -inf: O, l are 0
#pragma unroll
    for (int f = 0; f < D / 16; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) st.o[f][r] *= alpha;
    st.l *= alpha;
    st.m = grow ? mx : st.m;
  }
  // a row with no visible key so far has only -inf scores: any finite reference gives 0
  const float bias = (st.m == -INFINITY ? 0.0f : -st.m) + lvs;
  float sum = 0.0f;
  uint2 ph[4], pl[4];  // P^T operands: keys 16 c + 4 g .. + 3, bf16 hi and lo
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint32_t hw[2], lw[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {  // two probabilities per packed conversion (nearest-even)
      at_f32x2 pv;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        pv[e] = __builtin_amdgcn_exp2f(fmaf(s[c][2 * q + e], kscale2, bias));
        sum += pv[e];
      }
      const at_bf16x2 h = __builtin_convertvector(pv, at_bf16x2);
      const at_bf16x2 l = __builtin_convertvector(pv - __builtin_convertvector(h, at_f32x2), at_bf16x2);
      hw[q] = __builtin_bit_cast(uint32_t, h);
      lw[q] = __builtin_bit_cast(uint32_t, l);
    }
    ph[c] = make_uint2(hw[0], hw[1]);
    pl[c] = make_uint2(lw[0], lw[1]);
  }
  sum = rows_sum(sum);
  st.l += sum * ivs;
  // O^T += V^T P^T (V^T operand: dims 16 f + i, keys 16 c + 4 g .. + 3)
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int f = 0; f < D / 16; ++f) st.o[f] = mfma16(vf[f][c], ph[c], st.o[f]);
  stage();  // vector work that runs while the matrix cores take the products above
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int f = 0; f < D / 16; ++f) st.o[f] = mfma16(vf[f][c], pl[c], st.o[f]);
}

// Keys [k0, k1) of one source (the cache in format FMT, or the new tokens in bf16;
// `first` = the position of the source's row 0), 64 at a time, each chunk's loads
// issued while the previous chunk is multiplied.
template <int D, int FMT>
__device__ __forceinline__ void attend_range(AttnLds<D> (&lds)[2], const at_u32x4 (&qf)[D / 32],
                                             const void* kc, const void* vc, const uint8_t* kbs,
                                             const uint8_t* vbs, int first, int k0, int k1,
                                             int Hkv, int kh, float kscale2, float lvs,
                                             float ivs, RowState<D>& st) {
  if (k0 >= k1) return;
  auto chunk_end = [&](int c) { return c + kChunk < k1 ? c + kChunk : k1; };
  ChunkRaw<D> raw;
  fetch_chunk<D, FMT>(raw, kc, vc, kbs, vbs, k0, first, chunk_end(k0), Hkv, kh);
  // both buffers are free: every chunk step ends with a barrier
  store_chunk<D, FMT>(lds[0], raw);
  if (k0 + kChunk < k1) fetch_chunk<D, FMT>(raw, kc, vc, kbs, vbs, k0 + kChunk, first, chunk_end(k0 + kChunk), Hkv, kh);
  __syncthreads();
  int buf = 0;
  for (int c0 = k0; c0 < k1; c0 += kChunk) {
    const int n1 = c0 + kChunk, n2 = c0 + 2 * kChunk;
    // the next chunk goes to the other buffer (last read by the previous chunk, before
    // the previous barrier), between this chunk's P V products
    chunk_step<D, FMT>(lds[buf], qf, c0, chunk_end(c0), kscale2, lvs, ivs, st, [&]() {
      if (n1 < k1) {
        store_chunk<D, FMT>(lds[buf ^ 1], raw);
        if (n2 < k1) fetch_chunk<D, FMT>(raw, kc, vc, kbs, vbs, n2, first, chunk_end(n2), Hkv, kh);
      }
    });
    __syncthreads();
    buf ^= 1;
  }
}

template <int D, int FMT>
__global__ __launch_bounds__(kAttnWaves* kWave) void attn_extend_kernel(AttnParams p) {
  __shared__ AttnLds<D> lds[2];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int kh = blockIdx.y;
  const int G = p.Hq / p.Hkv;
  const int nrows = p.n_new * G;
  const int r0 = blockIdx.x * kAttnRows;  // first (token, head) row of the block
  auto token_of = [&](int r) { return (r < nrows ? r : nrows - 1) / G; };
  auto lo_of = [&](int t) {
    const int qpos = p.prefix + t;
    return p.window > 0 ? (qpos - p.window + 1 > 0 ? qpos - p.window + 1 : 0) : 0;
  };
  // this lane's query row: 16 wave + i (its row of the Q operand and of S^T, O^T)
  RowState<D> st;
  {
    const int t = token_of(r0 + 16 * wave + i);
    st.m = -INFINITY;
    st.l = 0.0f;
    st.lo = lo_of(t);
    st.hi = p.prefix + t;
  }
#pragma unroll
  for (int f = 0; f < D / 16; ++f) st.o[f] = at_f32x4{0.f, 0.f, 0.f, 0.f};
  at_u32x4 qf[D / 32];
  {
    const int rq = r0 + 16 * wave + i;
    const int rc = rq < nrows ? rq : nrows - 1;
    const int t = rc / G, h = kh * G + rc % G;
    const uint16_t* qrow = p.q + (static_cast<size_t>(t) * p.Hq + h) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) qf[ks] = *reinterpret_cast<const at_u32x4*>(qrow + 32 * ks + 8 * g);
  }
  // keys the block's rows can see: [lo of its first token, position of its last]
  const int t_first = token_of(r0), t_last = token_of(r0 + kAttnRows - 1);
  const int klo = lo_of(t_first), khi = p.prefix + t_last + 1;
  st.all_lo = lo_of(t_last);          // lo grows with the token
  st.all_hi = p.prefix + t_first;
  const float s2 = p.sm_scale * kLog2e;
  if (klo < p.prefix) {
    const float vs = FMT == 0 ? 1.0f : p.v_scale;
    attend_range<D, FMT>(lds, qf, p.k_cache, p.v_cache, p.k_bscale, p.v_bscale, 0, klo,
                         p.prefix < khi ? p.prefix : khi, p.Hkv, kh,
                         (FMT == 0 ? 1.0f : p.k_scale) * s2, __log2f(vs), 1.0f / vs, st);
  }
  const int n0 = klo > p.prefix ? klo : p.prefix;
  attend_range<D, 0>(lds, qf, p.k_new, p.v_new, nullptr, nullptr, p.prefix, n0, khi, p.Hkv, kh, s2,
                     0.0f, 1.0f, st);
  // O / l (every row sees its own position, so l > 0); lane: dims 16 f + 4 g .. + 3
  const int row = r0 + 16 * wave + i;
  if (row < nrows) {
    const int t = row / G, h = kh * G + row % G;
    uint16_t* orow = p.out + (static_cast<size_t>(t) * p.Hq + h) * D;
    const float inv = 1.0f / st.l;
#pragma unroll
    for (int f = 0; f < D / 16; ++f) {
      const uint32_t b0 = f32_to_bf16_bits(st.o[f][0] * inv), b1 = f32_to_bf16_bits(st.o[f][1] * inv);
      const uint32_t b2 = f32_to_bf16_bits(st.o[f][2] * inv), b3 = f32_to_bf16_bits(st.o[f][3] * inv);
      *reinterpret_cast<uint2*>(orow + 16 * f + 4 * g) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
    }
  }
}

template <int D>
hipError_t launch_d(const AttnParams& p, hipStream_t s) {
  const int nrows = p.n_new * (p.Hq / p.Hkv);
  const dim3 grid((nrows + kAttnRows - 1) / kAttnRows, p.Hkv), block(kAttnWaves * kWave);
  switch (p.format) {
    case 0: attn_extend_kernel<D, 0><<<grid, block, 0, s>>>(p); break;
    case 1: attn_extend_kernel<D, 1><<<grid, block, 0, s>>>(p); break;
    case 2: attn_extend_kernel<D, 2><<<grid, block, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_extend(const AttnParams& p, hipStream_t s) {
  if (p.n_new <= 0) return hipSuccess;
  switch (p.D) {
    case 64: return launch_d<64>(p, s);
    case 128: return launch_d<128>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ftmoe
