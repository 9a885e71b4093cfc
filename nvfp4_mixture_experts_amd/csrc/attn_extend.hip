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
// share a kv head share every staged key and value.  Per chunk of 64 keys:
//   1. the chunk's keys and values are turned into bf16 in LDS (exact for every
//      format: an e4m3 value, or an e2m1 code times its e4m3 block scale, has at most
//      6 significant bits), keys as rows [key][dim], values transposed [dim][key];
//   2. S = Q K^T on v_mfma_f32_16x16x32_bf16 (each wave its 16 rows x 64 keys, Q in
//      registers), times the key tensor scale and 1/sqrt(d) on the dot outputs, keys
//      outside a row's causal / window range masked;
//   3. online softmax per row in fp32 (base-2 exponentials); the normaliser sums the
//      unscaled probabilities; P times the value tensor scale goes through LDS to the
//      MFMA operand layout as a bf16 pair (hi = bf16(p), lo = bf16(p - hi): about 16
//      significant bits; one bf16 alone costs the output about 2e-3 of relative L2);
//   4. O = O * alpha + P V on the MFMA (each wave 16 rows x d; the hi and lo products
//      into the same accumulator).
// At the end O / l is rounded to bf16.
#include "ftmoe_device.hpp"
#include "ftmoe_kernels.hpp"

namespace ftmoe {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 at_bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float at_f32x4;
typedef unsigned int at_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAttnWaves = 4;
constexpr int kAttnRows = 16 * kAttnWaves;  // query rows per block
constexpr int kChunk = 64;                  // keys per chunk
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct AttnLds {
  uint16_t k[kChunk][D + 8];             // keys of the chunk, bf16 (8 of padding)
  uint16_t vt[D][kChunk + 8];            // values transposed, bf16
  uint16_t p[kAttnWaves][2][16][kChunk + 8];  // a wave's probabilities, bf16 hi and lo
};

__device__ __forceinline__ at_f32x4 mfma(at_u32x4 a, at_u32x4 b, at_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(at_bf16x8, a),
                                                 __builtin_bit_cast(at_bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pk(bf16x2 v) { return __builtin_bit_cast(uint32_t, v); }

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
  float m[4], l[4];       // running max (base 2) and normaliser of the lane's 4 rows
  at_f32x4 o[D / 16];     // output fragments (dims 16 f + lane % 16)
  int lo[4], hi[4];       // visible key positions [lo, hi] of the lane's 4 rows
};

// One chunk [c0, end) (end - c0 <= 64) of one source against the wave's 16 rows.
// kscale2 = key tensor scale x 1/sqrt(d) x log2(e); vscale multiplies P.
template <int D, int FMT>
__device__ __forceinline__ void chunk_step(AttnLds<D>& lds, const at_u32x4 (&qf)[D / 32], int c0,
                                           int end, float kscale2, float vscale, RowState<D>& st) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  // S = Q K^T: 4 key fragments of 16
  at_f32x4 s[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    s[c] = at_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      s[c] = mfma(qf[ks], *reinterpret_cast<const at_u32x4*>(&lds.k[16 * c + i][32 * ks + 8 * g]),
                  s[c]);
  }
  // lane: rows 4 g + r, keys 16 c + i
  float alpha[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int kpos = c0 + 16 * c + i;
      const bool vis = kpos < end && kpos >= st.lo[r] && kpos <= st.hi[r];
      const float v = vis ? s[c][r] * kscale2 : -INFINITY;
      s[c][r] = v;
      mx = fmaxf(mx, v);
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
    const float mn = fmaxf(st.m[r], mx);
    // no visible key so far: nothing to rescale, every probability 0
    alpha[r] = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(st.m[r] - mn);
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float pj = mn == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s[c][r] - mn);
      s[c][r] = pj;
      sum += pj;
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) sum += __shfl_xor(sum, off, kWave);
    st.l[r] = st.l[r] * alpha[r] + sum;
    st.m[r] = mn;
  }
  // P (times the value scale) as a bf16 pair into the wave's LDS rows, read back as
  // the A operand (row i, keys 32 ks + 8 g ..)
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pv = s[c][r] * vscale;
      const uint16_t hb = f32_to_bf16_bits(pv);
      lds.p[wave][0][4 * g + r][16 * c + i] = hb;
      lds.p[wave][1][4 * g + r][16 * c + i] = f32_to_bf16_bits(pv - bf16_bits_to_f32(hb));
    }
  wave_lds_sync();
  at_u32x4 pf[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      pf[h][ks] = *reinterpret_cast<const at_u32x4*>(&lds.p[wave][h][i][32 * ks + 8 * g]);
  // O = O alpha + P V
#pragma unroll
  for (int f = 0; f < D / 16; ++f) {
#pragma unroll
    for (int r = 0; r < 4; ++r) st.o[f][r] *= alpha[r];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const at_u32x4 v = *reinterpret_cast<const at_u32x4*>(&lds.vt[16 * f + i][32 * ks + 8 * g]);
      st.o[f] = mfma(pf[0][ks], v, st.o[f]);
      st.o[f] = mfma(pf[1][ks], v, st.o[f]);
    }
  }
}

// Keys [k0, k1) of one source (the cache in format FMT, or the new tokens in bf16;
// `first` = the position of the source's row 0), 64 at a time, each chunk's loads
// issued while the previous chunk is multiplied.
template <int D, int FMT>
__device__ __forceinline__ void attend_range(AttnLds<D>& lds, const at_u32x4 (&qf)[D / 32],
                                             const void* kc, const void* vc, const uint8_t* kbs,
                                             const uint8_t* vbs, int first, int k0, int k1,
                                             int Hkv, int kh, float kscale2, float vscale,
                                             RowState<D>& st) {
  if (k0 >= k1) return;
  ChunkRaw<D> raw;
  fetch_chunk<D, FMT>(raw, kc, vc, kbs, vbs, k0, first, k0 + kChunk < k1 ? k0 + kChunk : k1, Hkv, kh);
  for (int c0 = k0; c0 < k1; c0 += kChunk) {
    const int end = c0 + kChunk < k1 ? c0 + kChunk : k1;
    __syncthreads();  // the previous chunk's keys and values have been read
    store_chunk<D, FMT>(lds, raw);
    const int n0 = c0 + kChunk;
    if (n0 < k1) fetch_chunk<D, FMT>(raw, kc, vc, kbs, vbs, n0, first, n0 + kChunk < k1 ? n0 + kChunk : k1, Hkv, kh);
    __syncthreads();
    chunk_step<D, FMT>(lds, qf, c0, end, kscale2, vscale, st);
  }
}

template <int D, int FMT>
__global__ __launch_bounds__(kAttnWaves* kWave) void attn_extend_kernel(AttnParams p) {
  __shared__ AttnLds<D> lds;
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
  // this lane's rows of S and O: 16 wave + 4 g + r; its row of the Q operand: 16 wave + i
  RowState<D> st;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = token_of(r0 + 16 * wave + 4 * g + r);
    st.m[r] = -INFINITY;
    st.l[r] = 0.0f;
    st.lo[r] = lo_of(t);
    st.hi[r] = p.prefix + t;
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
  const float s2 = p.sm_scale * kLog2e;
  if (klo < p.prefix)
    attend_range<D, FMT>(lds, qf, p.k_cache, p.v_cache, p.k_bscale, p.v_bscale, 0, klo,
                         p.prefix < khi ? p.prefix : khi, p.Hkv, kh,
                         (FMT == 0 ? 1.0f : p.k_scale) * s2, FMT == 0 ? 1.0f : p.v_scale, st);
  const int n0 = klo > p.prefix ? klo : p.prefix;
  attend_range<D, 0>(lds, qf, p.k_new, p.v_new, nullptr, nullptr, p.prefix, n0, khi, p.Hkv, kh, s2,
                     1.0f, st);
  // O / l (every row sees its own position, so l > 0)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = r0 + 16 * wave + 4 * g + r;
    if (row >= nrows) continue;
    const int t = row / G, h = kh * G + row % G;
    uint16_t* orow = p.out + (static_cast<size_t>(t) * p.Hq + h) * D;
    const float inv = 1.0f / st.l[r];
#pragma unroll
    for (int f = 0; f < D / 16; ++f) orow[16 * f + i] = f32_to_bf16_bits(st.o[f][r] * inv);
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
