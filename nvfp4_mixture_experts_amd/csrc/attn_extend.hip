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
// One wave per (new token, query head).  Per chunk: lane j owns key j: its score is
// q . k_j with the key's codes turned into bf16 pairs in registers (exact for every
// format: an e4m3 value, or an e2m1 code times its e4m3 block scale, has at most 6
// significant bits) against q held as bf16 pairs in LDS, fp32 accumulation, then the
// tensor scale and 1/sqrt(d) on the dot output.  Online softmax across the wave.  The
// chunk's V rows are staged in LDS as exact bf16 (code x block scale); then lanes
// own output dimensions and accumulate p_j v_j over the chunk, and the V tensor scale
// multiplies that chunk's P.V output.
#include "ftmoe_device.hpp"
#include "ftmoe_kernels.hpp"

namespace ftmoe {
namespace {

constexpr int kAttnWaves = 4;

template <int D>
struct AttnLds {
  uint32_t q[kAttnWaves][D / 2];                    // bf16 pairs of the wave's query
  float p[kAttnWaves][kWave];                       // probabilities of the chunk's keys
  __align__(16) uint8_t v[kAttnWaves][kWave][2 * D + 16];  // V rows, bf16 (16-byte pad)
};

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ uint32_t pack_bf16x2(bf16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// One key row: the score dot product (codes against q, block scales applied) and the
// row's values as bf16 into `vrow` (2 * D bytes).  FMT 0 bf16, 1 e4m3, 2 NVFP4.
template <int D, int FMT>
__device__ __forceinline__ float key_dot(const void* kc, const uint8_t* kbs, size_t row,
                                         const uint32_t* q2) {
  float dot = 0.0f;
#pragma unroll
  for (int b = 0; b < D / 16; ++b) {  // 16 elements per step (one NVFP4 block)
    float part = 0.0f;
    if constexpr (FMT == 0) {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(kc) + row * D + 16 * b);
      const uint4 a = p[0], c = p[1];
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
      for (int m = 0; m < 8; ++m)
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[m]),
                                               __builtin_bit_cast(bf16x2, q2[8 * b + m]), part, false);
    } else if constexpr (FMT == 1) {
      const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(kc) + row * D + 16 * b);
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        part = __builtin_amdgcn_fdot2_f32_bf16(e4m3x2_to_bf16<false>(w[m]),
                                               __builtin_bit_cast(bf16x2, q2[8 * b + 2 * m]), part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(e4m3x2_to_bf16<true>(w[m]),
                                               __builtin_bit_cast(bf16x2, q2[8 * b + 2 * m + 1]), part, false);
      }
    } else {
      const uint2 a = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(kc) + row * (D / 2) + 8 * b);
      const uint32_t w[2] = {a.x, a.y};
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        part = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<0>(w[m]),
                                               __builtin_bit_cast(bf16x2, q2[8 * b + 4 * m]), part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<1>(w[m]),
                                               __builtin_bit_cast(bf16x2, q2[8 * b + 4 * m + 1]), part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<2>(w[m]),
                                               __builtin_bit_cast(bf16x2, q2[8 * b + 4 * m + 2]), part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<3>(w[m]),
                                               __builtin_bit_cast(bf16x2, q2[8 * b + 4 * m + 3]), part, false);
      }
      part *= e4m3_to_f32(kbs[row * (D / 16) + b]);
    }
    dot += part;
  }
  return dot;
}

template <int D, int FMT>
__device__ __forceinline__ void value_row_to_lds(const void* vc, const uint8_t* vbs, size_t row,
                                                 uint8_t* dst) {
#pragma unroll
  for (int b = 0; b < D / 16; ++b) {
    uint4 lo, hi;
    if constexpr (FMT == 0) {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(vc) + row * D + 16 * b);
      lo = p[0];
      hi = p[1];
    } else if constexpr (FMT == 1) {
      const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(vc) + row * D + 16 * b);
      lo = make_uint4(pack_bf16x2(e4m3x2_to_bf16<false>(a.x)), pack_bf16x2(e4m3x2_to_bf16<true>(a.x)),
                      pack_bf16x2(e4m3x2_to_bf16<false>(a.y)), pack_bf16x2(e4m3x2_to_bf16<true>(a.y)));
      hi = make_uint4(pack_bf16x2(e4m3x2_to_bf16<false>(a.z)), pack_bf16x2(e4m3x2_to_bf16<true>(a.z)),
                      pack_bf16x2(e4m3x2_to_bf16<false>(a.w)), pack_bf16x2(e4m3x2_to_bf16<true>(a.w)));
    } else {
      const uint2 a = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(vc) + row * (D / 2) + 8 * b);
      const float s = e4m3_to_f32(vbs[row * (D / 16) + b]);
      lo = dequant8_bf16(a.x, s);
      hi = dequant8_bf16(a.y, s);
    }
    reinterpret_cast<uint4*>(dst)[2 * b] = lo;
    reinterpret_cast<uint4*>(dst)[2 * b + 1] = hi;
  }
}

struct Online {
  float m, l;
};

// Keys [k0, k1) of one source (the cache in format FMT, or the new tokens in bf16),
// positions pos0 + (key - first) ... all visible; acc over this lane's DPL dims.
template <int D, int FMT>
__device__ void attend_range(const AttnParams& p, int kh, int first, int k0, int k1,
                             const void* kc, const void* vc, const uint8_t* kbs,
                             const uint8_t* vbs, float kscale, float vscale, AttnLds<D>& lds,
                             int wave, Online& st, float* acc) {
  constexpr int DPL = D / kWave;  // output dims per lane
  const int lane = threadIdx.x & (kWave - 1);
  for (int c0 = k0; c0 < k1; c0 += kWave) {
    const int key = c0 + lane;
    const bool valid = key < k1;
    const size_t row = static_cast<size_t>(valid ? key - first : k0 - first) * p.Hkv + kh;
    float s = -INFINITY;
    const float dot = key_dot<D, FMT>(kc, kbs, row, lds.q[wave]);
    if (valid) s = dot * kscale * p.sm_scale;
    value_row_to_lds<D, FMT>(vc, vbs, row, lds.v[wave][lane]);
    const float mc = wave_max_f32(s);
    const float mn = fmaxf(st.m, mc);  // finite: the chunk's first key is visible
    const float alpha = __builtin_amdgcn_exp2f((st.m - mn) * 1.4426950408889634f);
    const float pj = valid ? __builtin_amdgcn_exp2f((s - mn) * 1.4426950408889634f) : 0.0f;
    st.l = st.l * alpha + wave_sum_f32(pj);
    st.m = mn;
    lds.p[wave][lane] = pj;
    wave_lds_sync();
    float pv[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) pv[i] = 0.0f;
    const int n = k1 - c0 < kWave ? k1 - c0 : kWave;
    for (int j = 0; j < n; ++j) {
      const float pjj = lds.p[wave][j];
      const uint16_t* vr = reinterpret_cast<const uint16_t*>(lds.v[wave][j]) + lane * DPL;
#pragma unroll
      for (int i = 0; i < DPL; ++i) pv[i] = fmaf(pjj, bf16_bits_to_f32(vr[i]), pv[i]);
    }
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] = fmaf(pv[i], vscale, acc[i] * alpha);
    wave_lds_sync();  // the next chunk rewrites p and v
  }
}

template <int D, int FMT>
__global__ __launch_bounds__(kAttnWaves* kWave) void attn_extend_kernel(AttnParams p) {
  constexpr int DPL = D / kWave;
  __shared__ AttnLds<D> lds;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int item = blockIdx.x * kAttnWaves + wave;
  if (item >= p.n_new * p.Hq) return;  // whole wave; the kernel has no block barrier
  const int t = item / p.Hq, h = item % p.Hq;
  const int kh = h / (p.Hq / p.Hkv);
  const int qpos = p.prefix + t;
  const int lo = p.window > 0 ? (qpos - p.window + 1 > 0 ? qpos - p.window + 1 : 0) : 0;
  const uint32_t* qrow = reinterpret_cast<const uint32_t*>(p.q + (static_cast<size_t>(t) * p.Hq + h) * D);
  for (int i = lane; i < D / 2; i += kWave) lds.q[wave][i] = qrow[i];
  wave_lds_sync();
  Online st{-INFINITY, 0.0f};
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.0f;
  // cached keys [lo, prefix) in the cache's format, tensor scales on the dot outputs
  if (lo < p.prefix)
    attend_range<D, FMT>(p, kh, 0, lo, p.prefix, p.k_cache, p.v_cache, p.k_bscale, p.v_bscale,
                         FMT == 0 ? 1.0f : p.k_scale, FMT == 0 ? 1.0f : p.v_scale, lds, wave, st,
                         acc);
  // new keys [max(lo, prefix), qpos], bf16
  const int n0 = lo > p.prefix ? lo : p.prefix;
  attend_range<D, 0>(p, kh, p.prefix, n0, qpos + 1, p.k_new, p.v_new, nullptr, nullptr, 1.0f, 1.0f,
                     lds, wave, st, acc);
  uint16_t* orow = p.out + (static_cast<size_t>(t) * p.Hq + h) * D + lane * DPL;
#pragma unroll
  for (int i = 0; i < DPL; ++i) orow[i] = f32_to_bf16_bits(acc[i] / st.l);
}

template <int D>
hipError_t launch_d(const AttnParams& p, hipStream_t s) {
  const dim3 grid((p.n_new * p.Hq + kAttnWaves - 1) / kAttnWaves), block(kAttnWaves * kWave);
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
