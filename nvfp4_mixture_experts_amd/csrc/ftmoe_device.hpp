// ftmoe_device.hpp -- device helpers shared by every gfx950 kernel of libftmoe:
// the NVFP4 decode routine (the only place where codes and scales become
// numbers), bf16 conversions and wave-level reductions.
//
// NVFP4 element codes are OCP e2m1 (Microscaling v1.0); block scales are OCP
// e4m3 (8-bit Floating Point spec), one per 16 consecutive K elements; each
// tensor carries one fp32 global scale.  The codes are the weights of the
// NVFP4 MoE experts (FreeToken commit log, page 2, the 288- and 512-expert
// NVFP4 MoE entries); decoding them in registers by bit placement rather than
// through a lookup follows FreeToken fork PR #84 (page 1), the bullet on #578.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ftmoe {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ------------------------------------------------------------ NVFP4 codec --

// e4m3 byte (bits 7..0 of `b`) -> fp32, exactly (v_cvt_f32_fp8 decodes the OCP
// E4M3 encoding on gfx950, subnormals and NaN included).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(b), 0);
}

// e4m3 byte `sel` (0..3) of a 32-bit word -> fp32.
template <int Sel>
__device__ __forceinline__ float e4m3_byte_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(w), Sel);
}

// Byte `Sel` of `w` holds two e2m1 codes (low nibble = even element): decode
// both to fp32, exactly.  The hardware scale operand is 1.0 (an identity), the
// NVFP4 e4m3 block scale is applied by the caller.
template <int Sel>
__device__ __forceinline__ f32x2 e2m1x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, Sel);
}

// Same two codes decoded to a packed bf16 pair (every e2m1 value is exact in bf16).
template <int Sel>
__device__ __forceinline__ bf16x2 e2m1x2_to_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, Sel);
}

// One dequantised weight: fp32(fp32(e2m1 * e4m3) * g).  The first product is
// exact (at most 6 significant bits), so this is one rounding of the exact
// value code * scale * g.  `pair` is the e2m1 pair decoded by e2m1x2_to_f32.
__device__ __forceinline__ float dequant_one(float code_value, float scale, float g) {
  return (code_value * scale) * g;
}

// Eight e2m1 codes (one 32-bit word, low nibble = first element) times one e4m3
// block scale -> eight bf16 values packed in a uint4 (an MFMA A/B operand of
// 8 bf16).  Every code x scale product has at most 6 significant bits, so it is
// exact in fp32 and in bf16, and the bf16 is the upper half of the fp32 bits (a
// truncation that loses nothing).  The global scale is not applied here (the
// grouped kernels apply it to the fp32 accumulator).
__device__ __forceinline__ uint32_t upper_halves(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
__device__ __forceinline__ uint4 dequant8_bf16(uint32_t codes, float scale) {
  const f32x2 a = e2m1x2_to_f32<0>(codes), b = e2m1x2_to_f32<1>(codes);
  const f32x2 c = e2m1x2_to_f32<2>(codes), d = e2m1x2_to_f32<3>(codes);
  uint4 r;
  r.x = upper_halves(a.x * scale, a.y * scale);
  r.y = upper_halves(b.x * scale, b.y * scale);
  r.z = upper_halves(c.x * scale, c.y * scale);
  r.w = upper_halves(d.x * scale, d.y * scale);
  return r;
}

// The same eight products as fp16 (an MFMA operand of 8 halves): the codes are
// decoded straight to fp16 pairs and multiplied by the block scale as an fp16
// pair (v_pk_mul_f16), two products per instruction.  Exact as well: every
// product has at most 6 significant bits and lies in [2^-10, 2688] (or is 0),
// inside fp16's normal range, and every e4m3 scale is an fp16 value.  (The
// convert's own scale operand is not used for the block scale: it applies only
// the exponent of its argument.)
template <int Sel>
__device__ __forceinline__ f16x2 e2m1x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, Sel);
}
template <int Sel>
__device__ __forceinline__ _Float16 e4m3_byte_to_f16(uint32_t w) {
  return static_cast<_Float16>(e4m3_byte_to_f32<Sel>(w));  // exact
}
__device__ __forceinline__ uint4 dequant8_f16(uint32_t codes, _Float16 scale) {
  const f16x2 s2 = {scale, scale};
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, e2m1x2_to_f16<0>(codes) * s2);
  r.y = __builtin_bit_cast(uint32_t, e2m1x2_to_f16<1>(codes) * s2);
  r.z = __builtin_bit_cast(uint32_t, e2m1x2_to_f16<2>(codes) * s2);
  r.w = __builtin_bit_cast(uint32_t, e2m1x2_to_f16<3>(codes) * s2);
  return r;
}
// The tile builder of either 16-bit type (H16: fp16, else bf16), scale given as fp32.
template <bool H16>
__device__ __forceinline__ uint4 dequant8_tile(uint32_t codes, float scale) {
  if constexpr (H16) return dequant8_f16(codes, static_cast<_Float16>(scale));
  else return dequant8_bf16(codes, scale);
}

// ------------------------------------------------------- small divisions --
//
// n / d for 0 <= n < 2^24 and d >= 1 through an fp32 reciprocal: the estimate is
// within one of the quotient, and one correction step makes it exact.
struct FastDiv {
  int d;
  float inv;
};
__host__ __device__ inline FastDiv make_fastdiv(int d) { return FastDiv{d, 1.0f / static_cast<float>(d)}; }
__device__ __forceinline__ int fdiv(int n, FastDiv f) {
  int q = static_cast<int>(static_cast<float>(n) * f.inv);
  const int r = n - q * f.d;
  q += (r >= f.d) ? 1 : 0;
  q -= (r < 0) ? 1 : 0;
  return q;
}

// ------------------------------------------------------------ bf16 helpers --

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
// Written as a select (no branch: a wave stays converged).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet_nan = (u >> 16) | 0x0040u;
  return static_cast<uint16_t>((u & 0x7FFFFFFFu) > 0x7F800000u ? quiet_nan : rounded);
}

// Four consecutive h values of one row, as the grouped expert GEMMs hand them from
// the gate|up product to the down product: fp16, nearest-even (h16: the clamped
// activation bounds |h| far inside fp16's range), or a bf16 (hi, lo) pair, hi =
// bf16(h) and lo = bf16(h - hi), whose sum holds h to about 16 significant bits.
__device__ __forceinline__ void store_h4(uint16_t* hhi, uint16_t* hlo, size_t off,
                                         const float (&hv)[4], bool h16) {
  if (h16) {
    const f16x2 a = {static_cast<_Float16>(hv[0]), static_cast<_Float16>(hv[1])};
    const f16x2 b = {static_cast<_Float16>(hv[2]), static_cast<_Float16>(hv[3])};
    *reinterpret_cast<uint2*>(hhi + off) =
        make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
    return;
  }
  uint32_t hi[2], lo[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t h0 = f32_to_bf16_bits(hv[2 * i]), h1 = f32_to_bf16_bits(hv[2 * i + 1]);
    const uint32_t l0 = f32_to_bf16_bits(hv[2 * i] - __uint_as_float(h0 << 16));
    const uint32_t l1 = f32_to_bf16_bits(hv[2 * i + 1] - __uint_as_float(h1 << 16));
    hi[i] = h0 | (h1 << 16);
    lo[i] = l0 | (l1 << 16);
  }
  *reinterpret_cast<uint2*>(hhi + off) = make_uint2(hi[0], hi[1]);
  *reinterpret_cast<uint2*>(hlo + off) = make_uint2(lo[0], lo[1]);
}

// ------------------------------------------------------- wave reductions --

// Sum over aligned groups of `Width` lanes (Width a power of two <= 64); every
// lane of a group ends with the group's sum.  Fixed butterfly order, so the
// result does not depend on timing.
template <int Width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = Width / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

template <int Width>
__device__ __forceinline__ double group_sum(double v) {
#pragma unroll
  for (int off = Width / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Sum over aligned groups of `Width` lanes (8, 16, 32 or 64) with DPP row shifts
// and broadcasts; the sum lands in the LAST lane of each group (other lanes hold
// partial sums).  Fixed order.
template <int Ctrl, int RowMask>
__device__ __forceinline__ float dpp_shift_f32(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, RowMask, 0xf, false));
}

template <int Width>
__device__ __forceinline__ float group_sum_last(float v) {
  static_assert(Width == 8 || Width == 16 || Width == 32 || Width == 64, "group width");
  v += dpp_shift_f32<0x111, 0xf>(v);  // row_shr:1
  v += dpp_shift_f32<0x112, 0xf>(v);  // row_shr:2
  v += dpp_shift_f32<0x114, 0xf>(v);  // row_shr:4  -> lane 8j+7 holds its 8-lane group
  if (Width >= 16) v += dpp_shift_f32<0x118, 0xf>(v);  // row_shr:8 -> lane 15 of each row
  if (Width >= 32) v += dpp_shift_f32<0x142, 0xa>(v);  // row_bcast:15 -> lanes 31, 63
  if (Width >= 64) v += dpp_shift_f32<0x143, 0xc>(v);  // row_bcast:31 -> lane 63
  return v;
}

// ------------------------------------------------------- chunk dot kernels --

// A chunk is 32 consecutive K elements of one weight row: 16 code bytes (a
// uint4) and 2 e4m3 scale bytes (one per 16 elements).
//
// bf16 activations: x2[m] holds elements (2m, 2m+1) of the chunk as a packed bf16
// pair.  Each e2m1 x bf16 product is exact in fp32; the 16-element block sums
// are scaled by their e4m3 scale.  Returns sum_k code_k * scale_k * x_k.
__device__ __forceinline__ float chunk_dot_bf16(const uint4 q, uint32_t sc2, const bf16x2* x2) {
  float b0 = 0.0f, b1 = 0.0f;
  b0 = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<0>(q.x), x2[0], b0, false);
  b0 = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<1>(q.x), x2[1], b0, false);
  b0 = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<2>(q.x), x2[2], b0, false);
  b0 = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<3>(q.x), x2[3], b0, false);
  b0 = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<0>(q.y), x2[4], b0, false);
  b0 = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<1>(q.y), x2[5], b0, false);
  b0 = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<2>(q.y), x2[6], b0, false);
  b0 = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<3>(q.y), x2[7], b0, false);
  b1 = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<0>(q.z), x2[8], b1, false);
  b1 = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<1>(q.z), x2[9], b1, false);
  b1 = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<2>(q.z), x2[10], b1, false);
  b1 = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<3>(q.z), x2[11], b1, false);
  b1 = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<0>(q.w), x2[12], b1, false);
  b1 = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<1>(q.w), x2[13], b1, false);
  b1 = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<2>(q.w), x2[14], b1, false);
  b1 = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<3>(q.w), x2[15], b1, false);
  return b0 * e4m3_byte_to_f32<0>(sc2) + b1 * e4m3_byte_to_f32<1>(sc2);
}

// Four code bytes (8 elements) against 8 fp32 activations.
__device__ __forceinline__ float word_dot_f32(uint32_t w, const float* h, float acc) {
  f32x2 p0 = e2m1x2_to_f32<0>(w), p1 = e2m1x2_to_f32<1>(w);
  f32x2 p2 = e2m1x2_to_f32<2>(w), p3 = e2m1x2_to_f32<3>(w);
  acc = fmaf(p0.x, h[0], acc);
  acc = fmaf(p0.y, h[1], acc);
  acc = fmaf(p1.x, h[2], acc);
  acc = fmaf(p1.y, h[3], acc);
  acc = fmaf(p2.x, h[4], acc);
  acc = fmaf(p2.y, h[5], acc);
  acc = fmaf(p3.x, h[6], acc);
  acc = fmaf(p3.y, h[7], acc);
  return acc;
}

// fp32 activations h[0..31] (the SwiGLU output): the e2m1 codes are decoded to
// fp32 and accumulated with fp32 FMAs, block sums scaled by their e4m3 scale.
__device__ __forceinline__ float chunk_dot_f32(const uint4 q, uint32_t sc2, const float* h) {
  float b0 = word_dot_f32(q.x, h, 0.0f);
  b0 = word_dot_f32(q.y, h + 8, b0);
  float b1 = word_dot_f32(q.z, h + 16, 0.0f);
  b1 = word_dot_f32(q.w, h + 24, b1);
  return b0 * e4m3_byte_to_f32<0>(sc2) + b1 * e4m3_byte_to_f32<1>(sc2);
}

// ------------------------------------------------------- block-fp8 chunks --
//
// The block-fp8 codec: one OCP e4m3 byte per weight and one fp32 scale per 128 x 128
// block.  A chunk is again 32 consecutive K elements of one row: 32 code bytes (two
// uint4; element 4m + i in byte i of word m) inside one scale block.

// Bytes Sel*2, Sel*2+1 of `w` (two e4m3 codes) -> a bf16 pair, exactly (an e4m3 value
// has 4 significant bits and an exponent inside bf16's normal range).
template <bool Hi>
__device__ __forceinline__ bf16x2 e4m3x2_to_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, Hi);
}
// The same two codes -> fp32, exactly.
template <bool Hi>
__device__ __forceinline__ f32x2 e4m3x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, Hi);
}

__device__ __forceinline__ uint32_t word_of(const uint4& a, const uint4& b, int m) {
  const uint4& q = m < 4 ? a : b;
  const int i = m & 3;
  return i == 0 ? q.x : (i == 1 ? q.y : (i == 2 ? q.z : q.w));
}

// sum_k code_k * x_k over one chunk (bf16 activations x2[m] = elements 2m, 2m+1):
// exact products, fp32 accumulation in two chains; the block scale is applied by
// the caller.
__device__ __forceinline__ float chunk_dot_fp8_bf16(const uint4 q0, const uint4 q1,
                                                    const bf16x2* x2) {
  float b0 = 0.0f, b1 = 0.0f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    b0 = __builtin_amdgcn_fdot2_f32_bf16(e4m3x2_to_bf16<false>(word_of(q0, q1, m)), x2[2 * m],
                                         b0, false);
    b0 = __builtin_amdgcn_fdot2_f32_bf16(e4m3x2_to_bf16<true>(word_of(q0, q1, m)),
                                         x2[2 * m + 1], b0, false);
  }
#pragma unroll
  for (int m = 4; m < 8; ++m) {
    b1 = __builtin_amdgcn_fdot2_f32_bf16(e4m3x2_to_bf16<false>(word_of(q0, q1, m)), x2[2 * m],
                                         b1, false);
    b1 = __builtin_amdgcn_fdot2_f32_bf16(e4m3x2_to_bf16<true>(word_of(q0, q1, m)),
                                         x2[2 * m + 1], b1, false);
  }
  return b0 + b1;
}

// sum_k code_k * h_k over one chunk with fp32 activations h[0..31].
__device__ __forceinline__ float chunk_dot_fp8_f32(const uint4 q0, const uint4 q1, const float* h) {
  float b0 = 0.0f, b1 = 0.0f;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const uint32_t w = word_of(q0, q1, m);
    const f32x2 lo = e4m3x2_to_f32<false>(w), hi = e4m3x2_to_f32<true>(w);
    float& b = m < 4 ? b0 : b1;
    b = fmaf(lo.x, h[4 * m], b);
    b = fmaf(lo.y, h[4 * m + 1], b);
    b = fmaf(hi.x, h[4 * m + 2], b);
    b = fmaf(hi.y, h[4 * m + 3], b);
  }
  return b0 + b1;
}

// ------------------------------------------- device-coherent hand-offs --
//
// Data that one block of a kernel hands to another block of the same kernel is
// written and read with device-scope relaxed atomics: on gfx950 these are plain
// loads/stores carrying the device-coherence cache policy (they bypass the
// per-XCD L2 copies), so no cache-wide write-back or invalidate is needed.
// The producer waits for its stores to complete (wait_mem) before it signals a
// counter; the consumer reads the counter, then the data.

__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_dev(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_mem() { __builtin_amdgcn_s_waitcnt(0); }

// ------------------------------------------------------ DPP wave reductions --
//
// Reductions across the 64 lanes of a wave with DPP row shifts and row
// broadcasts (no LDS round trip); the result is returned to every lane.

template <uint32_t Identity, class Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(Identity), static_cast<int>(v), 0x111, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(Identity), static_cast<int>(v), 0x112, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(Identity), static_cast<int>(v), 0x114, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(Identity), static_cast<int>(v), 0x118, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(Identity), static_cast<int>(v), 0x142, 0xa, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(Identity), static_cast<int>(v), 0x143, 0xc, 0xf, false)));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// Sum of a double over the 64 lanes of a wave (fixed DPP tree), returned to
// every lane.
template <int Ctrl, int RowMask>
__device__ __forceinline__ double dpp_shift_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(u), Ctrl, RowMask, 0xf, false));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(u >> 32), Ctrl, RowMask, 0xf, false));
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_shift_f64<0x111, 0xf>(v);
  v += dpp_shift_f64<0x112, 0xf>(v);
  v += dpp_shift_f64<0x114, 0xf>(v);
  v += dpp_shift_f64<0x118, 0xf>(v);
  v += dpp_shift_f64<0x142, 0xa>(v);
  v += dpp_shift_f64<0x143, 0xc>(v);
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u), 63));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u >> 32), 63));
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// Lane `src` (wave-uniform) of a double, broadcast through scalar registers.
__device__ __forceinline__ double readlane_f64(double v, int src) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u), src));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u >> 32), src));
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_reduce_u32<0u>(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return wave_reduce_u32<0xFFFFFFFFu>(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}

// ------------------------------------------------------------------ top-k --
//
// Rank key of a logit: an unsigned integer that orders like the logit, with
// -0 folded onto +0 (they compare equal) and a NaN below every number (key 1).
// Key 0 marks "no candidate".
__device__ __forceinline__ uint32_t rank_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 1u;  // NaN
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;              // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {
  if (key == 1u) return __builtin_nanf("");
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Top-k of one token's E (<= 64 * SLOTS) logits by one wave: experts ordered by
// (logit descending, index ascending), then the softmax of the selected logits
// (fp64 exp, stored as fp32).  Lane l holds experts l, l + 64, ... in slots
// 0, 1, ..., so scanning the slots in order and taking the lowest set lane of
// the first non-empty ballot finds the lowest index among equal keys.  Returns
// the rank-i expert and weight in lane i (i < k); other lanes return -1 / 0.
template <int SLOTS>
__device__ __forceinline__ void wave_topk_vals(int E, int k, const float* lv, int* out_id,
                                               float* out_w) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t key[SLOTS];
#pragma unroll
  for (int m = 0; m < SLOTS; ++m) key[m] = (lane + kWave * m < E) ? rank_key(lv[m]) : 0u;
  auto local_max = [&]() {
    uint32_t mx = key[0];
#pragma unroll
    for (int m = 1; m < SLOTS; ++m) mx = key[m] > mx ? key[m] : mx;
    return mx;
  };
  uint32_t lmax = local_max();
  int my_id = -1;
  uint32_t my_key = 0u;
  for (int i = 0; i < k; ++i) {
    const uint32_t K = wave_max_u32(lmax);
    int win = -1;
#pragma unroll
    for (int m = 0; m < SLOTS; ++m) {
      if (win < 0) {
        const uint64_t b = __ballot(key[m] == K);
        if (b != 0) win = kWave * m + __ffsll(static_cast<unsigned long long>(b)) - 1;
      }
    }
    if (lane == i) {
      my_id = win;
      my_key = K;
    }
    if ((win & (kWave - 1)) == lane) {
#pragma unroll
      for (int m = 0; m < SLOTS; ++m)
        if (m == (win >> 6)) key[m] = 0u;
      lmax = local_max();
    }
  }
  // softmax over the selected logits, in fp64, summed in rank order
  const double top = static_cast<double>(key_value(static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(my_key), 0))));
  const double d = (lane < k) ? exp(static_cast<double>(key_value(my_key)) - top) : 0.0;
  double sum = 0.0;
  for (int i = 0; i < k; ++i) sum += readlane_f64(d, i);
  *out_id = my_id;
  *out_w = (lane < k) ? static_cast<float>(d / sum) : 0.0f;
}

// Same, loading the logits through `load_logit(e)` (every load issued first,
// indices clamped into range).
template <int SLOTS, class Load>
__device__ __forceinline__ void wave_topk(int E, int k, Load load_logit, int* out_id,
                                          float* out_w) {
  const int lane = threadIdx.x & (kWave - 1);
  float lv[SLOTS];
#pragma unroll
  for (int m = 0; m < SLOTS; ++m) {
    const int e = lane + kWave * m;
    lv[m] = load_logit(e < E ? e : E - 1);
  }
  wave_topk_vals<SLOTS>(E, k, lv, out_id, out_w);
}

// ------------------------------------------------- block top-k (rank counting) --

constexpr int kTopkMaxChunks = 16;  // 64-expert chunks (E <= 1024)
constexpr int kTopkMaxK = 16;

// Orders this wave's LDS accesses before and after the call for all of its lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// How many of the 64 keys at p (LDS, read at the same address by every lane: a
// broadcast) lie above key.  The reads go out 16 at a time ahead of their
// compares, so the 64 keys cost two LDS latencies rather than one per read.
__device__ __forceinline__ int count_above64(const uint64_t* p, uint64_t key) {
  const ulonglong2* p2 = reinterpret_cast<const ulonglong2*>(p);
  int above = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    ulonglong2 v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = p2[16 * h + j];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      above += (v[j].x > key) ? 1 : 0;
      above += (v[j].y > key) ? 1 : 0;
    }
  }
  return above;
}

// The top k of one token's E logits by all BW waves of a block, with no serial
// select rounds.  Expert e carries the 64-bit key (rank_key(logit) << 32) | ~e: a
// larger key is a larger logit, or an equal logit at a lower index, and no two
// keys are equal.  fetch(e) returns logit e; every lane of a wave calls it at once
// for the wave's chunk (so it may poll with wave-wide votes).
// 1. Wave w fetches the 64-expert chunks w, w + BW, ... and counts, for each expert,
//    the keys of its own chunk above its key.  An expert with fewer than k above
//    it is a candidate, stored at (chunk, count).
// 2. Each candidate counts the candidates above it (4 lanes per candidate, over
//    all waves).  For an expert of the top k every key above it is itself a
//    candidate (fewer than k keys lie above it in all), so the count is its
//    place; any other candidate counts at least k (some chunk holds k candidates
//    above it).  A count below k is the expert's place.
// Results: ids[place] and s_v[place] (the place's logit, in fp64), complete for
// every wave on return.  The softmax itself (softmax_of_places) is left to the
// caller: the decode kernel needs only the ids to start streaming the experts'
// weights, and takes the exponentials while those loads are in flight.
// LDS: s_key[BW][64], s_cand[kTopkMaxChunks * kTopkMaxK] (16-byte aligned), s_v[k].
template <int BW, class Fetch>
__device__ __forceinline__ void block_topk_rank(int E, int k, Fetch fetch,
                                                uint64_t (*s_key)[kWave], uint64_t* s_cand,
                                                double* s_v, int* ids) {
  static_assert(kTopkMaxChunks * kTopkMaxK <= BW * kWave, "one candidate per thread");
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nchunks = (E + kWave - 1) / kWave;
  const int nc = nchunks * k;                     // <= kTopkMaxChunks * kTopkMaxK
  const int nc64 = (nc + kWave - 1) & ~(kWave - 1);
  for (int i = nc + static_cast<int>(threadIdx.x); i < nc64; i += blockDim.x) s_cand[i] = 0ull;
  for (int c = wave; c < nchunks; c += BW) {
    const int e = c * kWave + lane;
    const float v = fetch(e < E ? e : E - 1);
    const uint64_t key =
        (e < E) ? (static_cast<uint64_t>(rank_key(v)) << 32) | static_cast<uint32_t>(~e) : 0ull;
    uint64_t* ck = s_key[wave];
    ck[lane] = key;
    if (lane < k) s_cand[c * k + lane] = 0ull;  // places a short chunk leaves empty
    wave_lds_sync();
    const int above = count_above64(ck, key);
    if (key != 0ull && above < k) s_cand[c * k + above] = key;
    wave_lds_sync();  // ck is rewritten by this wave's next chunk
  }
  __syncthreads();
  // Candidate i is counted by the 4 lanes 4i .. 4i + 3 (a quad, inside one wave):
  // lane q of the quad compares it with entries 16q .. 16q + 15 of every 64.
  for (int c0 = 0; c0 < nc; c0 += BW * kWave / 4) {
    const int cand = c0 + static_cast<int>(threadIdx.x >> 2);
    const int q = threadIdx.x & 3;
    const uint64_t mine = s_cand[cand < nc ? cand : 0];
    int above = 0;  // zero entries count for nothing
    for (int j0 = 0; j0 < nc64; j0 += kWave) {
      const ulonglong2* p2 = reinterpret_cast<const ulonglong2*>(s_cand + j0 + 16 * q);
      ulonglong2 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = p2[j];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        above += (v[j].x > mine) ? 1 : 0;
        above += (v[j].y > mine) ? 1 : 0;
      }
    }
    above += __builtin_amdgcn_update_dpp(0, above, 0xB1, 0xf, 0xf, false);  // lanes ^ 1
    above += __builtin_amdgcn_update_dpp(0, above, 0x4E, 0xf, 0xf, false);  // lanes ^ 2
    if (cand < nc && q == 0 && mine != 0ull && above < k) {
      ids[above] = static_cast<int>(~static_cast<uint32_t>(mine));
      s_v[above] = static_cast<double>(key_value(static_cast<uint32_t>(mine >> 32)));
    }
  }
  __syncthreads();
}

// The routing weights of one token from the logits v[0..k) of its places (place
// 0 the largest): the terms exp(v[i] - v[0]) in fp64, their sum in place order,
// then each term over it, by one wave in its own registers: lane i returns the
// weight of place i (0 from lane k on).
__device__ __forceinline__ float softmax_of_places(const double* s_v, int k) {
  const int lane = threadIdx.x & (kWave - 1);
  const double v = (lane < k) ? s_v[lane] : 0.0;
  const double top = readlane_f64(v, 0);
  const double d = (lane < k) ? exp(v - top) : 0.0;
  double sum = 0.0;
  for (int i = 0; i < k; ++i) sum += readlane_f64(d, i);
  return (lane < k) ? static_cast<float>(d / sum) : 0.0f;
}

// ------------------------------------------------------ vector-memory loads --
//
// base[index] through a buffer load (the vector memory path).  A wave-uniform
// fp32 load would otherwise be issued on the scalar path, whose completion
// counter is shared with LDS reads: every later LDS read would then wait for it.
__device__ __forceinline__ float ld_vmem_f32(const float* base, int index) {
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(base), static_cast<short>(0), 0x7fffffff, 0x00020000);
  return __uint_as_float(
      static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(r, 4 * index, 0, 0)));
}

// ------------------------------------------------------------- activation --

// silu(z) = z / (1 + exp(-z)), with the hardware base-2 exponential and
// reciprocal (each about 1 ulp; the result within a few fp32 ulp, far below the
// bf16 resolution of the outputs).  For very negative z, exp(-z) overflows to +inf,
// its reciprocal is 0 and the result is -0 (never NaN); NaN stays NaN.
__device__ __forceinline__ float silu(float z) {
  const float e = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// act 0: silu(g) * u.  act 1: silu(min(g, gate_max)) * clamp(u, -up_absmax, up_absmax).
// Written as compare-and-select so that a NaN input stays NaN.
__device__ __forceinline__ float swiglu(int act, float g, float u, float gate_max,
                                        float up_absmax) {
  if (act == 1) {
    g = (g > gate_max) ? gate_max : g;
    u = (u > up_absmax) ? up_absmax : u;
    u = (u < -up_absmax) ? -up_absmax : u;
  }
  return silu(g) * u;
}

}  // namespace ftmoe
