// fp8_linear.hip -- per-tensor FP8 W8A8 projection GEMM on gfx950, in its row-wise
// form (one GEMM, each output row scaled by its part's weight scale) and its per-part
// form (one tensor-wise GEMM per part over that part's row slice).
//
// FreeToken commit log (page 2), the paragraph on row-wise FP8 scaled matrix
// products: the fused per-tensor-FP8 projections (q/k/v stacked along the output
// rows) are W8A8 products; where the row-wise product cannot be used, each part runs
// as its own tensor-wise product over its row slice, the parts taken from the
// run-lengths of the per-row weight scales at load time.
//
//   s_x  = amax|x| / 448                       (fp32, correctly rounded; 1 if x == 0)
//   xq   = e4m3_rne(x / s_x)                   (fp32 quotient, round to nearest even)
//   y    = bf16( (sum_k xq * w) * s_x * s_w[n] )   fp32 accumulation on the MFMA units
//
// Kernels: per-block amax partials; quantisation (every block reduces the partials
// itself, so there is no atomic and nothing to reset between calls), or for small
// activations (M K <= 16 Ki) both in one block; the GEMM on v_mfma_f32_16x16x32_fp8_fp8,
// 64 x 64 output tiles per 4-wave block, 64-deep K slabs staged in LDS, or for M <= 8
// rows of activations (decode) a GEMV: a wave per 4 weight rows, each lane 32 K bytes
// of them with all of its loads in flight at once, codes widened to bf16 pairs
// (exactly: an e4m3 value has 4 significant bits) into v_dot2_f32_bf16.  The row-wise
// call with at most 8 rows of at most 2048 (and M K <= 16 Ki) runs as ONE kernel: every
// GEMV block forms the scale and the codes of x itself, in LDS.
#include "ftmoe_device.hpp"
#include "ftmoe_kernels.hpp"

namespace ftmoe {
namespace {

// 16-byte load without cache allocation (for weights read once per call)
__device__ __forceinline__ uint4 ldg16_nt(const void* p) {
  typedef unsigned int nt_u4 __attribute__((ext_vector_type(4)));
  const nt_u4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
// native vector: a HIP uint4 copied from global memory to LDS stays a memcpy through
// private memory
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAmaxThreads = 256;
constexpr int kAmaxMaxBlocks = 1024;  // amax partials at most
static_assert(kAmaxMaxBlocks % kAmaxThreads == 0, "partials per thread");
constexpr int kTile = 64;       // output rows and columns of a block
constexpr int kSlab = 64;       // K elements per LDS slab
constexpr int kLdsRow = kSlab + 16;  // bytes per LDS row (16 bytes of padding)

__device__ __forceinline__ float bf16_at(const uint16_t* x, size_t i) {
  return bf16_bits_to_f32(x[i]);
}

// max(m, |v|) over the eight bf16 values of a 16-byte piece.
__device__ __forceinline__ float absmax8(float m, const uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    m = fmaxf(m, fabsf(__uint_as_float(w[j] << 16)));
    m = fmaxf(m, fabsf(__uint_as_float(w[j] & 0xFFFF0000u)));
  }
  return m;
}

// Per-block amax partials of x, read as n8 16-byte pieces (x is 16-byte aligned), four
// pieces in flight per thread.
__global__ __launch_bounds__(kAmaxThreads) void fp8_amax_kernel(const uint4* __restrict__ x,
                                                                size_t n8, float* partial) {
  __shared__ float red[kAmaxThreads / kWave];
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  float m = 0.0f;
  for (; i + 3 * stride < n8; i += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = x[i + j * stride];
#pragma unroll
    for (int j = 0; j < 4; ++j) m = absmax8(m, v[j]);
  }
  for (; i < n8; i += stride) m = absmax8(m, x[i]);
  m = __int_as_float(static_cast<int>(wave_max_u32(__float_as_uint(m))));
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = red[0];
    for (int w = 1; w < kAmaxThreads / kWave; ++w) b = fmaxf(b, red[w]);
    partial[blockIdx.x] = b;
  }
}

// Four bf16 values (two words) -> four e4m3 codes in one word, lowest value first.
__device__ __forceinline__ uint32_t quant4(uint32_t w0, uint32_t w1, float s) {
  const float x4[4] = {__uint_as_float(w0 << 16), __uint_as_float(w0 & 0xFFFF0000u),
                       __uint_as_float(w1 << 16), __uint_as_float(w1 & 0xFFFF0000u)};
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = fminf(fmaxf(__fdiv_rn(x4[j], s), -448.0f), 448.0f);
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0u, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w, true);
}

// s_x from the partials (each block recomputes it: every thread loads at most
// kAmaxMaxBlocks / kAmaxThreads of them, all at once), then the codes of x: n8 16-byte
// pieces, each stored as one 8-byte word; a thread's first two pieces are loaded
// before the partials, so they travel while the scale is formed.  x is read for the last
// time here, without cache allocation (at 8192 x 2048: 16.1 -> 13.4 us; the same loads in
// the amax kernel, whose reads this kernel follows, were slower).  |x / s| <= 448 up
// to the quotient's rounding; the clamp keeps the convert inside the finite range (it
// changes no value that rounds to a finite code).
__global__ __launch_bounds__(kAmaxThreads) void fp8_quantize_kernel(
    const uint4* __restrict__ x, size_t n8, const float* __restrict__ partial, int nparts,
    uint2* __restrict__ q, float* scale_out) {
  __shared__ float red[kAmaxThreads / kWave];
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  const size_t i0 = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  const uint4 a = i0 < n8 ? ldg16_nt(x + i0) : zero;
  const uint4 b = i0 + stride < n8 ? ldg16_nt(x + i0 + stride) : zero;
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < kAmaxMaxBlocks / kAmaxThreads; ++j) {
    const int k = threadIdx.x + j * kAmaxThreads;
    if (k < nparts) m = fmaxf(m, partial[k]);
  }
  m = __int_as_float(static_cast<int>(wave_max_u32(__float_as_uint(m))));
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  float mx = red[0];
#pragma unroll
  for (int w = 1; w < kAmaxThreads / kWave; ++w) mx = fmaxf(mx, red[w]);
  const float s = mx > 0.0f ? __fdiv_rn(mx, 448.0f) : 1.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
  if (i0 < n8) q[i0] = make_uint2(quant4(a.x, a.y, s), quant4(a.z, a.w, s));
  if (i0 + stride < n8) q[i0 + stride] = make_uint2(quant4(b.x, b.y, s), quant4(b.z, b.w, s));
  for (size_t i = i0 + 2 * stride; i < n8; i += stride) {
    const uint4 c = ldg16_nt(x + i);
    q[i] = make_uint2(quant4(c.x, c.y, s), quant4(c.z, c.w, s));
  }
}

// y[m, col0 + n] = bf16(acc * s_x * (row_scale ? row_scale[n] : scale)) for the M x N
// product of xq [M, K] with w [N, K]; ldy is y's row stride.
__global__ __launch_bounds__(4 * kWave) void fp8_gemm_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ w, int M, int N, int K,
    const float* __restrict__ s_x, const float* __restrict__ row_scale, float scale,
    uint16_t* __restrict__ y, int ldy, int col0) {
  __shared__ __align__(16) uint8_t As[kTile * kLdsRow];
  __shared__ __align__(16) uint8_t Bs[kTile * kLdsRow];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int m0 = blockIdx.y * kTile, n0 = blockIdx.x * kTile;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  // staging: thread t moves 16 bytes of row t / 4 of each tile
  const int sr = threadIdx.x >> 2, sk = (threadIdx.x & 3) * 16;
  const bool a_in = m0 + sr < M, b_in = n0 + sr < N;
  const uint8_t* ag = xq + static_cast<size_t>(a_in ? m0 + sr : 0) * K + sk;
  const uint8_t* bg = w + static_cast<size_t>(b_in ? n0 + sr : 0) * K + sk;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 an = a_in ? *reinterpret_cast<const u32x4*>(ag) : zero;
  u32x4 bn = b_in ? *reinterpret_cast<const u32x4*>(bg) : zero;
  for (int k0 = 0; k0 < K; k0 += kSlab) {
    __syncthreads();  // the previous slab's fragments have been read
    *reinterpret_cast<u32x4*>(&As[sr * kLdsRow + sk]) = an;
    *reinterpret_cast<u32x4*>(&Bs[sr * kLdsRow + sk]) = bn;
    __syncthreads();
    if (k0 + kSlab < K) {  // next slab's loads travel during this slab's MFMAs
      an = a_in ? *reinterpret_cast<const u32x4*>(ag + k0 + kSlab) : zero;
      bn = b_in ? *reinterpret_cast<const u32x4*>(bg + k0 + kSlab) : zero;
    }
#pragma unroll
    for (int ks = 0; ks < kSlab; ks += 32) {
      const int kk = ks + (lane >> 4) * 8;
      long a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const long*>(&As[(wm + 16 * i + (lane & 15)) * kLdsRow + kk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const long*>(&Bs[(wn + 16 * j + (lane & 15)) * kLdsRow + kk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  const float sx = *s_x;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn + 16 * j + (lane & 15);
    if (n >= N) continue;
    const float sn = sx * (row_scale ? row_scale[n] : scale);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm + 16 * i + 4 * (lane >> 4) + r;
        if (m < M) y[static_cast<size_t>(m) * ldy + col0 + n] = f32_to_bf16_bits(acc[i][j][r] * sn);
      }
  }
}

// Many activation rows: 128 x 128 output tiles per 4-wave block on gfx950's
// v_mfma_scale_f32_16x16x128_f8f6f4 (both operands e4m3, unit block scales: the
// scale operand 127 is 2^0 in E8M0), 128-deep K slabs staged in LDS (rows padded by
// 16 bytes: the 16 rows one read covers fall on 16 distinct bank quadruples), the
// next slab's global loads in flight during the current slab's MFMAs.  A wave owns a
// 64 x 64 quarter of the tile: 4 x 4 fragments, each MFMA lane (i, g) holding row /
// column i and K 32 g .. 32 g + 31 of the slab for A and B alike.  K % 64 == 0: a
// trailing half slab is read as zeros past K.
constexpr int kBig = 128;              // output rows and columns of a block
constexpr int kBigSlab = 128;          // K bytes per LDS slab
constexpr int kBigRow = kBigSlab + 16; // bytes per LDS row

typedef int v8i __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(4 * kWave, 2) void fp8_gemm_big_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ w, int M, int N, int K,
    const float* __restrict__ s_x, const float* __restrict__ row_scale, float scale,
    uint16_t* __restrict__ y, int ldy, int col0) {
  __shared__ __align__(16) uint8_t As[kBig * kBigRow];
  __shared__ __align__(16) uint8_t Bs[kBig * kBigRow];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int m0 = blockIdx.y * kBig, n0 = blockIdx.x * kBig;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  // staging: load j of thread t moves bytes 16 (t % 8) .. + 15 of tile row t / 8 + 32 j
  // (8 lanes cover one 128-byte row segment)
  const int sc = (tid & 7) * 16;
  const uint8_t* ag[4];
  const uint8_t* bg[4];
  bool ain[4], bin[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = (tid >> 3) + 32 * j;
    ain[j] = m0 + r < M;
    bin[j] = n0 + r < N;
    ag[j] = xq + static_cast<size_t>(ain[j] ? m0 + r : 0) * K + sc;
    bg[j] = w + static_cast<size_t>(bin[j] ? n0 + r : 0) * K + sc;
  }
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 an[4], bn[4];
  auto load = [&](int k0) {
    const bool kin = k0 + sc < K;  // K % 64 == 0: a 16-byte piece is wholly in or out
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      an[j] = (ain[j] && kin) ? *reinterpret_cast<const u32x4*>(ag[j] + k0) : zero;
      bn[j] = (bin[j] && kin) ? *reinterpret_cast<const u32x4*>(bg[j] + k0) : zero;
    }
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  load(0);
  for (int k0 = 0; k0 < K; k0 += kBigSlab) {
    __syncthreads();  // the previous slab's fragments have been read
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = (tid >> 3) + 32 * j;
      *reinterpret_cast<u32x4*>(&As[r * kBigRow + sc]) = an[j];
      *reinterpret_cast<u32x4*>(&Bs[r * kBigRow + sc]) = bn[j];
    }
    __syncthreads();
    if (k0 + kBigSlab < K) load(k0 + kBigSlab);  // travels during this slab's MFMAs
    v8i af[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) af[a] = *reinterpret_cast<const v8i*>(&As[(wm + 16 * a + i) * kBigRow + 32 * g]);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const v8i bf = *reinterpret_cast<const v8i*>(&Bs[(wn + 16 * b + i) * kBigRow + 32 * g]);
#pragma unroll
      for (int a = 0; a < 4; ++a)
        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[a], bf, acc[a][b], 0, 0, 0,
                                                                      127, 0, 127);
    }
  }
  // C lane l: column l % 16, rows 4 (l / 16) + r of each 16 x 16 fragment
  const float sx = *s_x;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int n = n0 + wn + 16 * b + i;
    if (n >= N) continue;
    const float sn = sx * (row_scale ? row_scale[n] : scale);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm + 16 * a + 4 * g + r;
        if (m < M) y[static_cast<size_t>(m) * ldy + col0 + n] = f32_to_bf16_bits(acc[a][b][r] * sn);
      }
  }
}

// Small activations: amax, s_x and the codes in one block of 1024 threads (the
// same arithmetic as the two kernels above).
constexpr int kSmallQuantThreads = 1024;
constexpr size_t kSmallQuantMax = 16384;  // M K handled by the one-block kernel

__global__ __launch_bounds__(kSmallQuantThreads) void fp8_quantize_small_kernel(
    const uint16_t* __restrict__ x, int n, uint8_t* __restrict__ q, float* scale_out) {
  __shared__ float red[kSmallQuantThreads / kWave];
  __shared__ float s_scale;
  float m = 0.0f;
  for (int i = threadIdx.x; i < n; i += kSmallQuantThreads) m = fmaxf(m, fabsf(bf16_at(x, i)));
  m = __int_as_float(static_cast<int>(wave_max_u32(__float_as_uint(m))));
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = red[0];
    for (int w = 1; w < kSmallQuantThreads / kWave; ++w) b = fmaxf(b, red[w]);
    const float sc = b > 0.0f ? __fdiv_rn(b, 448.0f) : 1.0f;
    s_scale = sc;
    *scale_out = sc;
  }
  __syncthreads();
  const float sc = s_scale;
  for (int i = 4 * threadIdx.x; i < n; i += 4 * kSmallQuantThreads) {  // n % 4 == 0
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float t = __fdiv_rn(bf16_at(x, i + j), sc);
      v[j] = fminf(fmaxf(t, -448.0f), 448.0f);
    }
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0u, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w, true);
    *reinterpret_cast<uint32_t*>(q + i) = w;
  }
}

// y[m, col0 + n] for M <= MM rows of activation codes: wave (block b, wave v) takes
// weight rows n0 .. n0 + 3 (n0 = 4 (4 b + v)); lane l takes the 16-byte K chunks
// l, l + 64, ... of each row (loaded for the 4 rows and the M activation rows, then
// multiplied); per (row, m) the lanes' sums are added over the wave.  Rows past N
// and chunks past K contribute nothing.
constexpr int kGemvRows = 4;
constexpr int kGemvMaxM = 8;
constexpr int kGemvChunks = 2;  // 16-byte K chunks per lane and pass (K 2048 per pass)

template <int MM>
__global__ __launch_bounds__(4 * kWave) void fp8_gemv_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ w, int M, int N, int K,
    const float* __restrict__ s_x, const float* __restrict__ row_scale, float scale,
    uint16_t* __restrict__ y, int ldy, int col0) {
  const int lane = threadIdx.x & (kWave - 1);
  const int n0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kGemvRows;
  if (n0 >= N) return;
  const int nch = K / 16;
  float acc[kGemvRows][MM];
#pragma unroll
  for (int r = 0; r < kGemvRows; ++r)
#pragma unroll
    for (int m = 0; m < MM; ++m) acc[r][m] = 0.0f;
  for (int c0 = 0; c0 < nch; c0 += kGemvChunks * kWave) {
    uint4 wv[kGemvRows][kGemvChunks], xv[MM][kGemvChunks];
    bool ok[kGemvChunks];
#pragma unroll
    for (int j = 0; j < kGemvChunks; ++j) {
      const int ci = c0 + j * kWave + lane;
      ok[j] = ci < nch;
      const int cc = ok[j] ? ci : nch - 1;  // in range; its terms are dropped below
#pragma unroll
      for (int r = 0; r < kGemvRows; ++r) {
        const int n = n0 + r < N ? n0 + r : N - 1;
        wv[r][j] = *reinterpret_cast<const uint4*>(w + static_cast<size_t>(n) * K + 16 * cc);
      }
#pragma unroll
      for (int m = 0; m < MM; ++m) {
        const int mm = m < M ? m : M - 1;
        xv[m][j] = *reinterpret_cast<const uint4*>(xq + static_cast<size_t>(mm) * K + 16 * cc);
      }
    }
#pragma unroll
    for (int j = 0; j < kGemvChunks; ++j) {
      if (!ok[j]) continue;
#pragma unroll
      for (int m = 0; m < MM; ++m) {
        bf16x2 xb[8];
        const uint32_t xw[4] = {xv[m][j].x, xv[m][j].y, xv[m][j].z, xv[m][j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          xb[2 * q] = e4m3x2_to_bf16<false>(xw[q]);
          xb[2 * q + 1] = e4m3x2_to_bf16<true>(xw[q]);
        }
#pragma unroll
        for (int r = 0; r < kGemvRows; ++r) {
          const uint32_t ww[4] = {wv[r][j].x, wv[r][j].y, wv[r][j].z, wv[r][j].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[r][m] = __builtin_amdgcn_fdot2_f32_bf16(e4m3x2_to_bf16<false>(ww[q]), xb[2 * q],
                                                        acc[r][m], false);
            acc[r][m] = __builtin_amdgcn_fdot2_f32_bf16(e4m3x2_to_bf16<true>(ww[q]), xb[2 * q + 1],
                                                        acc[r][m], false);
          }
        }
      }
    }
  }
  const float sx = *s_x;
#pragma unroll
  for (int r = 0; r < kGemvRows; ++r) {
    const int n = n0 + r;
    const float sn = sx * (row_scale ? row_scale[n < N ? n : N - 1] : scale);
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      const float v = group_sum_last<kWave>(acc[r][m]);  // in lane 63
      if (lane == kWave - 1 && n < N && m < M)
        y[static_cast<size_t>(m) * ldy + col0 + n] = f32_to_bf16_bits(v * sn);
    }
  }
}

// Few activation rows with all of x small (M <= kGemvMaxM, M K <= kSmallQuantMax, K <=
// kGemvChunks * kWave * 16: one pass): the quantisation and the GEMV in ONE launch.  Every
// block reads all of x, forms s_x and the codes of x itself with the arithmetic of the
// quantisation kernels (the same bits), keeps the codes in LDS, and multiplies as
// fp8_gemv_kernel does; its weight loads are issued first, so they travel meanwhile.
// Blocks of 8 waves; each wave takes kFusedRows weight rows (2, not 4: twice the waves, so
// more CUs share the stream), and the weights, read once per call, are loaded
// non-temporally (no cache allocation).  Measured on the 1-token q|k|v projection (K 2048,
// N 5120): 6.01 us per call with 4-wave blocks, 4 rows and plain loads; 5.59 with 2 rows,
// 5.65 with non-temporal loads, 5.30 with both (1 row and non-temporal loads: 5.60); 8-wave
// blocks (half the blocks reducing x) 5.18 against 5.23.
constexpr int kFusedRows = 2;

template <int MM>
__global__ __launch_bounds__(8 * kWave) void fp8_gemv_fused_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ w, int M, int N, int K,
    const float* __restrict__ row_scale, uint16_t* __restrict__ y, int ldy, int col0) {
  constexpr int kXP = kSmallQuantMax / 8 / (8 * kWave);  // 16-byte pieces of x per thread
  __shared__ __align__(16) uint8_t xs[kSmallQuantMax];   // codes of x, [M][K]
  __shared__ float red[8];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int n0 = (blockIdx.x * 8 + wave) * kFusedRows;  // may be >= N: the wave still
  const int nch = K / 16;                              // takes part in the barriers
  uint4 wv[kFusedRows][kGemvChunks];
  bool ok[kGemvChunks];
#pragma unroll
  for (int j = 0; j < kGemvChunks; ++j) {
    const int ci = j * kWave + lane;
    ok[j] = ci < nch;
    const int cc = ok[j] ? ci : nch - 1;  // in range; its terms are dropped below
#pragma unroll
    for (int r = 0; r < kFusedRows; ++r) {
      const int n = n0 + r < N ? n0 + r : N - 1;
      wv[r][j] = ldg16_nt(w + static_cast<size_t>(n) * K + 16 * cc);
    }
  }
  const int n8 = M * K / 8;  // K % 64 == 0
  uint4 xp[kXP];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < kXP; ++i) {
    const int pc = tid + 8 * kWave * i;
    xp[i] = pc < n8 ? reinterpret_cast<const uint4*>(x)[pc] : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int i = 0; i < kXP; ++i) m = absmax8(m, xp[i]);
  m = __int_as_float(static_cast<int>(wave_max_u32(__float_as_uint(m))));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  const float mx = fmaxf(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])), fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7])));
  const float sx = mx > 0.0f ? __fdiv_rn(mx, 448.0f) : 1.0f;
#pragma unroll
  for (int i = 0; i < kXP; ++i) {
    const int pc = tid + 8 * kWave * i;
    if (pc < n8)
      reinterpret_cast<uint2*>(xs)[pc] = make_uint2(quant4(xp[i].x, xp[i].y, sx), quant4(xp[i].z, xp[i].w, sx));
  }
  __syncthreads();
  float acc[kFusedRows][MM];
#pragma unroll
  for (int r = 0; r < kFusedRows; ++r)
#pragma unroll
    for (int mm = 0; mm < MM; ++mm) acc[r][mm] = 0.0f;
#pragma unroll
  for (int j = 0; j < kGemvChunks; ++j) {
    if (!ok[j]) continue;
    const int cc = j * kWave + lane;
#pragma unroll
    for (int mm = 0; mm < MM; ++mm) {
      const int mr = mm < M ? mm : M - 1;
      const uint4 xv = *reinterpret_cast<const uint4*>(xs + mr * K + 16 * cc);
      bf16x2 xb[8];
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xb[2 * q] = e4m3x2_to_bf16<false>(xw[q]);
        xb[2 * q + 1] = e4m3x2_to_bf16<true>(xw[q]);
      }
#pragma unroll
      for (int r = 0; r < kFusedRows; ++r) {
        const uint32_t ww[4] = {wv[r][j].x, wv[r][j].y, wv[r][j].z, wv[r][j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[r][mm] = __builtin_amdgcn_fdot2_f32_bf16(e4m3x2_to_bf16<false>(ww[q]), xb[2 * q],
                                                       acc[r][mm], false);
          acc[r][mm] = __builtin_amdgcn_fdot2_f32_bf16(e4m3x2_to_bf16<true>(ww[q]), xb[2 * q + 1],
                                                       acc[r][mm], false);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kFusedRows; ++r) {
    const int n = n0 + r;
    const float sn = sx * row_scale[n < N ? n : N - 1];
#pragma unroll
    for (int mm = 0; mm < MM; ++mm) {
      const float v = group_sum_last<kWave>(acc[r][mm]);  // in lane 63
      if (lane == kWave - 1 && n < N && mm < M)
        y[static_cast<size_t>(mm) * ldy + col0 + n] = f32_to_bf16_bits(v * sn);
    }
  }
}

int amax_blocks(size_t n) {
  const size_t b = (n + kAmaxThreads * 16 - 1) / (kAmaxThreads * 16);
  return static_cast<int>(b < 1 ? 1 : (b > kAmaxMaxBlocks ? kAmaxMaxBlocks : b));
}

}  // namespace

size_t fp8_linear_workspace(int64_t M, int64_t K) {
  const size_t n = static_cast<size_t>(M) * K;
  return align256(n) + align256(kAmaxMaxBlocks * sizeof(float)) + 256;
}

hipError_t launch_fp8_quantize(const uint16_t* x, int64_t M, int64_t K, void* ws, uint8_t** xq,
                               float** s_x, hipStream_t s) {
  const size_t n = static_cast<size_t>(M) * K;
  uint8_t* base = static_cast<uint8_t*>(ws);
  *xq = base;
  float* partial = reinterpret_cast<float*>(base + align256(n));
  *s_x = reinterpret_cast<float*>(base + align256(n) + align256(kAmaxMaxBlocks * sizeof(float)));
  if (n <= kSmallQuantMax) {
    fp8_quantize_small_kernel<<<dim3(1), dim3(kSmallQuantThreads), 0, s>>>(x, static_cast<int>(n),
                                                                            *xq, *s_x);
    return hipGetLastError();
  }
  // x is 16-byte aligned and n = M K with K % 64 == 0 (checked by the caller)
  const int nb = amax_blocks(n);
  const size_t n8 = n / 8;
  fp8_amax_kernel<<<dim3(nb), dim3(kAmaxThreads), 0, s>>>(reinterpret_cast<const uint4*>(x), n8,
                                                          partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t qb = (n8 + 2 * kAmaxThreads - 1) / (2 * kAmaxThreads);
  fp8_quantize_kernel<<<dim3(static_cast<unsigned>(qb < 4096 ? qb : 4096)), dim3(kAmaxThreads), 0,
                        s>>>(reinterpret_cast<const uint4*>(x), n8, partial, nb,
                             reinterpret_cast<uint2*>(*xq), *s_x);
  return hipGetLastError();
}

bool fp8_linear_fused_fits(int64_t M, int64_t K) {
  return M >= 1 && M <= kGemvMaxM && static_cast<size_t>(M * K) <= kSmallQuantMax &&
         K <= kGemvChunks * kWave * 16;
}

hipError_t launch_fp8_linear_fused(const uint16_t* x, const uint8_t* w, int M, int N, int K,
                                   const float* row_scale, uint16_t* y, int ldy, int col0,
                                   hipStream_t s) {
  if (!fp8_linear_fused_fits(M, K) || !row_scale) return hipErrorInvalidValue;
  if (N <= 0) return hipSuccess;
  const dim3 g((N + 8 * kFusedRows - 1) / (8 * kFusedRows)), b(8 * kWave);
  if (M == 1) fp8_gemv_fused_kernel<1><<<g, b, 0, s>>>(x, w, M, N, K, row_scale, y, ldy, col0);
  else if (M == 2) fp8_gemv_fused_kernel<2><<<g, b, 0, s>>>(x, w, M, N, K, row_scale, y, ldy, col0);
  else if (M <= 4) fp8_gemv_fused_kernel<4><<<g, b, 0, s>>>(x, w, M, N, K, row_scale, y, ldy, col0);
  else fp8_gemv_fused_kernel<8><<<g, b, 0, s>>>(x, w, M, N, K, row_scale, y, ldy, col0);
  return hipGetLastError();
}

hipError_t launch_fp8_gemm(const uint8_t* xq, const uint8_t* w, int M, int N, int K,
                           const float* s_x, const float* row_scale, float scale, uint16_t* y,
                           int ldy, int col0, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (M <= kGemvMaxM) {
    const dim3 g((N + 4 * kGemvRows - 1) / (4 * kGemvRows)), b(4 * kWave);
    if (M == 1) fp8_gemv_kernel<1><<<g, b, 0, s>>>(xq, w, M, N, K, s_x, row_scale, scale, y, ldy, col0);
    else if (M == 2) fp8_gemv_kernel<2><<<g, b, 0, s>>>(xq, w, M, N, K, s_x, row_scale, scale, y, ldy, col0);
    else if (M <= 4) fp8_gemv_kernel<4><<<g, b, 0, s>>>(xq, w, M, N, K, s_x, row_scale, scale, y, ldy, col0);
    else fp8_gemv_kernel<8><<<g, b, 0, s>>>(xq, w, M, N, K, s_x, row_scale, scale, y, ldy, col0);
    return hipGetLastError();
  }
  if (M >= kBig) {
    const dim3 grid((N + kBig - 1) / kBig, (M + kBig - 1) / kBig);
    fp8_gemm_big_kernel<<<grid, dim3(4 * kWave), 0, s>>>(xq, w, M, N, K, s_x, row_scale, scale, y,
                                                         ldy, col0);
    return hipGetLastError();
  }
  const dim3 grid((N + kTile - 1) / kTile, (M + kTile - 1) / kTile);
  fp8_gemm_kernel<<<grid, dim3(4 * kWave), 0, s>>>(xq, w, M, N, K, s_x, row_scale, scale, y, ldy,
                                                   col0);
  return hipGetLastError();
}

}  // namespace ftmoe
