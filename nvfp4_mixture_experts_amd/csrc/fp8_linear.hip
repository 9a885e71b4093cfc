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
// itself, so there is no atomic and nothing to reset between calls); the GEMM on
// v_mfma_f32_16x16x32_fp8_fp8, 64 x 64 output tiles per 4-wave block, 64-deep K slabs
// staged in LDS.
#include "ftmoe_device.hpp"
#include "ftmoe_kernels.hpp"

namespace ftmoe {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kAmaxThreads = 256;
constexpr int kTile = 64;       // output rows and columns of a block
constexpr int kSlab = 64;       // K elements per LDS slab
constexpr int kLdsRow = kSlab + 16;  // bytes per LDS row (16 bytes of padding)

__device__ __forceinline__ float bf16_at(const uint16_t* x, size_t i) {
  return bf16_bits_to_f32(x[i]);
}

__global__ __launch_bounds__(kAmaxThreads) void fp8_amax_kernel(const uint16_t* __restrict__ x,
                                                                size_t n, float* partial) {
  __shared__ float red[kAmaxThreads / kWave];
  float m = 0.0f;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    m = fmaxf(m, fabsf(bf16_at(x, i)));
  // max is order-independent: the result does not depend on timing
  m = __int_as_float(static_cast<int>(wave_max_u32(__float_as_uint(m))));
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = red[0];
    for (int w = 1; w < kAmaxThreads / kWave; ++w) b = fmaxf(b, red[w]);
    partial[blockIdx.x] = b;
  }
}

// s_x from the partials (each block recomputes it), then codes of x.
__global__ __launch_bounds__(kAmaxThreads) void fp8_quantize_kernel(
    const uint16_t* __restrict__ x, size_t n, const float* __restrict__ partial, int nparts,
    uint8_t* __restrict__ q, float* scale_out) {
  __shared__ float s_scale;
  if (threadIdx.x < kWave) {
    float m = 0.0f;
    for (int i = threadIdx.x; i < nparts; i += kWave) m = fmaxf(m, partial[i]);
    m = __int_as_float(static_cast<int>(wave_max_u32(__float_as_uint(m))));
    if (threadIdx.x == 0) {
      const float s = m > 0.0f ? __fdiv_rn(m, 448.0f) : 1.0f;
      s_scale = s;
      if (blockIdx.x == 0) *scale_out = s;
    }
  }
  __syncthreads();
  const float s = s_scale;
  // four elements per thread and step (n % 4 == 0)
  for (size_t i = 4 * (static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x); i < n;
       i += 4 * static_cast<size_t>(gridDim.x) * blockDim.x) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // |x / s| <= 448 up to the quotient's rounding; the clamp keeps the convert
      // inside the finite range (it changes no value that rounds to a finite code)
      const float t = __fdiv_rn(bf16_at(x, i + j), s);
      v[j] = fminf(fmaxf(t, -448.0f), 448.0f);
    }
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0u, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w, true);
    *reinterpret_cast<uint32_t*>(q + i) = w;
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
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  uint4 an = a_in ? *reinterpret_cast<const uint4*>(ag) : zero;
  uint4 bn = b_in ? *reinterpret_cast<const uint4*>(bg) : zero;
  for (int k0 = 0; k0 < K; k0 += kSlab) {
    __syncthreads();  // the previous slab's fragments have been read
    *reinterpret_cast<uint4*>(&As[sr * kLdsRow + sk]) = an;
    *reinterpret_cast<uint4*>(&Bs[sr * kLdsRow + sk]) = bn;
    __syncthreads();
    if (k0 + kSlab < K) {  // next slab's loads travel during this slab's MFMAs
      an = a_in ? *reinterpret_cast<const uint4*>(ag + k0 + kSlab) : zero;
      bn = b_in ? *reinterpret_cast<const uint4*>(bg + k0 + kSlab) : zero;
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

int amax_blocks(size_t n) {
  const size_t b = (n + kAmaxThreads * 16 - 1) / (kAmaxThreads * 16);
  return static_cast<int>(b < 1 ? 1 : (b > 1024 ? 1024 : b));
}

}  // namespace

size_t fp8_linear_workspace(int64_t M, int64_t K) {
  const size_t n = static_cast<size_t>(M) * K;
  return align256(n) + align256(1024 * sizeof(float)) + 256;
}

hipError_t launch_fp8_quantize(const uint16_t* x, int64_t M, int64_t K, void* ws, uint8_t** xq,
                               float** s_x, hipStream_t s) {
  const size_t n = static_cast<size_t>(M) * K;
  uint8_t* base = static_cast<uint8_t*>(ws);
  *xq = base;
  float* partial = reinterpret_cast<float*>(base + align256(n));
  *s_x = reinterpret_cast<float*>(base + align256(n) + align256(1024 * sizeof(float)));
  const int nb = amax_blocks(n);
  fp8_amax_kernel<<<dim3(nb), dim3(kAmaxThreads), 0, s>>>(x, n, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t qb = (n / 4 + kAmaxThreads - 1) / kAmaxThreads;
  fp8_quantize_kernel<<<dim3(static_cast<unsigned>(qb < 2048 ? qb : 2048)), dim3(kAmaxThreads), 0,
                        s>>>(x, n, partial, nb, *xq, *s_x);
  return hipGetLastError();
}

hipError_t launch_fp8_gemm(const uint8_t* xq, const uint8_t* w, int M, int N, int K,
                           const float* s_x, const float* row_scale, float scale, uint16_t* y,
                           int ldy, int col0, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const dim3 grid((N + kTile - 1) / kTile, (M + kTile - 1) / kTile);
  fp8_gemm_kernel<<<grid, dim3(4 * kWave), 0, s>>>(xq, w, M, N, K, s_x, row_scale, scale, y, ldy,
                                                   col0);
  return hipGetLastError();
}

}  // namespace ftmoe
