// repack.hip -- load-time NVFP4 layout conversion and the dequantisation test
// export, gfx950.
//
// FreeToken fork PR #84 (page 1), bullet on #631 (the decode GEMV stops converting
// its weight layout on the fly): the decode GEMV reads weights already arranged for it,
// so the conversion happens once, when the weights are loaded.  The gate|up
// tensors are already in the order the gate|up GEMV reads (row-major, 16-byte
// chunks per lane); the down tensors are moved to K-chunk-major order so that 64
// lanes owning 64 consecutive output rows read 1 KiB contiguous per load.
#include "ftmoe_device.hpp"
#include "ftmoe_kernels.hpp"

namespace ftmoe {

// canonical w2 codes [n][H][I/2] -> [n][I/32][H][16]; scales [n][H][I/16] -> [n][I/32][H][2]
__global__ __launch_bounds__(256) void repack_w2_kernel(int H, int I, int n,
                                                        const uint8_t* __restrict__ w2,
                                                        const uint8_t* __restrict__ w2s,
                                                        uint8_t* __restrict__ out_w2,
                                                        uint8_t* __restrict__ out_w2s) {
  const int nch = I / 32;
  const size_t total = static_cast<size_t>(n) * H * nch;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    // destination order: (e, j, c)
    const size_t c = i % H;
    const size_t j = (i / H) % nch;
    const size_t e = i / (static_cast<size_t>(H) * nch);
    const size_t src_row = e * H + c;
    const uint4 q = *reinterpret_cast<const uint4*>(w2 + src_row * (I / 2) + 16 * j);
    *reinterpret_cast<uint4*>(out_w2 + i * 16) = q;
    const uint8_t* ss = w2s + src_row * (I / 16) + 2 * j;
    out_w2s[i * 2 + 0] = ss[0];
    out_w2s[i * 2 + 1] = ss[1];
  }
}

// block-fp8 down codes: canonical [n][H][I] -> [n][I/32][H][32] (32 e4m3 bytes of one
// row's K-chunk per record, so 64 lanes owning 64 consecutive rows read 2 KiB contiguous)
__global__ __launch_bounds__(256) void repack_fp8_w2_kernel(int H, int I, int n,
                                                            const uint8_t* __restrict__ w2,
                                                            uint8_t* __restrict__ out_w2) {
  const int nch = I / 32;
  const size_t total = static_cast<size_t>(n) * H * nch;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const size_t c = i % H;
    const size_t j = (i / H) % nch;
    const size_t e = i / (static_cast<size_t>(H) * nch);
    const uint4* src = reinterpret_cast<const uint4*>(w2 + (e * H + c) * I + 32 * j);
    uint4* dst = reinterpret_cast<uint4*>(out_w2 + i * 32);
    dst[0] = src[0];
    dst[1] = src[1];
  }
}

hipError_t launch_repack_fp8_w2(int H, int I, int n, const uint8_t* w2, uint8_t* out_w2,
                                hipStream_t s) {
  const size_t total = static_cast<size_t>(n) * H * (I / 32);
  if (total == 0) return hipSuccess;
  size_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  repack_fp8_w2_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(H, I, n, w2,
                                                                                out_w2);
  return hipGetLastError();
}

// Dequantise one tensor of one block-fp8 expert (repacked bank) to fp32 [rows][K]
// with the routines the one-launch decode kernel uses: mode 0 decodes the codes as
// its down GEMV does (e4m3 pair -> fp32 pair), mode 1 as its gate|up GEMV does
// (e4m3 pair -> bf16 pair); both then multiply by the block scale (one rounding).
__global__ __launch_bounds__(256) void fp8_dequant_kernel(int H, int I, Bank b, int e,
                                                          int tensor, int mode, float* out) {
  const bool down = (tensor == 2);
  const int rows = down ? H : I;
  const int K = down ? I : H;
  const size_t total = static_cast<size_t>(rows) * (K / 4);
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int r = static_cast<int>(idx / (K / 4));
  const int k0 = 4 * static_cast<int>(idx % (K / 4));
  uint32_t word;
  float scale;
  const float* sc13 = reinterpret_cast<const float*>(b.w13s);
  const float* sc2 = reinterpret_cast<const float*>(b.w2s);
  if (!down) {
    const size_t row = static_cast<size_t>(tensor == 1 ? I : 0) + r;
    word = *reinterpret_cast<const uint32_t*>(b.w13 + (static_cast<size_t>(e) * 2 * I + row) * H + k0);
    scale = sc13[(static_cast<size_t>(e) * (2 * I / 128) + row / 128) * (H / 128) + k0 / 128];
  } else {
    const size_t rec = (static_cast<size_t>(e) * (I / 32) + k0 / 32) * H + r;
    word = *reinterpret_cast<const uint32_t*>(b.w2 + rec * 32 + (k0 % 32));
    scale = sc2[(static_cast<size_t>(e) * (H / 128) + r / 128) * (I / 128) + k0 / 128];
  }
  float v[4];
  if (mode == 1) {
    const bf16x2 lo = e4m3x2_to_bf16<false>(word), hi = e4m3x2_to_bf16<true>(word);
    v[0] = static_cast<float>(lo[0]);
    v[1] = static_cast<float>(lo[1]);
    v[2] = static_cast<float>(hi[0]);
    v[3] = static_cast<float>(hi[1]);
  } else {
    const f32x2 lo = e4m3x2_to_f32<false>(word), hi = e4m3x2_to_f32<true>(word);
    v[0] = lo.x;
    v[1] = lo.y;
    v[2] = hi.x;
    v[3] = hi.y;
  }
  float* o = out + static_cast<size_t>(r) * K + k0;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = v[i] * scale;
}

hipError_t launch_fp8_dequant(int H, int I, const Bank& b, int expert, int tensor, int mode,
                              float* out, hipStream_t s) {
  const size_t total = static_cast<size_t>(H) * I / 4;
  fp8_dequant_kernel<<<dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s>>>(
      H, I, b, expert, tensor, mode, out);
  return hipGetLastError();
}

hipError_t launch_repack_w2(int H, int I, int n, const uint8_t* w2, const uint8_t* w2s,
                            uint8_t* out_w2, uint8_t* out_w2s, hipStream_t s) {
  const size_t total = static_cast<size_t>(n) * H * (I / 32);
  if (total == 0) return hipSuccess;
  size_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  repack_w2_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(H, I, n, w2, w2s,
                                                                            out_w2, out_w2s);
  return hipGetLastError();
}

// Dequantise one tensor of one expert of a repacked bank.  Each thread decodes
// one 32-bit word of codes (8 elements, inside one 16-element scale block) with
// the routines the compute kernels use, chosen by out_dtype (out: row-major
// [rows][K]):
//   0  fp32 code x scale x global, codes through e2m1x2_to_f32 (the down GEMV of
//      the one-launch decode kernel);
//   1  the same value rounded to bf16 (nearest-even);
//   2  bf16 code x scale, no global scale, as the grouped and prefill kernels build
//      their MFMA tiles (dequant8_bf16);
//   3  fp32 code x scale x global with the codes through e2m1x2_to_bf16 (the
//      gate|up GEMV of the one-launch decode kernel, which multiplies those bf16
//      codes with the activations and applies the scale per 16-element block);
//   4  fp16 code x scale, no global scale, as the down GEMMs of the grouped and
//      prefill kernels build their fp16 tiles (dequant8_tile<true>).
__global__ __launch_bounds__(256) void dequant_kernel(int H, int I, Bank b, int e, int tensor,
                                                      int out_dtype, void* out) {
  const bool down = (tensor == 2);
  const int rows = down ? H : I;
  const int K = down ? I : H;
  const int words_per_row = K / 8;
  const size_t total = static_cast<size_t>(rows) * words_per_row;
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int r = static_cast<int>(idx / words_per_row);
  const int wd = static_cast<int>(idx % words_per_row);
  const int k0 = 8 * wd;  // first element of the word
  uint32_t code_word, scale_byte;
  if (!down) {
    const size_t row = static_cast<size_t>(e) * 2 * I + (tensor == 1 ? I : 0) + r;
    code_word = *reinterpret_cast<const uint32_t*>(b.w13 + row * (H / 2) + 4 * wd);
    scale_byte = b.w13s[row * (H / 16) + k0 / 16];
  } else {
    const int nch = I / 32;
    const int j = k0 / 32;
    const size_t rec = (static_cast<size_t>(e) * nch + j) * H + r;
    code_word = *reinterpret_cast<const uint32_t*>(b.w2 + rec * 16 + (k0 % 32) / 2);
    scale_byte = b.w2s[rec * 2 + (k0 % 32) / 16];
  }
  const float s = e4m3_byte_to_f32<0>(scale_byte);
  const float g = b.gsc[3 * e + tensor];
  const size_t o = static_cast<size_t>(r) * K + k0;
  if (out_dtype == 2 || out_dtype == 4) {
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + o) =
        out_dtype == 2 ? dequant8_tile<false>(code_word, s) : dequant8_tile<true>(code_word, s);
    return;
  }
  float v[8];
  if (out_dtype == 3) {
    const bf16x2 c[4] = {e2m1x2_to_bf16<0>(code_word), e2m1x2_to_bf16<1>(code_word),
                         e2m1x2_to_bf16<2>(code_word), e2m1x2_to_bf16<3>(code_word)};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = dequant_one(static_cast<float>(c[i][0]), s, g);
      v[2 * i + 1] = dequant_one(static_cast<float>(c[i][1]), s, g);
    }
  } else {
    const f32x2 p0 = e2m1x2_to_f32<0>(code_word), p1 = e2m1x2_to_f32<1>(code_word);
    const f32x2 p2 = e2m1x2_to_f32<2>(code_word), p3 = e2m1x2_to_f32<3>(code_word);
    v[0] = dequant_one(p0.x, s, g);
    v[1] = dequant_one(p0.y, s, g);
    v[2] = dequant_one(p1.x, s, g);
    v[3] = dequant_one(p1.y, s, g);
    v[4] = dequant_one(p2.x, s, g);
    v[5] = dequant_one(p2.y, s, g);
    v[6] = dequant_one(p3.x, s, g);
    v[7] = dequant_one(p3.y, s, g);
  }
  if (out_dtype == 1) {
    uint16_t* ob = static_cast<uint16_t*>(out) + o;
#pragma unroll
    for (int i = 0; i < 8; ++i) ob[i] = f32_to_bf16_bits(v[i]);
  } else {
    float* of = static_cast<float*>(out) + o;
#pragma unroll
    for (int i = 0; i < 8; ++i) of[i] = v[i];
  }
}

hipError_t launch_dequant(int H, int I, const Bank& b, int expert, int tensor, int out_dtype,
                          void* out, hipStream_t s) {
  const size_t total = static_cast<size_t>(H) * I / 8;
  const unsigned blocks = static_cast<unsigned>((total + 255) / 256);
  dequant_kernel<<<dim3(blocks), dim3(256), 0, s>>>(H, I, b, expert, tensor, out_dtype, out);
  return hipGetLastError();
}

}  // namespace ftmoe
