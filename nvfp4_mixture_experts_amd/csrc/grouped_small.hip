// grouped_small.hip -- the expert GEMMs of the grouped path for few tokens per
// expert (decode batches of up to 64 tokens): every selected expert's weights
// are read once and applied to all of the tokens routed to it.
//
// FreeToken fork PR #84 (page 1), bullet on #631: the NVFP4 MoE decode GEMV;
// FreeToken commit log (page 2): clamped SwiGLU, 512 routed experts with top-10
// plus a gated shared expert.
//
// A wave owns 16 weight rows (gate|up: 16 gate rows and the 16 matching up rows).
// Per K block of 512 it issues the token-row loads for the LDS staging, then every
// code and scale load of its rows at once into registers (no prefetch ring carried
// across loop iterations, so nothing waits on a load in flight but the data it
// needs), then walks the block, dequantising 8 weights per lane per step into an
// exact bf16 A operand (code x e4m3 scale) for v_mfma_f32_16x16x32_bf16 while the
// later codes are still arriving.  The unit's token rows (B operand) are staged in
// LDS, 16 tokens at a time, shared by the block's 4 waves.  The MFMA does every
// token's products, so the VALU only dequantises (about 2 instructions per weight
// per 64 lanes).  The block is small in registers (about 100 per lane) so that 4
// waves share each SIMD: with few tokens the time is the weight stream, and it is
// the number of waves with loads in flight that sets its rate.
//
// K mapping: a lane loads the 16 code bytes of chunk 4q + g of its row (32 K
// elements; g = lane / 16) and feeds word j of it to step (q, j); the B operand of
// lane (token n, g) in step (q, j) is x[n][32 (4q + g) + 8 j .. + 8].  Which K a
// lane group holds only has to agree between A and B.
//
//   sg_gateup_kernel  h = SwiGLU(gate . x, up . x), stored as a bf16 (hi, lo) pair
//   sg_down_kernel    out[t][slot][row] = (W_down (h_hi + h_lo)) * g_down * weight
#include "ftmoe_device.hpp"
#include "ftmoe_kernels.hpp"

namespace ftmoe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 sg_bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float sg_f32x4;

namespace {

constexpr int kSgWaves = 4;
constexpr int kSgThreads = kSgWaves * kWave;
constexpr int kSgKBlock = 512;  // K elements of a row held in registers at once
constexpr int kSgQ = kSgKBlock / 128;  // 16-byte code loads per lane per row and K block

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ sg_f32x4 mfma(uint4 a, uint4 b, sg_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(sg_bf16x8, a),
                                                 __builtin_bit_cast(sg_bf16x8, b), c, 0, 0, 0);
}

// 8 codes x one e4m3 scale -> 8 bf16 (exact: the upper half of each fp32 product).
__device__ __forceinline__ uint32_t hi16x2(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
__device__ __forceinline__ uint4 dq8(uint32_t codes, float s) {
  const f32x2 a = e2m1x2_to_f32<0>(codes), b = e2m1x2_to_f32<1>(codes);
  const f32x2 c = e2m1x2_to_f32<2>(codes), d = e2m1x2_to_f32<3>(codes);
  uint4 r;
  r.x = hi16x2(a.x * s, a.y * s);
  r.y = hi16x2(b.x * s, b.y * s);
  r.z = hi16x2(c.x * s, c.y * s);
  r.w = hi16x2(d.x * s, d.y * s);
  return r;
}
__device__ __forceinline__ uint32_t word(const uint4& q, int j) {
  return j == 0 ? q.x : (j == 1 ? q.y : (j == 2 ? q.z : q.w));
}

__device__ __forceinline__ void sg_unit_tile(int ntiles, int* u, int* tile) {
  const int b = blockIdx.x;
  *u = (b / (8 * ntiles)) * 8 + (b & 7);
  *tile = (b >> 3) % ntiles;
}

}  // namespace

// Block: 64 h columns (4 waves x 16) of one unit; LDS: 16 token rows of K block.
__global__ __launch_bounds__(kSgThreads, 2) void sg_gateup_kernel(PrefillParams p) {
  constexpr int kRowU4 = kSgKBlock / 8 + 1;  // 16-byte words per staged token row (+1 pad)
  __shared__ uint4 xs[16 * kRowU4];
  int u, tile;
  sg_unit_tile(p.ntiles1, &u, &tile);
  if (u >= *p.nunits) return;
  const PfUnit un = p.units[u];
  const Bank bank = un.bank ? p.shared : p.routed;
  const int I = bank.inter;
  const int n0 = tile * 64;
  if (n0 >= I) return;
  const int H = p.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, g = lane >> 4;
  const int grow = n0 + wave * 16 + i;  // gate row; up row I + grow
  const size_t ebase = static_cast<size_t>(un.expert) * 2 * I;
  const uint8_t* gc = bank.w13 + (ebase + grow) * (H / 2);
  const uint8_t* uc = bank.w13 + (ebase + I + grow) * (H / 2);
  const uint8_t* gsp = bank.w13s + (ebase + grow) * (H / 16);
  const uint8_t* usp = bank.w13s + (ebase + I + grow) * (H / 16);
  const float gg = bank.gsc[un.expert * 3 + 0], gu = bank.gsc[un.expert * 3 + 1];
  for (int f0 = 0; f0 < un.count; f0 += 16) {
    sg_f32x4 ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < H; k0 += kSgKBlock) {
      const int kb = min(kSgKBlock, H - k0);  // a multiple of 256
      const int nq = kb / 128;
      // token rows f0 .. f0+15 of this K block (rows past the unit repeat its last
      // token), 16 bytes per load, into LDS
      // (a fixed number of loads per thread, indices clamped: every load is issued
      // before the first store)
      uint4 xv[16 * (kSgKBlock / 8) / kSgThreads];
#pragma unroll
      for (int r = 0; r < 16 * (kSgKBlock / 8) / kSgThreads; ++r) {
        const int v = min(tid + r * kSgThreads, 16 * (kb / 8) - 1);
        const int n = v / (kb / 8), c8 = v - n * (kb / 8);
        const int m = min(f0 + n, un.count - 1);
        const int t = un.bank ? un.start + m : p.sorted[un.start + m] / p.k;
        xv[r] = ldg16(p.x + static_cast<size_t>(t) * H + k0 + 8 * c8);
      }
      __builtin_amdgcn_sched_barrier(0);  // token rows first (the staging waits for them)
      // then this K block's codes and scales of the wave's 32 rows, all issued at
      // once: the K steps below wait only for their own codes, so the MFMAs run as
      // the later codes arrive
      uint4 qg[kSgQ], qu[kSgQ];
      uint32_t sg[kSgQ], su[kSgQ];
#pragma unroll
      for (int q = 0; q < kSgQ; ++q) {
        const int qq = q < nq ? q : nq - 1;
        const int ch = k0 / 32 + 4 * qq + g;  // chunk of 32 K along the row
        qg[q] = ldg16(gc + ch * 16);
        qu[q] = ldg16(uc + ch * 16);
        sg[q] = *reinterpret_cast<const uint16_t*>(gsp + ch * 2);
        su[q] = *reinterpret_cast<const uint16_t*>(usp + ch * 2);
      }
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();  // the previous block / fragment is done with xs
#pragma unroll
      for (int r = 0; r < 16 * (kSgKBlock / 8) / kSgThreads; ++r) {
        const int v = min(tid + r * kSgThreads, 16 * (kb / 8) - 1);
        const int n = v / (kb / 8), c8 = v - n * (kb / 8);
        xs[n * kRowU4 + c8] = xv[r];
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kSgQ; ++q) {
        if (q < nq) {
          const float g0 = e4m3_byte_to_f32<0>(sg[q]), g1 = e4m3_byte_to_f32<1>(sg[q]);
          const float u0 = e4m3_byte_to_f32<0>(su[q]), u1 = e4m3_byte_to_f32<1>(su[q]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint4 b = xs[i * kRowU4 + (4 * q + g) * 4 + j];
            ag = mfma(dq8(word(qg[q], j), j < 2 ? g0 : g1), b, ag);
            au = mfma(dq8(word(qu[q], j), j < 2 ? u0 : u1), b, au);
          }
        }
      }
    }
    // C lane l: rows 4 (l / 16) + jj (h columns), token l % 16 of the fragment
    const int m = f0 + i;
    if (m < un.count) {
      const int t = un.bank ? un.start + m : 0;
      const size_t row = un.bank ? static_cast<size_t>(p.P) + t : static_cast<size_t>(un.start) + m;
      const int col = n0 + wave * 16 + 4 * g;
      uint32_t hi[2], lo[2];
#pragma unroll
      for (int jj = 0; jj < 4; jj += 2) {
        float hv[2];
#pragma unroll
        for (int e = 0; e < 2; ++e)
          hv[e] = swiglu(p.act, ag[jj + e] * gg, au[jj + e] * gu, p.gate_max, p.up_absmax);
        const uint32_t h0 = f32_to_bf16_bits(hv[0]), h1 = f32_to_bf16_bits(hv[1]);
        const uint32_t l0 = f32_to_bf16_bits(hv[0] - bf16_bits_to_f32(h0));
        const uint32_t l1 = f32_to_bf16_bits(hv[1] - bf16_bits_to_f32(h1));
        hi[jj >> 1] = h0 | (h1 << 16);
        lo[jj >> 1] = l0 | (l1 << 16);
      }
      *reinterpret_cast<uint2*>(p.hhi + row * p.Imax + col) = make_uint2(hi[0], hi[1]);
      *reinterpret_cast<uint2*>(p.hlo + row * p.Imax + col) = make_uint2(lo[0], lo[1]);
    }
  }
}

// Block: 64 output rows (4 waves x 16) of one unit; LDS: 16 tokens' h (hi and lo)
// for a K block of up to 1024.
__global__ __launch_bounds__(kSgThreads, 2) void sg_down_kernel(PrefillParams p) {
  constexpr int kKB = 512;
  constexpr int kQ = kKB / 128;
  constexpr int kRowU4 = kKB / 8 + 1;
  __shared__ uint4 hs[2][16 * kRowU4];
  int u, tile;
  sg_unit_tile(p.ntiles2, &u, &tile);
  if (u >= *p.nunits) return;
  const PfUnit un = p.units[u];
  const Bank bank = un.bank ? p.shared : p.routed;
  const int I = bank.inter;
  const int H = p.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, g = lane >> 4;
  const int row = tile * 64 + wave * 16 + i;  // H % 256 == 0: always < H
  const size_t cbase = static_cast<size_t>(un.expert) * (I / 32);
  const float gd = bank.gsc[un.expert * 3 + 2];
  for (int f0 = 0; f0 < un.count; f0 += 16) {
    sg_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < I; k0 += kKB) {
      const int kb = min(kKB, I - k0);  // a multiple of 64
      const int nq = kb / 128;
      const int nhalf = (kb % 128) ? 1 : 0;  // a trailing 64-K piece: chunks 4 nq + {0, 1}
      constexpr int kLoads = 2 * 16 * (kKB / 8) / kSgThreads;
      uint4 hv[kLoads];
#pragma unroll
      for (int r = 0; r < kLoads; ++r) {
        const int v = min(tid + r * kSgThreads, 2 * 16 * (kb / 8) - 1);
        const int which = v / (16 * (kb / 8));
        const int rr = v - which * 16 * (kb / 8);
        const int n = rr / (kb / 8), c8 = rr - n * (kb / 8);
        const int m = min(f0 + n, un.count - 1);
        const size_t hrow = un.bank ? static_cast<size_t>(p.P) + un.start + m
                                    : static_cast<size_t>(un.start) + m;
        const uint16_t* src = which ? p.hlo : p.hhi;
        hv[r] = ldg16(src + hrow * p.Imax + k0 + 8 * c8);
      }
      __builtin_amdgcn_sched_barrier(0);  // h first (the staging waits for it), then codes
      uint4 q[kQ + 1];
      uint32_t sc[kQ + 1];
#pragma unroll
      for (int s = 0; s <= kQ; ++s) {
        // chunk 4 s + g of the K block; past the block's chunks repeat its last one
        const int nch = kb / 32;
        const int ch = min(4 * s + g, nch - 1);
        const size_t c = cbase + k0 / 32 + ch;
        q[s] = ldg16(bank.w2 + (c * H + row) * 16);
        sc[s] = *reinterpret_cast<const uint16_t*>(bank.w2s + (c * H + row) * 2);
      }
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();  // the previous block / fragment is done with hs
#pragma unroll
      for (int r = 0; r < kLoads; ++r) {
        const int v = min(tid + r * kSgThreads, 2 * 16 * (kb / 8) - 1);
        const int which = v / (16 * (kb / 8));
        const int rr = v - which * 16 * (kb / 8);
        const int n = rr / (kb / 8), c8 = rr - n * (kb / 8);
        hs[which][n * kRowU4 + c8] = hv[r];
      }
      __syncthreads();
#pragma unroll
      for (int s = 0; s <= kQ; ++s) {
        const bool full = s < nq;
        const bool half = (s == nq) && nhalf;  // only lane groups g < 2 hold K here
        if (full || half) {
          const float s0 = e4m3_byte_to_f32<0>(sc[s]), s1 = e4m3_byte_to_f32<1>(sc[s]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint4 a = dq8(word(q[s], j), j < 2 ? s0 : s1);
            const int kk = (4 * s + g) * 4 + j;  // 16-byte word of the staged row
            uint4 bh = hs[0][i * kRowU4 + min(kk, kb / 8 - 1)];
            uint4 bl = hs[1][i * kRowU4 + min(kk, kb / 8 - 1)];
            if (half && g >= 2) a = make_uint4(0u, 0u, 0u, 0u);  // K past the block: zero
            acc = mfma(a, bh, acc);
            acc = mfma(a, bl, acc);
          }
        }
      }
    }
    // C lane l: output rows 4 (l / 16) + jj, token l % 16 of the fragment
    const int m = f0 + i;
    if (m < un.count) {
      int t, slot;
      float wt;
      if (un.bank) {
        t = un.start + m;
        slot = p.k;
        wt = p.gamma[t];
      } else {
        const int pair = p.sorted[un.start + m];
        t = pair / p.k;
        slot = pair - t * p.k;
        wt = p.w[pair];
      }
      float4 v;
      v.x = (acc[0] * gd) * wt;
      v.y = (acc[1] * gd) * wt;
      v.z = (acc[2] * gd) * wt;
      v.w = (acc[3] * gd) * wt;
      *reinterpret_cast<float4*>(p.out + (static_cast<size_t>(t) * p.nslots + slot) * H +
                                 tile * 64 + wave * 16 + 4 * g) = v;
    }
  }
}

hipError_t launch_grouped_small(const PrefillParams& p0, int ugroups, hipStream_t s) {
  PrefillParams p = p0;
  p.ntiles1 = p.Imax / 64;
  p.ntiles2 = p.H / 64;
  sg_gateup_kernel<<<ugroups * 8 * p.ntiles1, kSgThreads, 0, s>>>(p);
  sg_down_kernel<<<ugroups * 8 * p.ntiles2, kSgThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace ftmoe
