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
//   sg_gateup_kernel  h = SwiGLU(gate . x, up . x), stored in fp16 when the clamped
//                     activation bounds it (h16), else as a bf16 (hi, lo) pair
//   sg_down_kernel    out[t][slot][row] = (W_down h) * g_down * weight, with fp16 weight
//                     tiles against fp16 h, or bf16 tiles against h_hi and h_lo
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
// Non-temporal: for the down codes of a decode batch (measured: 12.2 -> 11.8 us at T = 32;
// the gate|up codes, which hot experts' units share, were slower so).
__device__ __forceinline__ uint4 ldg16_nt(const void* p) {
  typedef unsigned int nt_u4 __attribute__((ext_vector_type(4)));
  const nt_u4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ sg_f32x4 mfma(uint4 a, uint4 b, sg_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(sg_bf16x8, a),
                                                 __builtin_bit_cast(sg_bf16x8, b), c, 0, 0, 0);
}
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 sg_f16x8;
// fp16 operands (H16: fp16 weight tile and fp16 h) or bf16
template <bool H16>
__device__ __forceinline__ sg_f32x4 mfma16(uint4 a, uint4 b, sg_f32x4 c) {
  if constexpr (H16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(sg_f16x8, a),
                                                  __builtin_bit_cast(sg_f16x8, b), c, 0, 0, 0);
  else
    return mfma(a, b, c);
}

__device__ __forceinline__ uint32_t word(const uint4& q, int j) {
  return j == 0 ? q.x : (j == 1 ? q.y : (j == 2 ? q.z : q.w));
}

// Row tiles of 64 per block in the pipelined down product: their codes are all in
// registers at once (NKC 16-byte words per tile and lane).  Two keep a block small
// enough in registers for 3 waves per SIMD, so the whole grid of a decode batch is
// resident at once (4 tiles share the staged h better but fit only 2 waves per SIMD,
// and the grid then ran in two rounds).
constexpr int kDownPipeTiles = 2;

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
  const int nun = *p.nunits;  // both loads issued before either is waited for
  const PfUnit un = p.units[u];  // in bounds: the table has kUnitSlack spare entries
  __asm__ volatile("" ::: "memory");  // keeps them here (not sunk past the check)
  if (u >= nun) return;
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
        const int tq = p.sorted[un.start + m] / p.k;  // read for both banks (in bounds: a
        const int t = un.bank ? un.start + m : tq;    // shared unit's start + m < T <= P)
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
            ag = mfma(dequant8_bf16(word(qg[q], j), j < 2 ? g0 : g1), b, ag);
            au = mfma(dequant8_bf16(word(qu[q], j), j < 2 ? u0 : u1), b, au);
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
      float hv[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        hv[jj] = swiglu(p.act, ag[jj] * gg, au[jj] * gu, p.gate_max, p.up_absmax);
      store_h4(p.hhi, p.hlo, row * p.Imax + col, hv, p.h16);
    }
  }
}

// The same product for H = NKB * 512, software-pipelined: the K loop is unrolled
// so that K block kb + 1's codes are in flight while K block kb is computed (every
// block of the grid is resident at once for these sizes, so without this all of
// them issue, drain and compute in lockstep and HBM idles between K blocks).  For
// H <= 2048 all of K of the 16 token rows is staged in LDS at once (66 KB: two
// blocks per CU), behind one barrier, and the K loop has none; for larger H the
// rows are staged per K block (two barriers each), loaded one K block ahead.  K
// mapping inside a 512-K block: lane group g takes the four consecutive 32-K chunks
// 4 g .. 4 g + 3 of its row (64 contiguous code bytes, 8 contiguous scale bytes: one
// 8-byte scale load per row instead of four).
template <int NKB>
__global__ __launch_bounds__(kSgThreads, 2) void sg_gateup_pipe_kernel(PrefillParams p) {
  constexpr int kKB = 512;
  constexpr bool kAll = NKB <= 4;                      // all of K staged at once
  constexpr int kSt = kAll ? NKB : 1;                  // K blocks per staged row
  constexpr int kRowU4 = kSt * kKB / 8 + 1;            // 16-byte words per staged row (+1 pad)
  constexpr int kXL = 16 * (kKB / 8) / kSgThreads;     // token-row loads per thread per K block
  __shared__ uint4 xs[16 * kRowU4];
  int u, tile;
  sg_unit_tile(p.ntiles1, &u, &tile);
  const int nun = *p.nunits;  // both loads issued before either is waited for
  const PfUnit un = p.units[u];  // in bounds: the table has kUnitSlack spare entries
  __asm__ volatile("" ::: "memory");  // keeps them here (not sunk past the check)
  if (u >= nun) return;
  const Bank bank = un.bank ? p.shared : p.routed;
  const int I = bank.inter;
  const int n0 = tile * 64;
  if (n0 >= I) return;
  constexpr int H = NKB * kKB;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, g = lane >> 4;
  const int grow = n0 + wave * 16 + i;  // gate row; up row I + grow
  const size_t ebase = static_cast<size_t>(un.expert) * 2 * I;
  const uint8_t* gc = bank.w13 + (ebase + grow) * (H / 2) + 64 * g;
  const uint8_t* uc = bank.w13 + (ebase + I + grow) * (H / 2) + 64 * g;
  const uint8_t* gsp = bank.w13s + (ebase + grow) * (H / 16) + 8 * g;
  const uint8_t* usp = bank.w13s + (ebase + I + grow) * (H / 16) + 8 * g;
  const float gg = bank.gsc[un.expert * 3 + 0], gu = bank.gsc[un.expert * 3 + 1];
  // staged layout: thread tid moves word c8 = tid % 64 of each K block of token rows
  // n = tid / 64 + 4 r
  const int c8 = tid & 63;
  for (int f0 = 0; f0 < un.count; f0 += 16) {
    const uint16_t* xrow[kXL];
#pragma unroll
    for (int r = 0; r < kXL; ++r) {
      const int m = min(f0 + (tid >> 6) + 4 * r, un.count - 1);  // past the unit: its last token
      const int tq = p.sorted[un.start + m] / p.k;  // read for both banks (in bounds: a
      const int t = un.bank ? un.start + m : tq;    // shared unit's start + m < T <= P)
      xrow[r] = p.x + static_cast<size_t>(t) * H + 8 * c8;
    }
    uint4 xv[kAll ? NKB : 2][kXL], qg[2][4], qu[2][4];
    uint2 sg[2], su[2];
    auto issue = [&](int kb, int b) {
      if constexpr (!kAll) {
#pragma unroll
        for (int r = 0; r < kXL; ++r) xv[b][r] = ldg16(xrow[r] + kb * kKB);
        __builtin_amdgcn_sched_barrier(0);  // token rows first: the staging waits for them
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        qg[b][q] = ldg16(gc + kb * (kKB / 2) + 16 * q);
        qu[b][q] = ldg16(uc + kb * (kKB / 2) + 16 * q);
      }
      sg[b] = *reinterpret_cast<const uint2*>(gsp + kb * (kKB / 16));
      su[b] = *reinterpret_cast<const uint2*>(usp + kb * (kKB / 16));
      __builtin_amdgcn_sched_barrier(0);
    };
    sg_f32x4 ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
    if constexpr (kAll) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < kXL; ++r) xv[kb][r] = ldg16(xrow[r] + kb * kKB);
      __builtin_amdgcn_sched_barrier(0);  // token rows first: the staging waits for them
      issue(0, 0);
      if (f0 > 0) __syncthreads();  // the previous fragment is done with xs
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < kXL; ++r)
          xs[((tid >> 6) + 4 * r) * kRowU4 + kb * (kKB / 8) + c8] = xv[kb][r];
      __syncthreads();
    } else {
      issue(0, 0);
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int b = kb & 1;
      if (kb + 1 < NKB) issue(kb + 1, b ^ 1);
      if constexpr (!kAll) {
        __syncthreads();  // the previous K block (or fragment) is done with xs
#pragma unroll
        for (int r = 0; r < kXL; ++r) xs[((tid >> 6) + 4 * r) * kRowU4 + c8] = xv[b][r];
        __syncthreads();
      }
      const int kx = kAll ? kb * (kKB / 8) : 0;  // the K block's first word in a staged row
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t gw = q < 2 ? sg[b].x : sg[b].y, uw = q < 2 ? su[b].x : su[b].y;
        const float g0 = (q & 1) ? e4m3_byte_to_f32<2>(gw) : e4m3_byte_to_f32<0>(gw);
        const float g1 = (q & 1) ? e4m3_byte_to_f32<3>(gw) : e4m3_byte_to_f32<1>(gw);
        const float u0 = (q & 1) ? e4m3_byte_to_f32<2>(uw) : e4m3_byte_to_f32<0>(uw);
        const float u1 = (q & 1) ? e4m3_byte_to_f32<3>(uw) : e4m3_byte_to_f32<1>(uw);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 bx = xs[i * kRowU4 + kx + (4 * g + q) * 4 + j];
          ag = mfma(dequant8_bf16(word(qg[b][q], j), j < 2 ? g0 : g1), bx, ag);
          au = mfma(dequant8_bf16(word(qu[b][q], j), j < 2 ? u0 : u1), bx, au);
        }
      }
    }
    // C lane l: rows 4 (l / 16) + jj (h columns), token l % 16 of the fragment
    const int m = f0 + i;
    if (m < un.count) {
      const int t = un.bank ? un.start + m : 0;
      const size_t row = un.bank ? static_cast<size_t>(p.P) + t : static_cast<size_t>(un.start) + m;
      const int col = n0 + wave * 16 + 4 * g;
      float hv[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        hv[jj] = swiglu(p.act, ag[jj] * gg, au[jj] * gu, p.gate_max, p.up_absmax);
      store_h4(p.hhi, p.hlo, row * p.Imax + col, hv, p.h16);
    }
  }
}

// Block: 64 output rows (4 waves x 16) of one unit; LDS: 16 tokens' h (fp16, or
// hi and lo) for a K block of up to 1024.
template <bool H16>
__global__ __launch_bounds__(kSgThreads, 2) void sg_down_kernel(PrefillParams p) {
  constexpr int kKB = 512;
  constexpr int kQ = kKB / 128;
  constexpr int kRowU4 = kKB / 8 + 1;
  constexpr int NB = H16 ? 1 : 2;  // staged h operands
  __shared__ uint4 hs[NB][16 * kRowU4];
  int u, tile;
  sg_unit_tile(p.ntiles2, &u, &tile);
  const int nun = *p.nunits;  // both loads issued before either is waited for
  const PfUnit un = p.units[u];  // in bounds: the table has kUnitSlack spare entries
  __asm__ volatile("" ::: "memory");  // keeps them here (not sunk past the check)
  if (u >= nun) return;
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
      constexpr int kLoads = NB * 16 * (kKB / 8) / kSgThreads;
      uint4 hv[kLoads];
#pragma unroll
      for (int r = 0; r < kLoads; ++r) {
        const int v = min(tid + r * kSgThreads, NB * 16 * (kb / 8) - 1);
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
        const int v = min(tid + r * kSgThreads, NB * 16 * (kb / 8) - 1);
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
            uint4 a = dequant8_tile<H16>(word(q[s], j), j < 2 ? s0 : s1);
            const int kk = (4 * s + g) * 4 + j;  // 16-byte word of the staged row
            const uint4 bh = hs[0][i * kRowU4 + min(kk, kb / 8 - 1)];
            if (half && g >= 2) a = make_uint4(0u, 0u, 0u, 0u);  // K past the block: zero
            acc = mfma16<H16>(a, bh, acc);
            if constexpr (!H16) acc = mfma(a, hs[NB - 1][i * kRowU4 + min(kk, kb / 8 - 1)], acc);
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

// The down product for I = 128 * NKC (both banks), one block per kRT row tiles of
// 64: the fragment's h (hi and lo, all of K) is staged in LDS once and serves the
// kRT tiles, and the codes of all kRT tiles are issued up front, so a block pays
// one memory latency, not one per tile.
template <int NKC, bool H16>
__global__ __launch_bounds__(kSgThreads, 2) void sg_down_pipe_kernel(PrefillParams p) {
  constexpr int kI = 128 * NKC;
  constexpr int kRowU4 = kI / 8 + 1;
  constexpr int kRT = kDownPipeTiles;                      // row tiles per block
  constexpr int NB = H16 ? 1 : 2;                          // staged h operands
  constexpr int kHL = NB * 16 * (kI / 8) / kSgThreads;     // h loads per thread
  static_assert(kHL * kSgThreads == NB * 16 * (kI / 8), "whole staging rounds");
  __shared__ uint4 hs[NB][16 * kRowU4];
  int u, tg;
  sg_unit_tile(p.ntiles2, &u, &tg);
  const int nun = *p.nunits;  // both loads issued before either is waited for
  const PfUnit un = p.units[u];  // in bounds: the table has kUnitSlack spare entries
  __asm__ volatile("" ::: "memory");  // keeps them here (not sunk past the check)
  if (u >= nun) return;
  const Bank bank = un.bank ? p.shared : p.routed;
  const int H = p.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, g = lane >> 4;
  const size_t cbase = static_cast<size_t>(un.expert) * (kI / 32);
  const float gd = bank.gsc[un.expert * 3 + 2];
  const int row0 = tg * (64 * kRT) + wave * 16;  // + 64 rt + i: this lane's weight row
  for (int f0 = 0; f0 < un.count; f0 += 16) {
    // C lane l: output rows 4 (l / 16) + jj of the wave's 16, token l % 16.  The
    // (token, slot) pair is loaded first, its weight (which depends on it) after
    // the h and code loads, so that neither waits in front of them.
    const int m = f0 + i;
    const int mm = min(m, un.count - 1);
    const int sv = p.sorted[un.start + mm];  // read for both banks (in bounds: a shared
    const int pair = un.bank ? 0 : sv;        // unit's start + mm < T <= P)
    uint4 hv[kHL];
#pragma unroll
    for (int r = 0; r < kHL; ++r) {
      const int v = tid + r * kSgThreads;
      const int which = v / (16 * (kI / 8));
      const int rr = v - which * 16 * (kI / 8);
      const int n = rr / (kI / 8), c8 = rr - n * (kI / 8);
      const int mh = min(f0 + n, un.count - 1);
      const size_t hrow = un.bank ? static_cast<size_t>(p.P) + un.start + mh
                                  : static_cast<size_t>(un.start) + mh;
      hv[r] = ldg16((which ? p.hlo : p.hhi) + hrow * p.Imax + 8 * c8);
    }
    __builtin_amdgcn_sched_barrier(0);  // h first (the staging waits for it)
    // scales: the 4-byte word holding this row's and its even/odd neighbour's two
    // bytes (a 2-byte load would be widened right at the load, which waits for it)
    uint4 q[kRT][NKC];
    uint32_t sc[kRT][NKC];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      const int row = row0 + 64 * rt + i;
#pragma unroll
      for (int s = 0; s < NKC; ++s) {
        const size_t c = cbase + 4 * s + g;  // chunk 4 s + g of 32 K
        q[rt][s] = ldg16_nt(bank.w2 + (c * H + row) * 16);
        sc[rt][s] = *reinterpret_cast<const uint32_t*>(bank.w2s + (c * H + (row & ~1)) * 2);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    int t, slot;
    float wt;
    if (un.bank) {
      t = un.start + mm;
      slot = p.k;
      wt = p.gamma[t];
    } else {
      t = pair / p.k;
      slot = pair - t * p.k;
      wt = p.w[pair];
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();  // the previous fragment is done with hs
#pragma unroll
    for (int r = 0; r < kHL; ++r) {
      const int v = tid + r * kSgThreads;
      const int which = v / (16 * (kI / 8));
      const int rr = v - which * 16 * (kI / 8);
      const int n = rr / (kI / 8), c8 = rr - n * (kI / 8);
      hs[which][n * kRowU4 + c8] = hv[r];
    }
    __syncthreads();
    // the tiles step through K together: each h word is read once for all tiles,
    // and consecutive MFMAs write different accumulators (h_hi products of every
    // tile, then h_lo; each accumulator adds its terms in the same order)
    sg_f32x4 acc[kRT];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) acc[rt] = sg_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NKC; ++s) {
      float s0[kRT], s1[kRT];
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        const uint32_t sw = sc[rt][s] >> (16 * (i & 1));  // rows are even + i
        s0[rt] = e4m3_byte_to_f32<0>(sw);
        s1[rt] = e4m3_byte_to_f32<1>(sw);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kk = (4 * s + g) * 4 + j;  // 16-byte word of the staged row
        const uint4 bh = hs[0][i * kRowU4 + kk];
        uint4 a[kRT];
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
          a[rt] = dequant8_tile<H16>(word(q[rt][s], j), j < 2 ? s0[rt] : s1[rt]);
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) acc[rt] = mfma16<H16>(a[rt], bh, acc[rt]);
        if constexpr (!H16) {
          const uint4 bl = hs[NB - 1][i * kRowU4 + kk];
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt) acc[rt] = mfma(a[rt], bl, acc[rt]);
        }
      }
    }
    if (m < un.count) {
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        float4 v;
        v.x = (acc[rt][0] * gd) * wt;
        v.y = (acc[rt][1] * gd) * wt;
        v.z = (acc[rt][2] * gd) * wt;
        v.w = (acc[rt][3] * gd) * wt;
        *reinterpret_cast<float4*>(p.out + (static_cast<size_t>(t) * p.nslots + slot) * H + row0 +
                                   64 * rt + 4 * g) = v;
      }
    }
  }
}

hipError_t launch_grouped_small(const PrefillParams& p0, int ugroups, hipStream_t s) {
  PrefillParams p = p0;
  p.ntiles1 = p.Imax / 64;
  p.ntiles2 = p.H / 64;
  const dim3 g1(ugroups * 8 * p.ntiles1), blk(kSgThreads);
  switch (p.H) {
    case 1024: sg_gateup_pipe_kernel<2><<<g1, blk, 0, s>>>(p); break;
    case 2048: sg_gateup_pipe_kernel<4><<<g1, blk, 0, s>>>(p); break;
    case 3072: sg_gateup_pipe_kernel<6><<<g1, blk, 0, s>>>(p); break;
    case 4096: sg_gateup_pipe_kernel<8><<<g1, blk, 0, s>>>(p); break;
    default: sg_gateup_kernel<<<g1, blk, 0, s>>>(p); break;
  }
  // the pipelined down product needs one I for both banks and H in whole row-tile groups
  const int I = p.routed.inter;
  const bool one_i = p.shared.inter == 0 || p.shared.inter == I;
  const int nkc = (one_i && p.H % 256 == 0 && I % 128 == 0) ? I / 128 : 0;
  if (nkc == 4 || nkc == 6 || nkc == 8) {
    p.ntiles2 = p.H / (64 * kDownPipeTiles);
    const dim3 g2(ugroups * 8 * p.ntiles2);
    if (p.h16) {
      if (nkc == 4) sg_down_pipe_kernel<4, true><<<g2, blk, 0, s>>>(p);
      else if (nkc == 6) sg_down_pipe_kernel<6, true><<<g2, blk, 0, s>>>(p);
      else sg_down_pipe_kernel<8, true><<<g2, blk, 0, s>>>(p);
    } else {
      if (nkc == 4) sg_down_pipe_kernel<4, false><<<g2, blk, 0, s>>>(p);
      else if (nkc == 6) sg_down_pipe_kernel<6, false><<<g2, blk, 0, s>>>(p);
      else sg_down_pipe_kernel<8, false><<<g2, blk, 0, s>>>(p);
    }
  } else {
    if (p.h16) sg_down_kernel<true><<<ugroups * 8 * p.ntiles2, blk, 0, s>>>(p);
    else sg_down_kernel<false><<<ugroups * 8 * p.ntiles2, blk, 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace ftmoe
