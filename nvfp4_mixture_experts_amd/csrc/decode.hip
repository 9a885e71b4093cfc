// decode.hip -- the NVFP4 expert GEMVs of the MoE layer at decode time, gfx950.
//
// FreeToken fork PR #84 (page 1), bullet on #631: the NVFP4 MoE decode GEMV runs
// in every layer at every decode step.  FreeToken commit log (page 2): the
// clamped-SwiGLU activation across the MoE stack, 512 routed experts with top-10
// plus a gated shared expert, and a "deep-K" decode configuration.
//
// Two kernels, both HBM-bound streams of 4-bit codes:
//  * gateup_kernel: gate and up rows of every selected expert (K = H, deep K).
//    LPR lanes share a row; each lane owns whole 32-element chunks (16 code bytes
//    + 2 scale bytes), so one wave load covers whole 128-byte lines.  The
//    activation chunk of a lane is loaded once into registers and reused for
//    every row the lane visits.  Codes are decoded in registers to packed bf16
//    (exact) and multiplied against the bf16 activations with v_dot2_f32_bf16;
//    each 16-element block sum is scaled by its e4m3 scale; the lane group is
//    reduced with a fixed butterfly; the row is scaled by the global scales and
//    passed through the (clamped) SwiGLU.  h stays fp32.
//  * down_kernel: down rows (K = I, short).  The down codes are stored
//    K-chunk-major, so lane l of a wave owns output row 64*g + l and a wave load
//    of one chunk reads 64 consecutive rows' 16-byte records (1 KiB contiguous).
//    h is the same for all lanes (uniform loads).  The waves of a block split the
//    chunks; their partial sums and then the per-expert results are combined in
//    a fixed order, the per-expert results across blocks by the last block to
//    arrive at a per-row-group counter (no floating-point atomics).
#include "ftmoe_device.hpp"
#include "ftmoe_kernels.hpp"

namespace ftmoe {

constexpr int kGUWaves = 4;
constexpr int kGUPairsPerGroup = 2;  // (gate, up) row pairs per lane group
constexpr int kDownWaves = 4;

template <int LPR, int CPL>
__global__ __launch_bounds__(kGUWaves* kWave) void gateup_kernel(GateUpParams p) {
  constexpr int GPW = kWave / LPR;  // lane groups per wave
  constexpr int PAIRS_PER_BLOCK = kGUWaves * GPW * kGUPairsPerGroup;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = blockIdx.y;
  const int t = blockIdx.z;
  const bool is_shared = (slot == p.k);
  const Bank b = is_shared ? p.shared : p.routed;
  const int I = b.inter;
  if (blockIdx.x * PAIRS_PER_BLOCK >= I) return;  // a smaller shared expert
  const int e = is_shared ? 0 : p.ids[t * p.k + slot];
  const int H = p.H;
  const int group = lane / LPR, col = lane % LPR;
  const int pair0 = blockIdx.x * PAIRS_PER_BLOCK + (wave * GPW + group) * kGUPairsPerGroup;
  float* __restrict__ hout = p.h + (static_cast<size_t>(t) * (p.k + 1) + slot) * p.Imax;
  if (!is_shared && static_cast<unsigned>(e) >= static_cast<unsigned>(p.E)) {
    // an expert id outside the bank: poison this slot's h instead of reading out of bounds
    for (int q = 0; q < kGUPairsPerGroup; ++q)
      if (col == LPR - 1 && pair0 + q < I) hout[pair0 + q] = __builtin_nanf("");
    return;
  }

  // activation chunks of this lane: x[t][32 j .. 32 j + 31], j = col + LPR c
  bf16x2 xr[CPL][16];
  const uint16_t* __restrict__ xt = p.x + static_cast<size_t>(t) * H;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const uint4* xp = reinterpret_cast<const uint4*>(xt + 32 * (col + LPR * c));
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint4 u = xp[v];
      xr[c][4 * v + 0] = __builtin_bit_cast(bf16x2, u.x);
      xr[c][4 * v + 1] = __builtin_bit_cast(bf16x2, u.y);
      xr[c][4 * v + 2] = __builtin_bit_cast(bf16x2, u.z);
      xr[c][4 * v + 3] = __builtin_bit_cast(bf16x2, u.w);
    }
  }

  const size_t row_bytes = static_cast<size_t>(H) / 2;
  const size_t srow_bytes = static_cast<size_t>(H) / 16;
  const uint8_t* __restrict__ codes = b.w13 + static_cast<size_t>(e) * 2 * I * row_bytes;
  const uint8_t* __restrict__ scales = b.w13s + static_cast<size_t>(e) * 2 * I * srow_bytes;

  // issue every load of this lane first (memory-level parallelism), then compute
  uint4 qg[kGUPairsPerGroup][CPL], qu[kGUPairsPerGroup][CPL];
  uint32_t sg[kGUPairsPerGroup][CPL], su[kGUPairsPerGroup][CPL];
#pragma unroll
  for (int q = 0; q < kGUPairsPerGroup; ++q) {
    const int r = pair0 + q;
    const size_t rr = static_cast<size_t>(r < I ? r : 0);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int j = col + LPR * c;
      qg[q][c] = *reinterpret_cast<const uint4*>(codes + rr * row_bytes + 16 * j);
      qu[q][c] = *reinterpret_cast<const uint4*>(codes + (I + rr) * row_bytes + 16 * j);
      sg[q][c] = *reinterpret_cast<const uint16_t*>(scales + rr * srow_bytes + 2 * j);
      su[q][c] = *reinterpret_cast<const uint16_t*>(scales + (I + rr) * srow_bytes + 2 * j);
    }
  }
  const float g_gate = b.gsc[3 * e + 0];
  const float g_up = b.gsc[3 * e + 1];
#pragma unroll
  for (int q = 0; q < kGUPairsPerGroup; ++q) {
    float ag = 0.0f, au = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      ag += chunk_dot_bf16(qg[q][c], sg[q][c], xr[c]);
      au += chunk_dot_bf16(qu[q][c], su[q][c], xr[c]);
    }
    ag = group_sum_last<LPR>(ag);
    au = group_sum_last<LPR>(au);
    const int r = pair0 + q;
    if (col == LPR - 1 && r < I)
      hout[r] = swiglu(p.act, ag * g_gate, au * g_up, p.gate_max, p.up_absmax);
  }
}

__global__ __launch_bounds__(kDownWaves* kWave) void down_kernel(DownParams p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = blockIdx.x;  // group of 64 output rows
  const int slot = blockIdx.y;
  const int t = blockIdx.z;
  const int H = p.H;
  const int nrg = H / kWave;
  const bool is_shared = (slot == p.k);
  const Bank b = is_shared ? p.shared : p.routed;
  const int e_in = is_shared ? 0 : p.ids[t * p.k + slot];
  // an expert id outside the bank contributes NaN and reads nothing of the bank
  const bool bad = !is_shared && static_cast<unsigned>(e_in) >= static_cast<unsigned>(p.E);
  const int e = bad ? 0 : e_in;
  const int nch = bad ? 0 : b.inter / 32;
  const int cpw = (nch + kDownWaves - 1) / kDownWaves;
  const int j0 = wave * cpw;
  const int j1 = min(nch, j0 + cpw);
  const int c = rg * kWave + lane;

  const float* __restrict__ hrow = p.h + (static_cast<size_t>(t) * (p.k + 1) + slot) * p.Imax;
  const uint8_t* __restrict__ codes = b.w2 + static_cast<size_t>(e) * nch * H * 16;
  const uint8_t* __restrict__ scales = b.w2s + static_cast<size_t>(e) * nch * H * 2;

  float acc = 0.0f;
  for (int j = j0; j < j1; ++j) {
    const uint4 q = *reinterpret_cast<const uint4*>(codes + (static_cast<size_t>(j) * H + c) * 16);
    const uint32_t s = *reinterpret_cast<const uint16_t*>(scales + (static_cast<size_t>(j) * H + c) * 2);
    float hv[32];
#pragma unroll
    for (int m = 0; m < 32; ++m) hv[m] = hrow[32 * j + m];
    acc += chunk_dot_f32(q, s, hv);
  }

  __shared__ float red[kDownWaves][kWave];
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  float o = red[0][lane];
#pragma unroll
  for (int w = 1; w < kDownWaves; ++w) o += red[w][lane];
  const float ws = is_shared ? p.gamma[t] : p.w[t * p.k + slot];
  o = bad ? __builtin_nanf("") : (o * b.gsc[3 * e + 2]) * ws;

  const size_t pbase = (static_cast<size_t>(t) * nrg + rg) * p.nslots;
  st_dev(&p.part[(pbase + slot) * kWave + lane], o);
  wait_mem();
  uint32_t old = 0;
  if (lane == 0) old = add_dev(&p.cnt[t * nrg + rg], 1u);
  old = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(old)));
  if (old != static_cast<uint32_t>(p.nslots - 1)) return;
  // last of the nslots blocks of this row group: combine in slot order
  float y = 0.0f;
  for (int sl = 0; sl < p.nslots; ++sl) y += ld_dev(&p.part[(pbase + sl) * kWave + lane]);
  p.y[static_cast<size_t>(t) * H + c] = f32_to_bf16_bits(y);
  if (lane == 0) st_dev(&p.cnt[t * nrg + rg], 0u);
}

template <int LPR>
static hipError_t launch_gateup_lpr(const GateUpParams& p, dim3 block, hipStream_t s) {
  constexpr int GPW = kWave / LPR;
  constexpr int PAIRS_PER_BLOCK = kGUWaves * GPW * kGUPairsPerGroup;
  const int cpl = p.H / (32 * LPR);
  const int imax = p.routed.inter > p.shared.inter ? p.routed.inter : p.shared.inter;
  dim3 grid((imax + PAIRS_PER_BLOCK - 1) / PAIRS_PER_BLOCK, p.k + (p.shared.inter > 0 ? 1 : 0),
            p.T);
  switch (cpl) {
    case 1: gateup_kernel<LPR, 1><<<grid, block, 0, s>>>(p); break;
    case 2: gateup_kernel<LPR, 2><<<grid, block, 0, s>>>(p); break;
    case 3: gateup_kernel<LPR, 3><<<grid, block, 0, s>>>(p); break;
    case 4: gateup_kernel<LPR, 4><<<grid, block, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Lanes per row and chunks per lane of the gate|up GEMV for hidden size H:
// the widest power of two <= 64 lanes that divides the H/32 chunks.
void gateup_geometry(int H, int* lpr, int* cpl) {
  const int chunks = H / 32;
  int l = 64;
  while (l > 8 && chunks % l != 0) l >>= 1;
  *lpr = (chunks % l == 0) ? l : 0;
  *cpl = (*lpr > 0) ? chunks / l : 0;
}

hipError_t launch_gateup(const GateUpParams& p, hipStream_t s) {
  dim3 block(kGUWaves * kWave);
  // lanes per row: the widest power of two <= 64 that divides the H/32 chunks
  const int chunks = p.H / 32;
  if (chunks % 64 == 0) return launch_gateup_lpr<64>(p, block, s);
  if (chunks % 32 == 0) return launch_gateup_lpr<32>(p, block, s);
  if (chunks % 16 == 0) return launch_gateup_lpr<16>(p, block, s);
  if (chunks % 8 == 0) return launch_gateup_lpr<8>(p, block, s);
  return hipErrorInvalidValue;
}

hipError_t launch_down(const DownParams& p, hipStream_t s) {
  dim3 grid(p.H / kWave, p.nslots, p.T);
  down_kernel<<<grid, dim3(kDownWaves * kWave), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace ftmoe
