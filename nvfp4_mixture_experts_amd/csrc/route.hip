// route.hip -- MoE router for gfx950: logits in fp64, the shared expert's
// sigmoid gate, and top-k selection with softmax weights over the selected
// logits.
//
// FreeToken commit log (page 2): the entry on router and shared-gate kernels and
// the entry on a top-k router whose k is not a power of two (k = 10 of 512); the 288-expert layer
// routes top-8.  Logits are accumulated in fp64 (every fp32 x bf16 product is
// exact in fp64) and rounded once to fp32, so the selection does not depend on
// the summation order; ties go to the lower expert index.
#include "ftmoe_device.hpp"
#include "ftmoe_kernels.hpp"

namespace ftmoe {

constexpr int kRouteWaves = 4;     // one expert row per wave
constexpr int kRouteMaxTokTile = 64;
constexpr int kRouteTargetWaves = 8192;  // enough waves to fill 256 CUs several times

// Tokens a router wave takes at once (their x pieces are held in registers together).
constexpr int route_token_group(int nc) { return nc <= 8 ? 4 : (nc <= 16 ? 2 : 1); }

// Top-k of one token by one wave (wave_topk), written in rank order.
template <class Load>
__device__ void topk_one_token(int E, int k, Load load, int32_t* ids, float* w, int32_t* ids2,
                               float* w2) {
  const int lane = threadIdx.x & (kWave - 1);
  int id;
  float wt;
  if (E <= 4 * kWave)
    wave_topk<4>(E, k, load, &id, &wt);
  else if (E <= 8 * kWave)
    wave_topk<8>(E, k, load, &id, &wt);
  else
    wave_topk<16>(E, k, load, &id, &wt);
  if (lane < k) {
    ids[lane] = id;
    w[lane] = wt;
    if (ids2) ids2[lane] = id;
    if (w2) w2[lane] = wt;
  }
}

// logits[t][e] for expert row e = blockIdx.x * kRouteWaves + wave; row E is the
// shared expert's gate (gamma[t] = sigmoid(sum_h gs[h] x[t][h])).  Each lane
// holds NC float4 pieces of the row (interleaved by lane so that every wave load
// reads 1 KiB contiguous) and reuses them across the token tile.  Tokens go in
// groups of G: the x loads of a group are issued together and the G dot
// products interleave (each still sums its own terms in the same order), so a
// group costs one load latency, not G.
template <int NC>
__global__ __launch_bounds__(kRouteWaves* kWave) void route_logits_kernel(RouteParams p,
                                                                          int fuse_topk) {
  constexpr int G = route_token_group(NC);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = blockIdx.x * kRouteWaves + wave;
  const int t0 = blockIdx.y * p.tok_tile;
  const int t1 = min(p.T, t0 + p.tok_tile);
  const int H = p.H;
  const bool gate_row = row == p.E;

  if (row < p.E || (gate_row && p.shared_gate != nullptr)) {
    float4 wv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (!gate_row) {
        wv[c] = *reinterpret_cast<const float4*>(p.wr + static_cast<size_t>(row) * H + 4 * lane +
                                                 4 * kWave * c);
      } else {
        const uint2 g2 = *reinterpret_cast<const uint2*>(p.shared_gate + 4 * lane + 4 * kWave * c);
        wv[c] = make_float4(bf16_bits_to_f32(g2.x & 0xFFFFu), bf16_bits_to_f32(g2.x >> 16),
                            bf16_bits_to_f32(g2.y & 0xFFFFu), bf16_bits_to_f32(g2.y >> 16));
      }
    }
    const double b = (!gate_row && p.bias) ? static_cast<double>(p.bias[row]) : 0.0;
    // the row in fp64 once, not once per token
    double wd[NC][4];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      wd[c][0] = static_cast<double>(wv[c].x);
      wd[c][1] = static_cast<double>(wv[c].y);
      wd[c][2] = static_cast<double>(wv[c].z);
      wd[c][3] = static_cast<double>(wv[c].w);
    }
    for (int tg = t0; tg < t1; tg += G) {
      uint2 xb[G][NC];
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const int t = min(tg + j, t1 - 1);  // past the tile: repeat its last token
        const uint16_t* __restrict__ xt = p.x + static_cast<size_t>(t) * H;
#pragma unroll
        for (int c = 0; c < NC; ++c)
          xb[j][c] = *reinterpret_cast<const uint2*>(xt + 4 * lane + 4 * kWave * c);
      }
      double acc[G];
#pragma unroll
      for (int j = 0; j < G; ++j) acc[j] = 0.0;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
          const uint2 x2 = xb[j][c];
          acc[j] = fma(wd[c][0], static_cast<double>(bf16_bits_to_f32(x2.x & 0xFFFFu)), acc[j]);
          acc[j] = fma(wd[c][1], static_cast<double>(bf16_bits_to_f32(x2.x >> 16)), acc[j]);
          acc[j] = fma(wd[c][2], static_cast<double>(bf16_bits_to_f32(x2.y & 0xFFFFu)), acc[j]);
          acc[j] = fma(wd[c][3], static_cast<double>(bf16_bits_to_f32(x2.y >> 16)), acc[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < G; ++j) acc[j] = wave_sum_f64(acc[j]);
      if (lane == 0) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
          const int t = tg + j;
          if (t >= t1) break;
          if (!gate_row) {
            st_dev(&p.logits[static_cast<size_t>(t) * p.E + row],
                   static_cast<float>(p.bias ? acc[j] + b : acc[j]));
          } else {
            p.gamma[t] = static_cast<float>(1.0 / (1.0 + exp(-acc[j])));
          }
        }
      }
    }
  }

  if (!fuse_topk) return;
  // Last-arriver top-k: every block publishes its logits (device-coherent
  // stores), and the block that arrives last at one device-scope counter selects
  // the experts of all tokens.  No block waits for another.
  __shared__ uint32_t s_last;
  wait_mem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t nblocks = gridDim.x * gridDim.y;
    const uint32_t old = add_dev(p.counter, 1u);
    s_last = (old == nblocks - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!s_last) return;
  for (int t = wave; t < p.T; t += kRouteWaves) {
    const float* lg = p.logits + static_cast<size_t>(t) * p.E;
    topk_one_token(p.E, p.k, [&](int e) { return ld_dev(lg + e); },
                   p.ids + static_cast<size_t>(t) * p.k, p.w + static_cast<size_t>(t) * p.k,
                   p.ids_copy ? p.ids_copy + static_cast<size_t>(t) * p.k : nullptr,
                   p.w_copy ? p.w_copy + static_cast<size_t>(t) * p.k : nullptr);
  }
  if (threadIdx.x == 0) st_dev(p.counter, 0u);
}

// One wave per token (used when the token count is too large for one block).
__global__ __launch_bounds__(kRouteWaves* kWave) void topk_kernel(RouteParams p) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = blockIdx.x * kRouteWaves + wave;
  if (t >= p.T) return;
  const float* __restrict__ lg = p.logits + static_cast<size_t>(t) * p.E;
  topk_one_token(p.E, p.k, [&](int e) { return lg[e]; },
                 p.ids + static_cast<size_t>(t) * p.k, p.w + static_cast<size_t>(t) * p.k,
                 p.ids_copy ? p.ids_copy + static_cast<size_t>(t) * p.k : nullptr,
                 p.w_copy ? p.w_copy + static_cast<size_t>(t) * p.k : nullptr);
}

// One block of kTopkWaves waves per token, by rank counting (block_topk_rank):
// lower latency than a wave per token, which a call of few tokens waits on.
constexpr int kTopkWaves = 8;
constexpr int kTopkBlockMaxTokens = 256;  // above this a wave per token (less work in all)

__global__ __launch_bounds__(kTopkWaves* kWave) void topk_block_kernel(RouteParams p) {
  __shared__ __align__(16) uint64_t s_key[kTopkWaves][kWave];
  __shared__ __align__(16) uint64_t s_cand[kTopkMaxChunks * kTopkMaxK];
  __shared__ double s_v[kTopkMaxK];
  __shared__ int s_ids[kTopkMaxK];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const float* __restrict__ lg = p.logits + static_cast<size_t>(t) * p.E;
  block_topk_rank<kTopkWaves>(p.E, p.k, [&](int e) { return lg[e]; }, s_key, s_cand, s_v, s_ids);
  if (threadIdx.x < kWave) {
    const float wt = softmax_of_places(s_v, p.k);
    if (lane < p.k) {
      const size_t o = static_cast<size_t>(t) * p.k + lane;
      p.ids[o] = s_ids[lane];
      p.w[o] = wt;
      if (p.ids_copy) p.ids_copy[o] = s_ids[lane];
      if (p.w_copy) p.w_copy[o] = wt;
    }
  }
}

// Many tokens: logits as an fp64 matrix product on the MFMA units
// (v_mfma_f64_16x16x4f64).  A = router rows (16 experts x 4 K, lane l holding
// expert l % 16 at K group l / 16), B = token rows (4 K x 16 tokens, lane l
// holding token l % 16 at the same K group), C lane l holds experts l / 16 + 4 j,
// j < 4, of token l % 16.  Every fp32 x bf16 product is exact in fp64 and the sum
// is kept in fp64, then rounded once to fp32, as in the kernel above; only the
// order of the fp64 additions differs.  Which K a lane group holds only has to
// agree between A and B: in a 64-K block, group g holds K = 16 g + m in step m.
// A wave computes 16 experts x 64 tokens; a block of 4 waves 64 experts x 64
// tokens, so the 4 waves read the same token rows.
constexpr int kRouteMmExperts = 64;  // per block
constexpr int kRouteMmTokens = 64;   // per block (4 fragments of 16 per wave)

typedef __attribute__((__vector_size__(4 * sizeof(double)))) double f64x4;

__global__ __launch_bounds__(256) void route_mfma_kernel(RouteParams p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int e0 = blockIdx.x * kRouteMmExperts + wave * 16;
  const int t0 = blockIdx.y * kRouteMmTokens;
  const int H = p.H;
  const int g = lane >> 4, i = lane & 15;
  // rows past the end repeat the last valid row (their results are not stored)
  const float* wrow = p.wr + static_cast<size_t>(min(e0 + i, p.E - 1)) * H + 16 * g;
  const uint16_t* xrow[4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
    xrow[f] = p.x + static_cast<size_t>(min(t0 + 16 * f + i, p.T - 1)) * H + 16 * g;

  f64x4 acc[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) acc[f] = f64x4{0.0, 0.0, 0.0, 0.0};
  float4 wa[4];
  uint4 xa[4][2];
  auto load = [&](int k0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) wa[c] = *reinterpret_cast<const float4*>(wrow + k0 + 4 * c);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      xa[f][0] = *reinterpret_cast<const uint4*>(xrow[f] + k0);
      xa[f][1] = *reinterpret_cast<const uint4*>(xrow[f] + k0 + 8);
    }
  };
  load(0);
  for (int k0 = 0; k0 < H; k0 += 64) {
    float w[16];
    uint32_t xw[4][8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      w[4 * c + 0] = wa[c].x;
      w[4 * c + 1] = wa[c].y;
      w[4 * c + 2] = wa[c].z;
      w[4 * c + 3] = wa[c].w;
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      xw[f][0] = xa[f][0].x; xw[f][1] = xa[f][0].y; xw[f][2] = xa[f][0].z; xw[f][3] = xa[f][0].w;
      xw[f][4] = xa[f][1].x; xw[f][5] = xa[f][1].y; xw[f][6] = xa[f][1].z; xw[f][7] = xa[f][1].w;
    }
    if (k0 + 64 < H) load(k0 + 64);
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const double a = static_cast<double>(w[m]);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const uint32_t pair = xw[f][m >> 1];
        const double b = static_cast<double>(bf16_bits_to_f32((m & 1) ? (pair >> 16) : (pair & 0xFFFFu)));
        acc[f] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[f], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int t = t0 + 16 * f + i;
    if (t >= p.T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + g + 4 * j;
      if (e >= p.E) continue;
      double v = acc[f][j];
      if (p.bias) v += static_cast<double>(p.bias[e]);
      p.logits[static_cast<size_t>(t) * p.E + e] = static_cast<float>(v);
    }
  }
}

// A few to a thousand tokens: the same fp64 MFMA product, split along K so that
// the whole chip shares it (an fp64 MFMA takes 64 cycles, so one block per 64
// experts would leave most CUs idle).  Block (row block, token block, split):
// W waves x 16 rows (expert rows, then row E = the shared gate, bf16) x 32 tokens
// (2 fragments of 16) over K [split * kc, (split + 1) * kc), into
// part[split][t][row].  topk_split_kernel sums the splits in split order.
// W (route_split_waves) is the fewest from 4 that give at most kRouteSplitMaxRowBlocks
// row blocks: with the full 32 splits of a call of up to 32 tokens the grid then
// fits one block per CU (E = 512 with the shared gate, 513 rows: 64-row blocks
// would leave a ninth block of one row per split, 288 blocks, 32 CUs running two).
constexpr int kRouteSplitMinWaves = 4;
constexpr int kRouteSplitMaxWaves = 8;
constexpr int kRouteSplitMaxRowBlocks = 8;

int route_split_waves(int R) {
  int w = kRouteSplitMinWaves;
  while (w < kRouteSplitMaxWaves && (R + 16 * w - 1) / (16 * w) > kRouteSplitMaxRowBlocks) ++w;
  return w;
}

__global__ __launch_bounds__(kRouteSplitMaxWaves* kWave) void route_split_kernel(RouteParams p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int R = p.E + 1;
  const int r0 = blockIdx.x * (blockDim.x / kWave) * 16 + wave * 16;
  const int t0 = blockIdx.y * kRouteSplitTokens;
  const int kc = p.H / p.ksplit;
  const int kbeg = blockIdx.z * kc;
  const int H = p.H;
  const int g = lane >> 4, i = lane & 15;
  const int row = min(r0 + i, R - 1);  // rows past the end repeat the last (not stored)
  const bool gate_row = row == p.E;
  const bool zero_row = gate_row && p.shared_gate == nullptr;
  const float* wrow = p.wr + static_cast<size_t>(gate_row ? 0 : row) * H + 16 * g;
  const uint16_t* grow = p.shared_gate ? p.shared_gate + 16 * g : nullptr;
  const uint16_t* xrow[2];
#pragma unroll
  for (int f = 0; f < 2; ++f)
    xrow[f] = p.x + static_cast<size_t>(min(t0 + 16 * f + i, p.T - 1)) * H + 16 * g;
  f64x4 acc[2] = {f64x4{0.0, 0.0, 0.0, 0.0}, f64x4{0.0, 0.0, 0.0, 0.0}};
  for (int k0 = kbeg; k0 < kbeg + kc; k0 += 64) {
    // lane group g holds K = k0 + 16 g + m in step m, for A and B alike
    float w[16];
    if (!gate_row) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 v = *reinterpret_cast<const float4*>(wrow + k0 + 4 * c);
        w[4 * c] = v.x;
        w[4 * c + 1] = v.y;
        w[4 * c + 2] = v.z;
        w[4 * c + 3] = v.w;
      }
    } else if (!zero_row) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint4 v = *reinterpret_cast<const uint4*>(grow + k0 + 8 * c);
        const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          w[8 * c + 2 * m] = bf16_bits_to_f32(q[m] & 0xFFFFu);
          w[8 * c + 2 * m + 1] = bf16_bits_to_f32(q[m] >> 16);
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < 16; ++m) w[m] = 0.0f;
    }
    uint32_t xw[2][8];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const uint4 a = *reinterpret_cast<const uint4*>(xrow[f] + k0);
      const uint4 b = *reinterpret_cast<const uint4*>(xrow[f] + k0 + 8);
      xw[f][0] = a.x; xw[f][1] = a.y; xw[f][2] = a.z; xw[f][3] = a.w;
      xw[f][4] = b.x; xw[f][5] = b.y; xw[f][6] = b.z; xw[f][7] = b.w;
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const double a = static_cast<double>(w[m]);
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const uint32_t pair = xw[f][m >> 1];
        const double b =
            static_cast<double>(bf16_bits_to_f32((m & 1) ? (pair >> 16) : (pair & 0xFFFFu)));
        acc[f] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[f], 0, 0, 0);
      }
    }
  }
  // C lane l: rows r0 + l / 16 + 4 j of token t0 + 16 f + l % 16
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int t = t0 + 16 * f + i;
    if (t >= p.T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = r0 + g + 4 * j;
      if (r < R) p.part[(static_cast<size_t>(blockIdx.z) * p.T + t) * R + r] = acc[f][j];
    }
  }
}

// One block per token: the logits from the split partial sums (summed in split
// order, the bias added in fp64, one fp32 rounding; row E gives the shared gate),
// then the rank-count top-k.  KS = the split count: with it fixed, every load of a
// row is unconditional, so all of them are in flight before the first sum.  GL:
// E is a multiple of the block's thread count, so that the loop over rows would
// take a pass of its own for row E alone; instead lane l of every wave loads split
// l of row E ahead of the loop, and the wave sums them after it, in split order.
template <int KS, bool GL>
__global__ __launch_bounds__(kTopkWaves* kWave) void topk_split_kernel(RouteParams p) {
  __shared__ float s_logit[kMaxExperts];
  __shared__ __align__(16) uint64_t s_key[kTopkWaves][kWave];
  __shared__ __align__(16) uint64_t s_cand[kTopkMaxChunks * kTopkMaxK];
  __shared__ double s_v[kTopkMaxK];
  __shared__ int s_ids[kTopkMaxK];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int R = p.E + 1;
  const size_t stride = static_cast<size_t>(p.T) * R;
  // without a bias the bias load reads the router weights (at least E floats) and
  // its value is masked off: the load is unconditional, so that no branch waits
  // for it, and it is issued ahead of the split loads
  const float* bsrc = p.bias ? p.bias : p.wr;
  double gpart = 0.0, gsum = 0.0;
  if constexpr (GL)
    gpart = p.part[static_cast<size_t>(lane % KS) * stride + static_cast<size_t>(t) * R + p.E];
  for (int r = threadIdx.x; r < (GL ? p.E : R); r += blockDim.x) {
    const float b = bsrc[min(r, p.E - 1)];
    const double* src = p.part + static_cast<size_t>(t) * R + r;
    double pv[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) pv[ks] = src[static_cast<size_t>(ks) * stride];
    // no add is scheduled between the loads (it would wait for the first of them
    // before the rest are issued)
    __builtin_amdgcn_sched_barrier(0);
    double v = 0.0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) v += pv[ks];
    // The bias is added on every row, masked to +0.0 where there is none (no bias,
    // or the shared-gate row): the sum starts from +0.0 and so is never -0.0, and
    // adding +0.0 leaves it unchanged.  The mask is hidden from the optimiser, so
    // that the add is not turned back into a branch that the load would sink into.
    uint32_t keep = (p.bias != nullptr && r < p.E) ? 0xFFFFFFFFu : 0u;
    __asm__ volatile("" : "+v"(keep));
    v += static_cast<double>(__uint_as_float(__float_as_uint(b) & keep));
    if constexpr (GL) {
      // row E's sum, before this pass's stores (a wait after them would also wait
      // for their completion); every pass forms the same value
      gsum = 0.0;
      for (int ks = 0; ks < KS; ++ks) gsum += readlane_f64(gpart, ks);
    }
    if (r < p.E) {
      const float lf = static_cast<float>(v);
      s_logit[r] = lf;
      if (p.logits) p.logits[static_cast<size_t>(t) * p.E + r] = lf;
    } else if (p.gamma && p.shared_gate) {
      p.gamma[t] = static_cast<float>(1.0 / (1.0 + exp(-v)));
    }
  }
  if constexpr (GL) {  // thread 0 made at least one pass (E >= the thread count)
    if (threadIdx.x == 0 && p.gamma && p.shared_gate)
      p.gamma[t] = static_cast<float>(1.0 / (1.0 + exp(-gsum)));
  }
  __syncthreads();
  block_topk_rank<kTopkWaves>(p.E, p.k, [&](int e) { return s_logit[e]; }, s_key, s_cand, s_v,
                              s_ids);
  if (threadIdx.x < kWave) {
    const float wt = softmax_of_places(s_v, p.k);
    if (lane < p.k) {
      const size_t o = static_cast<size_t>(t) * p.k + lane;
      p.ids[o] = s_ids[lane];
      p.w[o] = wt;
      if (p.ids_copy) p.ids_copy[o] = s_ids[lane];
      if (p.w_copy) p.w_copy[o] = wt;
    }
  }
}


hipError_t launch_route_split(const RouteParams& p0, hipStream_t s) {
  RouteParams p = p0;
  p.ksplit = route_split_k(p.E, p.T, p.H);
  const int waves = route_split_waves(p.E + 1);
  dim3 grid((p.E + 1 + 16 * waves - 1) / (16 * waves),
            (p.T + kRouteSplitTokens - 1) / kRouteSplitTokens, p.ksplit);
  route_split_kernel<<<grid, waves * kWave, 0, s>>>(p);
  const dim3 tgrid(p.T), tblock(kTopkWaves * kWave);
  const bool gl = p.E % (kTopkWaves * kWave) == 0;
  switch (p.ksplit) {  // a power of two up to kRouteMaxSplits (route_split_k)
#define FTMOE_TOPK_SPLIT_CASE(ks)                                              \
  case ks:                                                                     \
    if (gl)                                                                    \
      topk_split_kernel<ks, true><<<tgrid, tblock, 0, s>>>(p);                 \
    else                                                                       \
      topk_split_kernel<ks, false><<<tgrid, tblock, 0, s>>>(p);                \
    break;
    FTMOE_TOPK_SPLIT_CASE(1) FTMOE_TOPK_SPLIT_CASE(2) FTMOE_TOPK_SPLIT_CASE(4)
    FTMOE_TOPK_SPLIT_CASE(8) FTMOE_TOPK_SPLIT_CASE(16) FTMOE_TOPK_SPLIT_CASE(32)
#undef FTMOE_TOPK_SPLIT_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int route_fused_topk_tokens() { return kRouteWaves; }

hipError_t launch_route(const RouteParams& p0, bool fuse_topk, hipStream_t s) {
  RouteParams p = p0;
  const int rows = p.E + (p.shared_gate ? 1 : 0);
  const int gx = rows > 0 ? (rows + kRouteWaves - 1) / kRouteWaves : 1;
  // tokens per wave: as few as keep about kRouteTargetWaves waves busy (each
  // wave keeps its row in registers across its tokens)
  const long long work = static_cast<long long>(rows > 0 ? rows : 1) * p.T;
  const int grp = route_token_group(p.H / (4 * kWave));
  p.tok_tile = static_cast<int>((work + kRouteTargetWaves - 1) / kRouteTargetWaves);
  p.tok_tile = (p.tok_tile + grp - 1) / grp * grp;  // whole token groups
  p.tok_tile = p.tok_tile < 1 ? 1 : (p.tok_tile > kRouteMaxTokTile ? kRouteMaxTokTile : p.tok_tile);
  dim3 grid(gx, (p.T + p.tok_tile - 1) / p.tok_tile);
  dim3 block(kRouteWaves * kWave);
  const int fuse = fuse_topk ? 1 : 0;
  switch (p.H / (4 * kWave)) {
#define FTMOE_ROUTE_CASE(n) \
  case n: route_logits_kernel<n><<<grid, block, 0, s>>>(p, fuse); break;
    FTMOE_ROUTE_CASE(1) FTMOE_ROUTE_CASE(2) FTMOE_ROUTE_CASE(3) FTMOE_ROUTE_CASE(4)
    FTMOE_ROUTE_CASE(5) FTMOE_ROUTE_CASE(6) FTMOE_ROUTE_CASE(7) FTMOE_ROUTE_CASE(8)
    FTMOE_ROUTE_CASE(9) FTMOE_ROUTE_CASE(10) FTMOE_ROUTE_CASE(11) FTMOE_ROUTE_CASE(12)
    FTMOE_ROUTE_CASE(13) FTMOE_ROUTE_CASE(14) FTMOE_ROUTE_CASE(15) FTMOE_ROUTE_CASE(16)
    FTMOE_ROUTE_CASE(17) FTMOE_ROUTE_CASE(18) FTMOE_ROUTE_CASE(19) FTMOE_ROUTE_CASE(20)
    FTMOE_ROUTE_CASE(21) FTMOE_ROUTE_CASE(22) FTMOE_ROUTE_CASE(23) FTMOE_ROUTE_CASE(24)
    FTMOE_ROUTE_CASE(25) FTMOE_ROUTE_CASE(26) FTMOE_ROUTE_CASE(27) FTMOE_ROUTE_CASE(28)
    FTMOE_ROUTE_CASE(29) FTMOE_ROUTE_CASE(30) FTMOE_ROUTE_CASE(31) FTMOE_ROUTE_CASE(32)
#undef FTMOE_ROUTE_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_route_mfma(const RouteParams& p, hipStream_t s) {
  dim3 grid((p.E + kRouteMmExperts - 1) / kRouteMmExperts,
            (p.T + kRouteMmTokens - 1) / kRouteMmTokens);
  route_mfma_kernel<<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_topk(const RouteParams& p, hipStream_t s) {
  if (p.T <= kTopkBlockMaxTokens) {
    topk_block_kernel<<<dim3(p.T), dim3(kTopkWaves * kWave), 0, s>>>(p);
  } else {
    dim3 grid((p.T + kRouteWaves - 1) / kRouteWaves);
    topk_kernel<<<grid, dim3(kRouteWaves * kWave), 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace ftmoe
