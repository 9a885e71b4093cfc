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

// ------------------------------------------- many tokens: bounded approximation --
//
// The router of the pages sums each logit in fp64 and rounds it once to fp32; the
// k largest win, ties to the lower index.  For thousands of tokens the fp64 MFMA
// product of every (token, expert) pair is replaced by three steps that select
// exactly the same experts with exactly the same logits:
//  1. route_prep_kernel: each fp32 router row w is split into two bf16 pieces,
//     hi = bf16(w) and mid = bf16(w - hi) (nearest-even, so |w - hi - mid| <=
//     2^-16 |w|), and its 2-norm is taken in fp64 and rounded up.
//  2. route_approx_kernel: A[t][e] = fp32(x_t . (hi_e + mid_e)) + bias_e, a bf16
//     MFMA product (x is bf16, so every product is exact) accumulated in fp32.
//  3. route_recheck_kernel, one wave per token: a rigorous bound d_e >= |A[t][e] -
//     logit[t][e]| (below); theta = the k-th largest of A - d; every expert with
//     A + d >= theta keeps its place as a candidate (no other one can be among the
//     k largest logits, nor tie with them); the candidates' logits are computed
//     exactly as the other routers do (fp64 sum, one fp32 rounding) and the top k
//     of those are selected.  A token whose approximations or bound are not finite
//     (NaN or infinite inputs) takes every expert as a candidate.
//
// The bound.  The 2H products of step 2 are exact; any order of fp32 additions,
// each with relative error <= 2^-23 (so truncation is covered too), errs by at most
// g_n * sum|terms|, g_n = n 2^-23 / (1 - n 2^-23) with n = 2H, and sum|terms| <=
// (1 + 2^-7) sum_h |x_h| |w_h| <= (1 + 2^-7) ||x_t|| ||w_e|| (Cauchy-Schwarz).  The
// dropped third piece adds 2^-16 ||x_t|| ||w_e||, the bias addition and the final
// rounding of the exact logit at most 2^-22 |A| between them.  Step 3 takes
// d = 1.25 (g_n (1 + 2^-7) + 2^-16) ||x_t|| ||w_e|| + 2^-21 |A| + 2^-120.

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 rb_bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float rb_f32x4;
typedef unsigned int rb_u32x4 __attribute__((ext_vector_type(4)));

// the largest of the wave's 64 values (every lane gets it); no NaN among them
__device__ __forceinline__ double wave_max_f64(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const double o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

// One wave per router row: the two bf16 pieces and the row's 2-norm (rounded up).
__global__ __launch_bounds__(256) void route_prep_kernel(RouteParams p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int e = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (e >= p.E) return;
  const int H = p.H;
  const float* row = p.wr + static_cast<size_t>(e) * H;
  uint16_t* hi = p.wsplit + static_cast<size_t>(e) * 2 * H;
  uint16_t* mid = hi + H;
  double ss = 0.0;
  for (int k = 8 * lane; k < H; k += 8 * kWave) {  // H % 8 == 0: whole groups of 8
    const float4 a = *reinterpret_cast<const float4*>(row + k);
    const float4 b = *reinterpret_cast<const float4*>(row + k + 4);
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t h[4], m[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t hp = 0, mp = 0;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float w = v[2 * i + j];
        const uint32_t hb = f32_to_bf16_bits(w);
        const uint32_t mb = f32_to_bf16_bits(w - __uint_as_float(hb << 16));
        hp |= hb << (16 * j);
        mp |= mb << (16 * j);
        ss = fma(static_cast<double>(w), static_cast<double>(w), ss);
      }
      h[i] = hp;
      m[i] = mp;
    }
    *reinterpret_cast<uint4*>(hi + k) = make_uint4(h[0], h[1], h[2], h[3]);
    *reinterpret_cast<uint4*>(mid + k) = make_uint4(m[0], m[1], m[2], m[3]);
  }
  ss = wave_sum_f64(ss);
  if (lane == 0) {
    // sqrt in fp64 (error far below the factor), widened, rounded up to fp32
    const double n = sqrt(ss) * (1.0 + 0x1p-40);
    float f = static_cast<float>(n);
    if (static_cast<double>(f) < n) f = __uint_as_float(__float_as_uint(f) + 1u);  // next up (n >= 0)
    p.wnorm[e] = f;
  }
}

// A[t][e] for a block of 64 experts x 256 tokens, 4 waves of 64 tokens each.  The
// block's 64 rows (both pieces) are staged in LDS, 64 K at a time, and shared by
// the 4 waves; each wave takes its own tokens straight from global memory into
// registers (nothing to share), a stage ahead.  A wave computes 4 x 4 fragments of
// 16 x 16 with both pieces of a row into the same fp32 accumulator.  Rows and
// tokens past the end repeat the last one (their results are not stored).
constexpr int kApproxE = 64;         // experts per block
constexpr int kApproxT = 128;        // tokens per block (32 per wave)
constexpr int kApproxFB = kApproxT / (4 * 16);  // token fragments per wave
constexpr int kApproxRowU4 = 8 + 1;  // 16-byte words of a staged row of 64 K (one of padding)

__global__ __launch_bounds__(256) void route_approx_kernel(RouteParams p) {
  __shared__ uint4 sa[2][2 * kApproxE * kApproxRowU4];  // [stage][(piece * 64 + row) * 9 + word]
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = p.H;
  const int e0 = blockIdx.x * kApproxE;
  const int t0 = blockIdx.y * kApproxT + 16 * kApproxFB * wave;
  const int i = lane & 15, g = lane >> 4;
  // staging: thread tid moves words tid + 256 j (j < 4) of the stage: row (w >> 4),
  // piece ((w >> 3) & 1), word (w & 7) of the row's 64 K
  const uint16_t* asrc[4];
  int adst[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int w = tid + 256 * j;
    const int row = w >> 4, pc = (w >> 3) & 1, c8 = w & 7;
    asrc[j] = p.wsplit + static_cast<size_t>(min(e0 + row, p.E - 1)) * 2 * H + pc * H + 8 * c8;
    adst[j] = (pc * kApproxE + row) * kApproxRowU4 + c8;
  }
  const uint16_t* bsrc[kApproxFB];
#pragma unroll
  for (int f = 0; f < kApproxFB; ++f)
    bsrc[f] = p.x + static_cast<size_t>(min(t0 + 16 * f + i, p.T - 1)) * H + 8 * g;
  rb_f32x4 acc[4][kApproxFB];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < kApproxFB; ++b) acc[a][b] = rb_f32x4{0.f, 0.f, 0.f, 0.f};
  rb_u32x4 ra[4];  // native vectors: a copy of HIP's uint4 between memory spaces stays a memcpy
  uint4 rb[2][kApproxFB][2];
  auto load_a = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) ra[j] = *reinterpret_cast<const rb_u32x4*>(asrc[j] + k0);
  };
  auto load_b = [&](int k0, uint4 (&dst)[kApproxFB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < kApproxFB; ++f)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) dst[f][ks] = *reinterpret_cast<const uint4*>(bsrc[f] + k0 + 32 * ks);
  };
  auto store_a = [&](uint4* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) reinterpret_cast<rb_u32x4*>(dst)[adst[j]] = ra[j];
  };
  auto compute = [&](const uint4* sa_cur, const uint4 (&b)[kApproxFB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 af[2][4];
#pragma unroll
      for (int pc = 0; pc < 2; ++pc)
#pragma unroll
        for (int fa = 0; fa < 4; ++fa)
          af[pc][fa] = sa_cur[(pc * kApproxE + 16 * fa + i) * kApproxRowU4 + 4 * ks + g];
#pragma unroll
      for (int pc = 0; pc < 2; ++pc)
#pragma unroll
        for (int fa = 0; fa < 4; ++fa)
#pragma unroll
          for (int fb = 0; fb < kApproxFB; ++fb)
            acc[fa][fb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(rb_bf16x8, af[pc][fa]), __builtin_bit_cast(rb_bf16x8, b[fb][ks]),
                acc[fa][fb], 0, 0, 0);
    }
  };
  const int ns = H / 64;  // stages; H % 256 == 0, so ns is even
  load_a(0);
  load_b(0, rb[0]);
  store_a(sa[0]);
  __syncthreads();
  // two stages per pass, so that the stage buffers are compile-time indices
  for (int s = 0; s < ns; s += 2) {
    // stage s (buffer 0); stage s + 1's loads in flight
    load_a(64 * (s + 1));
    load_b(64 * (s + 1), rb[1]);
    compute(sa[0], rb[0]);
    store_a(sa[1]);
    __syncthreads();
    // stage s + 1 (buffer 1); stage s + 2's loads in flight (the last pass reloads
    // stage s + 1, in range and never used)
    const int kn = s + 2 < ns ? 64 * (s + 2) : 64 * (s + 1);
    load_a(kn);
    load_b(kn, rb[0]);
    compute(sa[1], rb[1]);
    if (s + 2 < ns) store_a(sa[0]);
    __syncthreads();
  }
  // C lane l: expert rows 4 (l / 16) + r of the fragment, token l % 16
#pragma unroll
  for (int fb = 0; fb < kApproxFB; ++fb) {
    const int t = t0 + 16 * fb + i;
    if (t >= p.T) continue;
    float* out = p.logits + static_cast<size_t>(t) * p.E;
#pragma unroll
    for (int fa = 0; fa < 4; ++fa)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = e0 + 16 * fa + 4 * g + r;
        if (e < p.E) out[e] = acc[fa][fb][r] + (p.bias ? p.bias[e] : 0.0f);
      }
  }
}

// One wave per token (see the section comment).  NC = H / 256 float4 pieces of a
// row per lane, the token's activations held in registers in fp64, or 0: any H,
// the activations re-read (from L1) for each candidate.  SL = slots of experts per
// lane (E <= 64 SL).  With at most 64 candidates (the usual case) each lane holds
// one candidate and the top k are found by counting, for each candidate, the
// candidates above it (keys (rank_key(logit), ~expert): unique, larger wins, ties to
// the lower index); otherwise every candidate's logit goes into its slot and the
// wave's slot top-k selects.  Either way the weights are the softmax of the
// selected logits exactly as the other routers take it.
template <int NC, int SL>
__global__ __launch_bounds__(kRouteWaves* kWave) void route_recheck_kernel(RouteParams p, float cbound) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int t = blockIdx.x * kRouteWaves + __builtin_amdgcn_readfirstlane(wv);
  if (t >= p.T) return;
  const int H = p.H, E = p.E, k = p.k;
  const int nc = NC > 0 ? NC : H / (4 * kWave);
  const uint16_t* __restrict__ xt = p.x + static_cast<size_t>(t) * H;
  const float* __restrict__ at = p.logits + static_cast<size_t>(t) * E;
  float av[SL], wn[SL];
#pragma unroll
  for (int m = 0; m < SL; ++m) {
    const int e = min(lane + kWave * m, E - 1);
    av[m] = at[e];
    wn[m] = p.wnorm[e];
  }
  // the token's activations (in fp64 when held) and 2-norm, rounded up
  double xd[NC > 0 ? NC : 1][4];
  auto xpiece = [&](int c) -> uint2 { return *reinterpret_cast<const uint2*>(xt + 4 * lane + 4 * kWave * c); };
  auto widen = [&](uint2 x2, double (&o)[4]) {
    o[0] = bf16_bits_to_f32(x2.x & 0xFFFFu);
    o[1] = bf16_bits_to_f32(x2.x >> 16);
    o[2] = bf16_bits_to_f32(x2.y & 0xFFFFu);
    o[3] = bf16_bits_to_f32(x2.y >> 16);
  };
  double ss = 0.0;
  if constexpr (NC > 0) {
    uint2 xr[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) xr[c] = xpiece(c);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      widen(xr[c], xd[c]);
#pragma unroll
      for (int q = 0; q < 4; ++q) ss = fma(xd[c][q], xd[c][q], ss);
    }
  } else {
    for (int c = 0; c < nc; ++c) {
      double o[4];
      widen(xpiece(c), o);
#pragma unroll
      for (int q = 0; q < 4; ++q) ss = fma(o[q], o[q], ss);
    }
  }
  const double xnd = sqrt(wave_sum_f64(ss)) * (1.0 + 0x1p-40);
  float xn = static_cast<float>(xnd);
  if (static_cast<double>(xn) < xnd) xn = __uint_as_float(__float_as_uint(xn) + 1u);  // up
  // bounds in fp32: the bound's own roundings (a few 2^-24 relative) are covered by
  // the (1 + 2^-20) on its first term and 2^-20 instead of 2^-21 on |A|
  float lo[SL], hi[SL];
  bool finite = __builtin_isfinite(xn);
#pragma unroll
  for (int m = 0; m < SL; ++m) {
    const bool valid = lane + kWave * m < E;
    const float a = av[m];
    const float d = (cbound * xn * wn[m]) * (1.0f + 0x1p-20f) + 0x1p-20f * __builtin_fabsf(a) + 0x1p-120f;
    lo[m] = valid ? a - d : -__builtin_inff();
    hi[m] = a + d;
    if (valid) finite = finite && __builtin_isfinite(a) && __builtin_isfinite(d);
  }
  const bool all = __ballot(!finite) != 0;  // a non-finite value: every expert a candidate
  float theta = -__builtin_inff();
  if (!all) {
    // k rounds on rank keys: the largest remaining lower end, one instance removed
    uint32_t rk[SL];
#pragma unroll
    for (int m = 0; m < SL; ++m) rk[m] = rank_key(lo[m]);  // -inf (past E) still ranks
    uint32_t kth = 0;
    for (int r = 0; r < k; ++r) {
      uint32_t lm = rk[0];
#pragma unroll
      for (int m = 1; m < SL; ++m) lm = rk[m] > lm ? rk[m] : lm;
      kth = wave_max_u32(lm);
      const uint64_t holders = __ballot(lm == kth);
      if (lane == __ffsll(static_cast<unsigned long long>(holders)) - 1) {
        bool done = false;
#pragma unroll
        for (int m = 0; m < SL; ++m)
          if (!done && rk[m] == kth) {
            rk[m] = 0u;
            done = true;
          }
      }
    }
    theta = key_value(kth);
  }
  // candidates, listed in LDS in expert order
  __shared__ int s_list[kRouteWaves][kMaxExperts];
  int* list = s_list[wv];
  int n = 0;
#pragma unroll
  for (int m = 0; m < SL; ++m) {
    const bool c = (lane + kWave * m < E) && (all || hi[m] >= theta);
    const uint64_t bits = __ballot(c);
    if (c) list[n + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bits >> 32),
                                               __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bits), 0))] =
        lane + kWave * m;
    n += __builtin_popcountll(bits);
  }
  wave_lds_sync();
  // exact logit of expert e, as the row router sums it (per lane in piece order,
  // then the wave's fixed tree), CB experts at a time with their loads together
  constexpr int CB = 2;
  auto exact = [&](const int (&ce)[CB], float (&out)[CB]) {
    double acc[CB];
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[j] = 0.0;
    if constexpr (NC > 0) {
      float4 w4[CB][NC];
#pragma unroll
      for (int j = 0; j < CB; ++j)
#pragma unroll
        for (int c = 0; c < NC; ++c)
          w4[j][c] = *reinterpret_cast<const float4*>(p.wr + static_cast<size_t>(ce[j]) * H + 4 * lane + 4 * kWave * c);
#pragma unroll
      for (int j = 0; j < CB; ++j)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          acc[j] = fma(static_cast<double>(w4[j][c].x), xd[c][0], acc[j]);
          acc[j] = fma(static_cast<double>(w4[j][c].y), xd[c][1], acc[j]);
          acc[j] = fma(static_cast<double>(w4[j][c].z), xd[c][2], acc[j]);
          acc[j] = fma(static_cast<double>(w4[j][c].w), xd[c][3], acc[j]);
        }
    } else {
      for (int c = 0; c < nc; ++c) {
        double o[4];
        widen(xpiece(c), o);
#pragma unroll
        for (int j = 0; j < CB; ++j) {
          const float4 w = *reinterpret_cast<const float4*>(p.wr + static_cast<size_t>(ce[j]) * H + 4 * lane + 4 * kWave * c);
          acc[j] = fma(static_cast<double>(w.x), o[0], acc[j]);
          acc[j] = fma(static_cast<double>(w.y), o[1], acc[j]);
          acc[j] = fma(static_cast<double>(w.z), o[2], acc[j]);
          acc[j] = fma(static_cast<double>(w.w), o[3], acc[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      double v = wave_sum_f64(acc[j]);
      if (p.bias) v += static_cast<double>(p.bias[ce[j]]);
      out[j] = static_cast<float>(v);
    }
  };
  auto batch = [&](int j0, int (&ce)[CB]) {
#pragma unroll
    for (int j = 0; j < CB; ++j)
      ce[j] = __builtin_amdgcn_readfirstlane(list[j0 + j < n ? j0 + j : n - 1]);  // past the end: repeat
  };
  int id = -1;
  float wt = 0.0f;
  if (!all && n <= kWave) {
    // lane j: candidate j
    float cv = 0.0f;
    for (int j0 = 0; j0 < n; j0 += CB) {
      int ce[CB];
      float v[CB];
      batch(j0, ce);
      exact(ce, v);
#pragma unroll
      for (int j = 0; j < CB; ++j)
        if (lane == j0 + j) cv = v[j];
    }
    const int ce_mine = lane < n ? list[lane] : 0;
    const uint64_t key = lane < n ? (static_cast<uint64_t>(rank_key(cv)) << 32) |
                                        static_cast<uint32_t>(~ce_mine)
                                  : 0ull;
    int above = 0;
    for (int i = 0; i < n; ++i) {
      const uint64_t ki = (static_cast<uint64_t>(static_cast<uint32_t>(
                               __builtin_amdgcn_readlane(static_cast<int>(key >> 32), i)))
                           << 32) |
                          static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(key), i));
      above += ki > key ? 1 : 0;
    }
    // place r -> lane r: the candidate with r candidates above it
    __shared__ int s_pid[kRouteWaves][kTopkMaxK];
    __shared__ float s_pv[kRouteWaves][kTopkMaxK];
    if (lane < n && above < k) {
      s_pid[wv][above] = ce_mine;
      s_pv[wv][above] = key_value(rank_key(cv));
    }
    wave_lds_sync();
    const double vd = lane < k ? static_cast<double>(s_pv[wv][lane]) : 0.0;
    const double top = readlane_f64(vd, 0);
    const double dd = lane < k ? exp(vd - top) : 0.0;
    double sum = 0.0;
    for (int i = 0; i < k; ++i) sum += readlane_f64(dd, i);
    if (lane < k) {
      id = s_pid[wv][lane];
      wt = static_cast<float>(dd / sum);
    }
  } else {
    float lv[SL];
#pragma unroll
    for (int m = 0; m < SL; ++m) lv[m] = -__builtin_inff();
    for (int j0 = 0; j0 < n; j0 += CB) {
      int ce[CB];
      float v[CB];
      batch(j0, ce);
      exact(ce, v);
#pragma unroll
      for (int j = 0; j < CB; ++j)
        if (j0 + j < n) {
#pragma unroll
          for (int m = 0; m < SL; ++m)
            if (lane + kWave * m == ce[j]) lv[m] = v[j];
        }
    }
    wave_topk_vals<SL>(E, k, lv, &id, &wt);
  }
  if (lane < k) {
    const size_t o = static_cast<size_t>(t) * k + lane;
    p.ids[o] = id;
    p.w[o] = wt;
    if (p.ids_copy) p.ids_copy[o] = id;
    if (p.w_copy) p.w_copy[o] = wt;
  }
}

// 1.25 (g_n (1 + 2^-7) + 2^-16) for n = 2H products (see the section comment)
static float route_bound_factor(int H) {
  const double nu = 2.0 * H * 0x1p-23;
  return static_cast<float>(1.25 * (nu / (1.0 - nu) * (1.0 + 0x1p-7) + 0x1p-16));
}


hipError_t launch_route_bounded(const RouteParams& p, hipStream_t s) {
  if (p.T <= 0) return hipSuccess;
  route_prep_kernel<<<dim3((p.E + 3) / 4), dim3(256), 0, s>>>(p);
  route_approx_kernel<<<dim3((p.E + kApproxE - 1) / kApproxE, (p.T + kApproxT - 1) / kApproxT),
                        dim3(256), 0, s>>>(p);
  const float cb = route_bound_factor(p.H);
  const dim3 grid((p.T + kRouteWaves - 1) / kRouteWaves), block(kRouteWaves * kWave);
  const int nc = p.H / (4 * kWave);
  const int sl = p.E <= 4 * kWave ? 4 : (p.E <= 8 * kWave ? 8 : 16);
#define FTMOE_RECHECK(NCV)                                                         \
  if (sl == 4) route_recheck_kernel<NCV, 4><<<grid, block, 0, s>>>(p, cb);        \
  else if (sl == 8) route_recheck_kernel<NCV, 8><<<grid, block, 0, s>>>(p, cb);   \
  else route_recheck_kernel<NCV, 16><<<grid, block, 0, s>>>(p, cb);
  if (nc == 4) {
    FTMOE_RECHECK(4)
  } else if (nc == 8) {
    FTMOE_RECHECK(8)
  } else if (nc == 16) {
    FTMOE_RECHECK(16)
  } else {
    FTMOE_RECHECK(0)
  }
#undef FTMOE_RECHECK
  return hipGetLastError();
}

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
