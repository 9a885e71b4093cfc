// route_group.hip -- the routing of a decode batch (8..64 tokens) in ONE
// persistent launch on gfx950: router logits, top-k with softmax weights, and the
// grouping of the (token, slot) pairs by expert that the grouped expert kernels
// read.
//
// FreeToken commit log (page 2): the router / shared-gate kernel entry and the
// top-k entry (k need not be a power of two).  FreeToken fork PR #84 (page 1),
// bullet on #631: the decode GEMV on the per-token path of every MoE layer; for a
// batch of tokens each selected expert's weights are read once for all of its
// tokens, which needs the pairs grouped by expert before the expert kernels start.
//
// As three kernels (split router, top-k, grouping) the routing paid three launches
// and a memory round trip between each, for a few tens of MFLOP of fp64 work.
// Here one block per CU runs every phase, and values cross between blocks as
// generation-tagged words (handoff.hpp):
//   R  block (row tile, K split): the fp64 MFMA product (v_mfma_f64_16x16x4f64) of
//      16 router rows with every token over H / KS of K, the block's waves
//      splitting that range further; the waves' sums are added in wave order in
//      LDS and the block's partial sums published tagged (an fp64 value as two
//      tagged words: its low and high halves).
//   Q  the same block, for a KS-th of the tokens: the logits of its row tile = the
//      KS partial sums added in split order, plus the bias in fp64, rounded once
//      to fp32, published tagged.
//   S  block t < T: token t's logits, polled; rank-count top-k; softmax
//      weights of the selected logits; ids and weights stored for the expert
//      kernels (over a slot bank: slot ids, a non-resident expert becoming slot 0
//      with weight 0) and the ids published tagged.  Blocks T .. 2T-1: the shared
//      gate of token b - T (read only by the expert kernels: no hand-off).
//   G  the last block: the T * k ids, polled; per-expert counts, the work-unit
//      table and the pairs scattered into per-expert groups (LDS cursors).
// The blocks share the per-block call counters of the one-launch decode kernel:
// both launch one block per CU and every block counts every call, so a call's
// generation is new whichever kernel ran before it on the workspace.
#include "ftmoe_device.hpp"
#include "ftmoe_kernels.hpp"
#include "handoff.hpp"

namespace ftmoe {

namespace {

constexpr int kRgWaves = 8;
constexpr int kRgThreads = kRgWaves * kWave;
constexpr int kRgMaxSplits = 8;
constexpr int kRgPieces = 4;  // 16-K pieces of a wave in flight at once
constexpr int kRgHalf = kRgWaves / 2;
constexpr int kQWaitSpins = 1 << 14;  // LDS polls of the block's Q-done flag, at most

typedef __attribute__((__vector_size__(4 * sizeof(double)))) double rg_f64x4;

__device__ __forceinline__ void st_tag_u32(uint64_t* p, uint32_t v, uint32_t gen) {
  __hip_atomic_store(p, (static_cast<uint64_t>(gen) << 32) | v, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// fp64 dot product of the bf16 vector gv with the bf16 row xt (the wave's sum)
__device__ double wave_dot_bf16_f64(const uint16_t* gv, const uint16_t* xt, int H) {
  const int lane = threadIdx.x & (kWave - 1);
  double acc = 0.0;
  for (int k0 = 4 * lane; k0 < H; k0 += 4 * kWave) {
    const uint2 a = *reinterpret_cast<const uint2*>(gv + k0);
    const uint2 b = *reinterpret_cast<const uint2*>(xt + k0);
    acc = fma(static_cast<double>(bf16_bits_to_f32(a.x & 0xFFFFu)),
              static_cast<double>(bf16_bits_to_f32(b.x & 0xFFFFu)), acc);
    acc = fma(static_cast<double>(bf16_bits_to_f32(a.x >> 16)),
              static_cast<double>(bf16_bits_to_f32(b.x >> 16)), acc);
    acc = fma(static_cast<double>(bf16_bits_to_f32(a.y & 0xFFFFu)),
              static_cast<double>(bf16_bits_to_f32(b.y & 0xFFFFu)), acc);
    acc = fma(static_cast<double>(bf16_bits_to_f32(a.y >> 16)),
              static_cast<double>(bf16_bits_to_f32(b.y >> 16)), acc);
  }
  return wave_sum_f64(acc);
}

}  // namespace

// NTT: 16-token tiles of the call (T <= 16 NTT).
template <int NTT>
__global__ __launch_bounds__(kRgThreads, 1) void route_group_kernel(RouteGroupParams p) {
  __shared__ double s_acc[kRgWaves][4 * NTT][kWave];  // the waves' MFMA sums (R)
  __shared__ float s_logit[kMaxExperts];
  __shared__ __align__(16) uint64_t s_key[kRgWaves][kWave];
  __shared__ __align__(16) uint64_t s_cand[kTopkMaxChunks * kTopkMaxK];
  __shared__ double s_v[kTopkMaxK];
  __shared__ int s_ids[kTopkMaxK];
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_cur[kMaxExperts];
  __shared__ int s_wa[kRgWaves], s_wb[kRgWaves];
  __shared__ uint32_t s_qdone;  // this call's generation once the block's Q stage is out

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = static_cast<int>(threadIdx.x);
  const int G = static_cast<int>(gridDim.x), b = static_cast<int>(blockIdx.x);
  const int T = p.T, E = p.E, H = p.H, k = p.k, KS = p.ksplit;
  // this block's call count + 1 (stored back at the end of the block's work)
  const uint32_t gen = ld_dev(&p.gen[b]) + 1u;

  // ---------------------------------------------------------------- R --
  {
    const int nrt = (E + 15) / 16;
    const int kc = H / KS;
    const int npc = kc / 16;  // 16-K pieces of one split
    const int i = lane & 15, g = lane >> 4;
    for (int task = b; task < nrt * KS; task += G) {
      const int rt = task % nrt, ks = task / nrt;
      // rows and tokens past the end repeat the last (their sums are not published)
      const float* wrow = p.wr + static_cast<size_t>(min(rt * 16 + i, E - 1)) * H + ks * kc + 4 * g;
      const uint16_t* xrow[NTT];
#pragma unroll
      for (int f = 0; f < NTT; ++f)
        xrow[f] = p.x + static_cast<size_t>(min(16 * f + i, T - 1)) * H + ks * kc + 4 * g;
      rg_f64x4 acc[NTT];
#pragma unroll
      for (int f = 0; f < NTT; ++f) acc[f] = rg_f64x4{0.0, 0.0, 0.0, 0.0};
      // piece j of the split: K = 16 j + 4 g + m (m = 0..3) for lane group g, in A
      // (router row i) and B (token i) alike; wave w takes pieces w, w + 8, ...
      for (int j0 = wave; j0 < npc; j0 += kRgPieces * kRgWaves) {
        float4 wv[kRgPieces];
        uint2 xv[kRgPieces][NTT];
#pragma unroll
        for (int u = 0; u < kRgPieces; ++u) {
          const int j = j0 + u * kRgWaves;
          if (j < npc) {
            wv[u] = *reinterpret_cast<const float4*>(wrow + 16 * j);
#pragma unroll
            for (int f = 0; f < NTT; ++f)
              xv[u][f] = *reinterpret_cast<const uint2*>(xrow[f] + 16 * j);
          }
        }
#pragma unroll
        for (int u = 0; u < kRgPieces; ++u) {
          const int j = j0 + u * kRgWaves;
          if (j < npc) {
            const float wa[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              const double a = static_cast<double>(wa[m]);
#pragma unroll
              for (int f = 0; f < NTT; ++f) {
                const uint32_t pair = (m < 2) ? xv[u][f].x : xv[u][f].y;
                const double bv = static_cast<double>(
                    bf16_bits_to_f32((m & 1) ? (pair >> 16) : (pair & 0xFFFFu)));
                acc[f] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bv, acc[f], 0, 0, 0);
              }
            }
          }
        }
      }
      // C lane l: rows 16 rt + l / 16 + 4 jj of token 16 f + l % 16
#pragma unroll
      for (int f = 0; f < NTT; ++f)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) s_acc[wave][4 * f + jj][lane] = acc[f][jj];
      __syncthreads();
      // The block's sums, stored by waves 0 .. 3 only (waves 4 .. 7 then poll in Q
      // with no stores of their own in flight: a wave's loads complete only after
      // every store it issued before them), into the task's slab
      // part[ks][rt][r][t][low, high] (r = row in the tile): the 16 lanes of one row
      // write 16 consecutive tokens, so a store instruction covers 4 runs of 256 bytes.
      uint64_t* slab = p.part + (static_cast<size_t>(ks) * nrt + rt) * 16 * T * 2;
      for (int v = tid; wave < kRgHalf && v < NTT * 4 * kWave; v += kRgHalf * kWave) {
        const int q = v / kWave, l = v % kWave;
        const int f = q / 4, jj = q % 4;
        double sum = s_acc[0][q][l];
#pragma unroll
        for (int w = 1; w < kRgWaves; ++w) sum += s_acc[w][q][l];
        const int t = 16 * f + (l & 15), r = (l >> 4) + 4 * jj;
        if (t < T && rt * 16 + r < E) {
          const uint64_t bits = static_cast<uint64_t>(__double_as_longlong(sum));
          uint64_t* dst = slab + (static_cast<size_t>(r) * T + t) * 2;
          st_tag_u32(dst, static_cast<uint32_t>(bits), gen);
          st_tag_u32(dst + 1, static_cast<uint32_t>(bits >> 32), gen);
        }
      }
      if (task + G < nrt * KS) __syncthreads();  // s_acc is rewritten by the next task
    }
  }

  // ---------------------------------------------------------------- Q --
  // Task (rt, ks) also finishes the logits of row tile rt for tokens
  // [ks tpr, (ks + 1) tpr): the KS partial sums added in split order, the bias in
  // fp64, one fp32 rounding, published tagged.  A lane per (row, token), all of
  // its loads in flight at once: the hand-off to the selecting blocks is then one
  // word per logit, and these partial sums are read once, spread over every CU.
  {
    const int nrt = (E + 15) / 16;
    const int tpr = (T + KS - 1) / KS;
    const float* bsrc = p.bias ? p.bias : p.wr;  // masked off below when there is no bias
    for (int task = b; task < nrt * KS; task += G) {
      const int rt = task % nrt, ks = task / nrt;
      for (int v = tid - kRgHalf * kWave; wave >= kRgHalf && v < 16 * tpr; v += kRgHalf * kWave) {
        const int t = ks * tpr + v % tpr, row = rt * 16 + v / tpr;
        const bool mine = t < T && row < E;
        // value (r, t) of split sp: words 2 (r T + t), + 1 of slab part[sp][rt]
        const uint64_t* src = p.part + static_cast<size_t>(rt) * 16 * T * 2 +
                              (static_cast<size_t>(v / tpr) * T + min(t, T - 1)) * 2;
        const size_t split_stride = static_cast<size_t>(nrt) * 16 * T * 2;
        uint64_t wd[kRgMaxSplits][2];
#pragma unroll
        for (int sp = 0; sp < kRgMaxSplits; ++sp)
          if (sp < KS) {
            wd[sp][0] = ld_tag(src + sp * split_stride);
            wd[sp][1] = ld_tag(src + sp * split_stride + 1);
          }
        const float bias = bsrc[min(row, E - 1)];
        for (int spins = 0;; ++spins) {
          bool ok = true;
#pragma unroll
          for (int sp = 0; sp < kRgMaxSplits; ++sp)
            if (sp < KS) ok = ok && tag_is(wd[sp][0], gen) && tag_is(wd[sp][1], gen);
          if (__ballot(mine && !ok) == 0) break;
          if (stop_waiting(spins, p.spin_limit, p.err, gen, kWaitLogits)) break;
          __builtin_amdgcn_s_sleep(1);
#pragma unroll
          for (int sp = 0; sp < kRgMaxSplits; ++sp)
            if (sp < KS) {
              if (!tag_is(wd[sp][0], gen)) wd[sp][0] = ld_tag(src + sp * split_stride);
              if (!tag_is(wd[sp][1], gen)) wd[sp][1] = ld_tag(src + sp * split_stride + 1);
            }
        }
        double sum = 0.0;
#pragma unroll
        for (int sp = 0; sp < kRgMaxSplits; ++sp)
          if (sp < KS) {
            const uint64_t bits = (wd[sp][0] & 0xFFFFFFFFull) | (wd[sp][1] << 32);
            sum += __longlong_as_double(static_cast<long long>(bits));
          }
        if (p.bias) sum += static_cast<double>(bias);
        if (mine) st_tag(&p.lg[static_cast<size_t>(t) * E + row], static_cast<float>(sum), gen);
      }
    }
    if (wave == kRgHalf && lane == 0)
      __hip_atomic_store(&s_qdone, gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }

  // ---------------------------------------------------------------- S --
  if (b < T && wave < kRgHalf) {
    // token b's logits (e = tid + 256 r), polled by waves 0 .. 3 (their R stores
    // are long done) once this block's own Q stage is (when the other blocks' are
    // due too; polling earlier only adds device-coherent traffic), until tagged
    for (int sp = 0; sp < kQWaitSpins; ++sp) {
      if (__hip_atomic_load(&s_qdone, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == gen) break;
      __builtin_amdgcn_s_sleep(2);
    }
    constexpr int kRows = kMaxExperts / (kRgHalf * kWave);
    const uint64_t* lg = p.lg + static_cast<size_t>(b) * E;
    uint64_t wd[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) wd[r] = ld_tag(lg + min(tid + r * kRgHalf * kWave, E - 1));
    for (int spins = 0;; ++spins) {
      bool ok = true;
#pragma unroll
      for (int r = 0; r < kRows; ++r)
        ok = ok && (tid + r * kRgHalf * kWave >= E || tag_is(wd[r], gen));
      if (__ballot(!ok) == 0) break;
      if (stop_waiting(spins, p.spin_limit, p.err, gen, kWaitLogits)) break;
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int r = 0; r < kRows; ++r)
        if (!tag_is(wd[r], gen)) wd[r] = ld_tag(lg + min(tid + r * kRgHalf * kWave, E - 1));
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r)
      if (tid + r * kRgHalf * kWave < E) s_logit[tid + r * kRgHalf * kWave] = tag_value(wd[r]);
  }
  if (b < T) {
    const int t = b;
    __syncthreads();
    block_topk_rank<kRgWaves>(E, k, [&](int e) { return s_logit[e]; }, s_key, s_cand, s_v, s_ids);
    if (wave == 0) {
      const float wt = softmax_of_places(s_v, k);
      if (lane < k) {
        const int o = t * k + lane;
        const int e = s_ids[lane];
        if (p.ids_copy) p.ids_copy[o] = e;
        if (p.w_copy) p.w_copy[o] = wt;
        int id = e;
        float w = wt;
        if (p.slot_of) {
          const int sl = p.slot_of[e];
          const bool present = sl >= 0 && sl < p.n_slots;
          id = present ? sl : 0;
          w = present ? wt : 0.0f;
          if (p.miss_out) p.miss_out[o] = present ? -1 : e;
        }
        p.ids[o] = id;
        p.w[o] = w;
        if (p.group) st_tag_u32(&p.tids[o], static_cast<uint32_t>(id), gen);
      }
    }
  } else if (b < 2 * T) {
    // the shared expert's gate of token b - T: sigmoid of the fp64 dot product
    if (wave == 0 && p.gamma && p.shared_gate) {
      const int t = b - T;
      const double z = wave_dot_bf16_f64(p.shared_gate, p.x + static_cast<size_t>(t) * H, H);
      if (lane == 0) p.gamma[t] = static_cast<float>(1.0 / (1.0 + exp(-z)));
    }
  }

  // ---------------------------------------------------------------- G --
  if (p.group && b == G - 1) {
    const int P = T * k;
    const int EG = p.n_group;  // experts (or slots) of the grouping
    constexpr int kPer = kMaxDecodeTokens * kMaxTopK / kRgThreads;  // pairs per thread
    int ev[kPer];
    for (int e = tid; e < kMaxExperts; e += kRgThreads) s_cnt[e] = 0;
    // the pairs' ids, polled (past P: a word that already carries the tag)
    {
      uint64_t wq[kPer];
#pragma unroll
      for (int jq = 0; jq < kPer; ++jq) {
        const int pr = tid + jq * kRgThreads;
        wq[jq] = pr < P ? ld_tag(&p.tids[pr]) : (static_cast<uint64_t>(gen) << 32);
      }
      for (int spins = 0;; ++spins) {
        bool ok = true;
#pragma unroll
        for (int jq = 0; jq < kPer; ++jq) ok = ok && tag_is(wq[jq], gen);
        if (__syncthreads_and(ok)) break;
        if (__syncthreads_or(stop_waiting(spins, p.spin_limit, p.err, gen, kWaitRoutes))) break;
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int jq = 0; jq < kPer; ++jq) {
          const int pr = tid + jq * kRgThreads;
          if (!tag_is(wq[jq], gen)) wq[jq] = ld_tag(&p.tids[pr < P ? pr : 0]);
        }
      }
#pragma unroll
      for (int jq = 0; jq < kPer; ++jq) {
        const int pr = tid + jq * kRgThreads;
        const int e = static_cast<int>(static_cast<uint32_t>(wq[jq]));
        ev[jq] = (pr < P && e >= 0 && e < EG) ? e : -1;
      }
    }
    __syncthreads();
#pragma unroll
    for (int jq = 0; jq < kPer; ++jq)
      if (ev[jq] >= 0) atomicAdd(&s_cnt[ev[jq]], 1);
    __syncthreads();
    // exclusive offsets of the counts and of the unit counts: thread i holds
    // experts 2i and 2i + 1; scans within each wave by lane shuffles, then across
    // the waves' totals
    const int ut = p.unit_tokens;
    const int e0 = 2 * tid, e1 = 2 * tid + 1;
    const int c0 = s_cnt[e0], c1 = s_cnt[e1];
    const int n0 = (c0 + ut - 1) / ut, n1 = (c1 + ut - 1) / ut;
    int a = c0 + c1, bu = n0 + n1;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int ta = __shfl_up(a, off, kWave), tb = __shfl_up(bu, off, kWave);
      if (lane >= off) {
        a += ta;
        bu += tb;
      }
    }
    if (lane == kWave - 1) {
      s_wa[wave] = a;
      s_wb[wave] = bu;
    }
    __syncthreads();
    for (int w = 0; w < wave; ++w) {
      a += s_wa[w];
      bu += s_wb[w];
    }
    const int off0 = a - (c0 + c1), ub0 = bu - (n0 + n1);
    const int offs[2] = {off0, off0 + c0}, ubs[2] = {ub0, ub0 + n0}, cs[2] = {c0, c1},
              ns[2] = {n0, n1};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = e0 + h;
      s_cur[e] = offs[h];
      if (e < EG) {
        for (int c = 0; c < ns[h]; ++c) {
          PfUnit un;
          un.bank = 0;
          un.expert = e;
          un.start = offs[h] + c * ut;
          un.count = min(ut, cs[h] - c * ut);
          p.units[ubs[h] + c] = un;
        }
      }
    }
    if (tid == kRgThreads - 1) {  // holds the inclusive totals
      int n = bu;
      if (p.shared_units) {
        for (int t0 = 0; t0 < T; t0 += ut) {
          PfUnit un;
          un.bank = 1;
          un.expert = 0;
          un.start = t0;
          un.count = min(ut, T - t0);
          p.units[n++] = un;
        }
      }
      *p.nunits = n;
    }
    __syncthreads();
#pragma unroll
    for (int jq = 0; jq < kPer; ++jq)
      if (ev[jq] >= 0) p.sorted[atomicAdd(&s_cur[ev[jq]], 1)] = tid + jq * kRgThreads;
  }

  if (tid == 0) st_dev(&p.gen[b], gen);
}

template <int NTT>
static hipError_t launch_rg(const RouteGroupParams& p, int grid, hipStream_t s) {
  route_group_kernel<NTT><<<dim3(grid), dim3(kRgThreads), 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_route_group(const RouteGroupParams& p, int grid, hipStream_t s) {
  switch ((p.T + 15) / 16) {
    case 1: return launch_rg<1>(p, grid, s);
    case 2: return launch_rg<2>(p, grid, s);
    case 3: return launch_rg<3>(p, grid, s);
    default: return launch_rg<4>(p, grid, s);
  }
}

hipError_t route_group_min_occupancy(int* blocks_per_cu) {
  using K = void (*)(RouteGroupParams);
  static const K kernels[] = {route_group_kernel<1>, route_group_kernel<2>,
                              route_group_kernel<3>, route_group_kernel<4>};
  int lowest = 1 << 30;
  for (K kf : kernels) {
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &n, reinterpret_cast<const void*>(kf), kRgThreads, 0);
    if (e != hipSuccess) return e;
    lowest = n < lowest ? n : lowest;
  }
  *blocks_per_cu = lowest;
  return hipSuccess;
}

}  // namespace ftmoe
