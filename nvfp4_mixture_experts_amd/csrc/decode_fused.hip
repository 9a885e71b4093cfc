// decode_fused.hip -- the whole NVFP4 MoE layer at decode time in ONE persistent
// kernel launch on gfx950.
//
// FreeToken fork PR #84 (page 1), bullet on #631: the NVFP4 MoE decode GEMV sits
// on the per-token path of each MoE layer.  FreeToken commit log (page 2): the
// router / shared-gate kernel entry, the top-k entry (k need not be a power of
// two), the clamped-SwiGLU entry, the 512-expert top-10 entry with its gated
// shared expert, and the decode configuration for long reduction rows.
//
// At batch 1 the layer moves ~24 MB: about 3 us of HBM time, the same order as
// one kernel launch or one grid-wide barrier.  So the layer is one launch of one
// block per CU, and no phase waits on a barrier: every value one block hands to
// another is TAGGED with the call's generation number (value in the low half of
// an 8-byte word, generation in the high half, written and read with single
// device-coherent 8-byte accesses), and a consumer polls exactly the values it
// needs until their tags match.  Each block counts its own calls, so all blocks
// agree on the generation without talking to each other, and nothing needs
// resetting between calls.
//
//   R  router rows (one row per wave, rows spread one per CU; fp64 dot products
//      with a DPP tree sum) and the shared gate; each logit is published in
//      kLogitCopies replicas so that 256 blocks do not read the same lines.
//   S  every block selects the experts itself from its replica by counting,
//      for each expert, the keys above its own: first inside its 64-expert
//      chunk, then among the chunks' candidates (no serial select rounds; ties
//      go to the lower index).
//   W  every wave issues its gate|up loads, takes the routing weights (in its
//      own registers), then computes: e2m1 -> bf16 in registers,
//      v_dot2_f32_bf16 against bf16 x, per-16 e4m3 block scales, global
//      scales, (clamped) SwiGLU; h published tagged.  Only then does it issue
//      the loads of its first down-projection chunks (kept in registers for D):
//      the gate|up stream, which every h waits for, has HBM to itself, and the
//      down loads travel while h crosses between blocks.
//   D  down GEMV from the prefetched chunks (lane = output row, K-chunk-major
//      codes; the h chunks of a wave's units polled together, one round trip,
//      and broadcast from LDS), weighted by routing weight or
//      shared gate; the blocks of one row group publish tagged partials and one
//      of them sums them in a fixed order into bf16 y.
//
// Every poll is bounded: if a value never arrives (a grid that is not
// co-resident), the kernel stops waiting, records why in the error word and
// finishes; the caller reads the word with ft_moe_device_status.
#include "ftmoe_device.hpp"
#include "ftmoe_kernels.hpp"
#include "handoff.hpp"

namespace {
// Non-temporal 16-byte load (no cache allocation) for the NVFP4 gate|up codes, each read
// once per call: ~1% per call at both batch-1 shapes; for the down codes, and for the
// block-fp8 codes (15.9 -> 17.0 us), it was slower.
__device__ __forceinline__ uint4 ldnt16(const void* a) {
  typedef unsigned int nt_u4 __attribute__((ext_vector_type(4)));
  const nt_u4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u4*>(a));
  return make_uint4(v.x, v.y, v.z, v.w);
}
}  // namespace

namespace ftmoe {

constexpr int kFWaves = 8;     // waves per block
constexpr int kUW = 3;         // gate|up units per wave and batch
constexpr int kUD = 3;         // down units per wave and batch (first batch prefetched)
constexpr int kMaxTK = 64 * 16;
constexpr int kMaxK = kTopkMaxK;
constexpr int kRouterWaitSpins = 1 << 16;  // LDS polls of the router-done flag, at most

// The 32 tagged h values of each of the N units of a down batch, polled together
// so that the batch costs one round trip, not one per unit.  Word w of the batch
// (unit w / 32, value w % 32) is read by lane w % 64 and its value stored to
// hs[w] (this wave's LDS slice); units with need[u] false are not waited for
// (their addresses are still in range).
template <int N>
__device__ __forceinline__ void poll_h_batch(const uint64_t* const (&hrow)[N],
                                             const bool (&need)[N], uint32_t gen, float* hs,
                                             int spin_limit, uint32_t* err) {
  constexpr int kL = (32 * N + kWave - 1) / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const bool upper = lane >= 32;
  const uint64_t* addr[kL];
  bool want[kL];
  uint64_t wd[kL];
#pragma unroll
  for (int m = 0; m < kL; ++m) {
    const int u0 = 2 * m;
    const int u1 = (2 * m + 1 < N) ? 2 * m + 1 : u0;  // the upper half's unit
    const bool has1 = 2 * m + 1 < N;
    addr[m] = (upper ? hrow[u1] : hrow[u0]) + (lane & 31);
    want[m] = upper ? (has1 && need[u1]) : need[u0];
    wd[m] = ld_tag(addr[m]);
  }
  for (int spins = 0;; ++spins) {
    bool ok = true;
#pragma unroll
    for (int m = 0; m < kL; ++m) ok = ok && (!want[m] || tag_is(wd[m], gen));
    if (__ballot(!ok) == 0) break;
    if (stop_waiting(spins, spin_limit, err, gen, kWaitH)) break;
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int m = 0; m < kL; ++m)
      if (want[m] && !tag_is(wd[m], gen)) wd[m] = ld_tag(addr[m]);
  }
#pragma unroll
  for (int m = 0; m < kL; ++m) {
    const int w = m * kWave + lane;
    if (w < 32 * N) hs[w] = tag_value(wd[m]);
  }
}

// ------------------------------------------------------------- top-k --

// The shared expert's gate of one token (word E of its logits row), by one lane.
__device__ __forceinline__ float poll_gate(const uint64_t* lg, int E, uint32_t gen,
                                           int spin_limit, uint32_t* err) {
  uint64_t wd = ld_tag(lg + E);
  for (int spins = 0; !tag_is(wd, gen); ++spins) {
    if (stop_waiting(spins, spin_limit, err, gen, kWaitGate)) break;
    __builtin_amdgcn_s_sleep(1);
    wd = ld_tag(lg + E);
  }
  return tag_value(wd);
}

// The experts of one token's logits row (tagged, E + 1 words; word E is the
// shared gate) by all waves of the block: block_topk_rank with each chunk's
// logits polled until they carry this call's generation.  ids[place] and
// s_v[place] are complete for every wave on return.
__device__ __forceinline__ void block_topk_one_token(const uint64_t* lg, int E, int k,
                                                     uint32_t gen, int spin_limit, uint32_t* err,
                                                     uint64_t (*s_key)[kWave], uint64_t* s_cand,
                                                     double* s_v, int* ids) {
  block_topk_rank<kFWaves>(
      E, k,
      [&](int e) { return tag_value(poll_tag(lg + e, gen, spin_limit, err)); },
      s_key, s_cand, s_v, ids);
}

// One token's experts by one wave (used when the block handles several tokens).
template <int SLOTS>
__device__ void wave_topk_tagged(const uint64_t* lg, int E, int k, uint32_t gen, int spin_limit,
                                 uint32_t* err, int* ids, float* w, float* gamma,
                                 bool has_shared) {
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t wd[SLOTS];
#pragma unroll
  for (int m = 0; m < SLOTS; ++m) {
    const int e = lane + kWave * m;
    wd[m] = ld_tag(lg + (e < E ? e : E - 1));
  }
  for (int spins = 0;; ++spins) {
    bool ok = true;
#pragma unroll
    for (int m = 0; m < SLOTS; ++m) ok = ok && tag_is(wd[m], gen);
    if (__ballot(!ok) == 0) break;
    if (stop_waiting(spins, spin_limit, err, gen, kWaitLogits)) break;
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int m = 0; m < SLOTS; ++m) {
      const int e = lane + kWave * m;
      if (!tag_is(wd[m], gen)) wd[m] = ld_tag(lg + (e < E ? e : E - 1));
    }
  }
  float lv[SLOTS];
#pragma unroll
  for (int m = 0; m < SLOTS; ++m) lv[m] = tag_value(wd[m]);
  int id;
  float wt;
  wave_topk_vals<SLOTS>(E, k, lv, &id, &wt);
  if (lane < k) {
    ids[lane] = id;
    w[lane] = wt;
  }
  if (lane == 0) *gamma = has_shared ? poll_gate(lg, E, gen, spin_limit, err) : 0.0f;
}

// --------------------------------------------------------------- units --

struct Unit13 {  // one (token, slot, pair) of the gate|up GEMV, for one lane group
  int t, slot, r;
  bool valid;
};

// Pair u of the flattened (token, slot, row) space: per token, the k routed
// experts' I rows, then the shared expert's Is rows.
__device__ __forceinline__ Unit13 unit13(int u, int total, int k, int kI, FastDiv ppt,
                                         FastDiv inter) {
  Unit13 o;
  o.valid = u < total;
  if (!o.valid) u = 0;
  o.t = fdiv(u, ppt);
  const int rem = u - o.t * ppt.d;
  if (rem < kI) {
    o.slot = fdiv(rem, inter);
    o.r = rem - o.slot * inter.d;
  } else {
    o.slot = k;
    o.r = rem - kI;
  }
  return o;
}

struct Unit2 {  // one (slot, K-chunk) of the down GEMV of one row group
  int slot, chunk;
};

__device__ __forceinline__ Unit2 unit2(int v, int k, FastDiv nch) {
  Unit2 o;
  if (v < k * nch.d) {
    o.slot = fdiv(v, nch);
    o.chunk = v - o.slot * nch.d;
  } else {
    o.slot = k;
    o.chunk = v - k * nch.d;
  }
  return o;
}

// ---------------------------------------------------------------- kernel --

// ONE: the call has one token (T == 1).  That instantiation has no activation
// loads inside the gate|up compute loop: vmcnt counts stores too and completes in
// order, so a load there would make the next unit's wait cover the device-coherent
// h stores issued before it, and every unit would wait for their acknowledgement.
//
// SLOTS: the routed experts live in a bank of expert slots (p.slot_of maps expert
// -> slot; a slot outside [0, p.n_slots) means the expert is not resident).  The
// map is read into LDS together with the router loads, so looking a selected
// expert up costs no memory round trip.  A non-resident expert's units read slot
// 0's weights (every access stays unconditional and in range), produce h = 0 and
// enter the down GEMV with weight 0; its id goes to p.miss_out.
//
// FP8: the experts use the block-fp8 codec (e4m3 bytes, one fp32 scale per 128 x 128
// block, no global scale): a 32-element chunk is 32 code bytes (two 16-byte loads per
// lane), gate|up rows stay row-major, down records are 32 bytes (K-chunk-major).
template <int LPR, int CPL, bool ONE, bool SLOTS, bool FP8>
__global__ __launch_bounds__(kFWaves* kWave, 1) void moe_decode_fused_kernel(FusedParams p) {
  constexpr int GPW = kWave / LPR;   // lane groups per wave
  constexpr int NC = LPR * CPL / 8;  // float4 pieces of a router row per lane (H / 256)
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = gridDim.x;
  const int gw = blockIdx.x * kFWaves + wave;
  const int NW = G * kFWaves;
  const int H = p.H, E = p.E, T = ONE ? 1 : p.T, k = p.k;
  const int nrg = H / kWave;
  const int E1 = E + 1;

  __shared__ int s_ids[kMaxTK];
  __shared__ float s_w[kMaxTK];
  __shared__ float s_gamma[64];
  __shared__ float s_red[kFWaves][kWave];
  __shared__ __align__(16) uint64_t s_key[kFWaves][kWave];
  __shared__ __align__(16) uint64_t s_cand[kTopkMaxChunks * kTopkMaxK];
  __shared__ double s_v[kMaxK];
  __shared__ __align__(16) float s_hb[kFWaves][32 * kUD];  // h values of a down batch
  __shared__ uint32_t s_gen[kFWaves];
  __shared__ uint32_t s_rdone;  // this call's generation once wave 0's router rows are out
  __shared__ int s_map[SLOTS ? kMaxExperts : 1];  // expert -> slot (SLOTS)

  // SLOTS: the expert -> slot map, two entries per thread (E <= 1024), loaded now
  // and stored to LDS before the selection's barriers
  int map0 = 0, map1 = 0;
  if constexpr (SLOTS) {
    const int i0 = static_cast<int>(threadIdx.x), i1 = i0 + kFWaves * kWave;
    map0 = p.slot_of[i0 < E ? i0 : E - 1];
    map1 = p.slot_of[i1 < E ? i1 : E - 1];
  }
  // slot of expert e, or -1 when it is not resident
  auto slot_of = [&](int e) -> int {
    if constexpr (!SLOTS) {
      return e;
    } else {
      const int sl = s_map[e];
      return (sl >= 0 && sl < p.n_slots) ? sl : -1;
    }
  };

  // Generation of this call: this block's own call count.  Every wave reads the
  // counter itself and nothing waits for it here, so the read travels together
  // with the router loads instead of costing a round trip (and a barrier) before
  // them.  The new count is stored after the selection's barrier; each wave puts
  // its copy into LDS before that barrier, so every read has returned by then.
  const uint32_t gen = ld_dev(&p.gen[blockIdx.x]) + 1u;

  // ---------------------------------------------------------------- R --
  {
    // the bf16 shared-gate vector as fp32, the same pieces as a router row
    auto gate_vector = [&](float4 (&wv)[NC]) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint2 g2 = *reinterpret_cast<const uint2*>(p.shared_gate + 4 * lane + 4 * kWave * c);
        wv[c] = make_float4(bf16_bits_to_f32(g2.x & 0xFFFFu), bf16_bits_to_f32(g2.x >> 16),
                            bf16_bits_to_f32(g2.y & 0xFFFFu), bf16_bits_to_f32(g2.y >> 16));
      }
    };
    // fp64 dot product of a row with token t's activations (the whole wave's sum)
    auto dot_x = [&](const float4 (&wv)[NC], int t) -> double {
      const uint16_t* __restrict__ xt = p.x + static_cast<size_t>(t) * H;
      uint2 xv[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c)
        xv[c] = *reinterpret_cast<const uint2*>(xt + 4 * lane + 4 * kWave * c);
      double acc = 0.0;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint2 xb = xv[c];
        acc = fma(static_cast<double>(wv[c].x), static_cast<double>(bf16_bits_to_f32(xb.x & 0xFFFFu)), acc);
        acc = fma(static_cast<double>(wv[c].y), static_cast<double>(bf16_bits_to_f32(xb.x >> 16)), acc);
        acc = fma(static_cast<double>(wv[c].z), static_cast<double>(bf16_bits_to_f32(xb.y & 0xFFFFu)), acc);
        acc = fma(static_cast<double>(wv[c].w), static_cast<double>(bf16_bits_to_f32(xb.y >> 16)), acc);
      }
      return wave_sum_f64(acc);
    };
    // Row r goes to block r % G, wave r / G: consecutive rows on different CUs.
    // With several tokens the shared gate is row E; with one token every block
    // takes the gate itself (its last wave, below), so that it needs no hand-off
    // and no block's selection waits behind the gate row's first access.
    const int rows = E + ((!ONE && p.shared_gate) ? 1 : 0);
    for (int row = wave * G + blockIdx.x; row < rows; row += kFWaves * G) {
      const bool gate_row = (row == E);
      float4 wv[NC];
      if (!gate_row) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
          wv[c] = *reinterpret_cast<const float4*>(p.wr + static_cast<size_t>(row) * H +
                                                   4 * lane + 4 * kWave * c);
      } else {
        gate_vector(wv);
      }
      const double bias = (!gate_row && p.bias) ? static_cast<double>(ld_vmem_f32(p.bias, row)) : 0.0;
      for (int t = 0; t < T; ++t) {
        double acc = dot_x(wv, t);
        float v;
        if (!gate_row) {
          if (p.bias) acc += bias;
          v = static_cast<float>(acc);
        } else {
          v = static_cast<float>(1.0 / (1.0 + exp(-acc)));
        }
        if (lane < kLogitCopies)
          st_tag(&p.logits[(static_cast<size_t>(lane) * T + t) * E1 + row], v, gen);
      }
    }
    if (ONE && p.shared_gate && wave == kFWaves - 1) {
      float4 wv[NC];
      gate_vector(wv);
      const double acc = dot_x(wv, 0);
      if (lane == 0) s_gamma[0] = static_cast<float>(1.0 / (1.0 + exp(-acc)));
    }
  }

  if (wave == 0 && lane == 0)
    __hip_atomic_store(&s_rdone, gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);

  // ---------------------------------------------------------------- S --
  if (lane == 0) s_gen[wave] = gen;  // needs the counter read to have returned
  if constexpr (SLOTS) {
    const int i0 = static_cast<int>(threadIdx.x), i1 = i0 + kFWaves * kWave;
    if (i0 < E) s_map[i0] = map0;
    if (i1 < E) s_map[i1] = map1;
  }
  {
    const uint64_t* lgc = p.logits + static_cast<size_t>(blockIdx.x % kLogitCopies) * T * E1;
    const bool has_shared = p.shared_gate != nullptr;
    // A wave with no router row waits for its block's wave 0 to have issued its
    // router row's stores before its first poll of the logits (every block's
    // router rows finish within a few hundred ns of each other; a short sleep
    // covers their propagation).  Polling from the start instead sends thousands
    // of device-coherent reads at a few replica lines while the router loads and
    // stores are in flight, and slowed the whole call by about 1 us.  The flag
    // holds the call's generation, so a value left in LDS by an earlier launch
    // never matches; the wait is bounded.
    const int rrows = E + (p.shared_gate ? 1 : 0);
    if (wave * G + static_cast<int>(blockIdx.x) >= rrows &&
        static_cast<int>(blockIdx.x) < rrows) {
      for (int sp = 0; sp < kRouterWaitSpins; ++sp) {
        if (__hip_atomic_load(&s_rdone, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == gen)
          break;
        __builtin_amdgcn_s_sleep(2);
      }
      __builtin_amdgcn_s_sleep(8);
    }
    if (T == 1) {
      block_topk_one_token(lgc, E, k, gen, p.spin_limit, p.err, s_key, s_cand, s_v, s_ids);
    } else {
      for (int t = wave; t < T; t += kFWaves) {
        const uint64_t* lg = lgc + static_cast<size_t>(t) * E1;
        if (E <= 4 * kWave)
          wave_topk_tagged<4>(lg, E, k, gen, p.spin_limit, p.err, &s_ids[t * k], &s_w[t * k],
                              &s_gamma[t], has_shared);
        else if (E <= 8 * kWave)
          wave_topk_tagged<8>(lg, E, k, gen, p.spin_limit, p.err, &s_ids[t * k], &s_w[t * k],
                              &s_gamma[t], has_shared);
        else
          wave_topk_tagged<16>(lg, E, k, gen, p.spin_limit, p.err, &s_ids[t * k], &s_w[t * k],
                               &s_gamma[t], has_shared);
      }
      __syncthreads();
      if (blockIdx.x == 0) {
        for (int i = threadIdx.x; i < T * k; i += blockDim.x) {
          if (p.ids_out) p.ids_out[i] = s_ids[i];
          if (p.w_out) p.w_out[i] = s_w[i];
        }
      }
    }
  }
  // past the selection's barrier: every wave of the block holds this call's count
  // (all copies are equal; reading them all keeps each wave's LDS store live)
  if (threadIdx.x == 0) {
    uint32_t g = s_gen[0];
#pragma unroll
    for (int w = 1; w < kFWaves; ++w) g = s_gen[w] > g ? s_gen[w] : g;
    st_dev(&p.gen[blockIdx.x], g);
  }

  // One token: the routing weights (lane i: place i), taken by every wave in its
  // own registers once its first expert loads are out (the exponentials then
  // overlap those loads), and the shared gate, which the block's last wave left
  // in LDS before the selection's barriers.
  float w1 = 0.0f, gamma1 = 0.0f;
  bool have_w1 = T != 1;
  auto weights_one_token = [&]() {
    if (have_w1) return;
    have_w1 = true;
    w1 = softmax_of_places(s_v, k);
  };
  auto gate_one_token = [&]() {
    if (T != 1 || !p.shared_gate) return;
    gamma1 = s_gamma[0];
  };
  // routing weight (or shared gate) of slot `slot` (k: the shared expert) of token t
  auto slot_weight = [&](int t, int slot) -> float {
    if (T == 1)
      return slot == k ? gamma1
                       : __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w1), slot));
    return slot == k ? s_gamma[t] : s_w[t * k + slot];
  };

  // ------------------------------------------------ D assignment (prefetch) --
  const int nch = p.routed.inter / 32;
  const int nch_s = p.shared.inter / 32;
  const FastDiv fd_nch = make_fastdiv(nch);
  const FastDiv fd_nrg = make_fastdiv(nrg);
  const int upg = k * nch + nch_s;  // down units per (token, row group)
  int bpg, g_first, g_step, sub;
  if (p.d_groups >= G) {
    bpg = 1;
    g_first = blockIdx.x;
    g_step = G;
    sub = 0;
  } else {
    bpg = p.blocks_per_group;
    g_first = blockIdx.x / bpg;
    g_step = p.d_groups;  // one group per block
    sub = blockIdx.x - g_first * bpg;
  }

  // Everything a down unit needs except h: code/scale addresses, its weight
  // (routing weight x down global scale) and where its h chunk lives.  All
  // wave-uniform except the row; computed and loaded at issue time.
  struct DownUnit {
    const uint8_t* cp;
    const uint8_t* sp;
    const float* spf;      // FP8: the unit's block scale
    const uint64_t* hrow;  // 32 tagged h values of this unit
    int slot;              // the unit's slot (k: the shared expert)
    float gdown;           // down global scale of the unit's expert (multiplied at use:
                           // using a load result at issue time would wait for every
                           // load issued before it)
    bool present;          // the unit's expert is resident (always, without SLOTS)
    bool valid;
  };
  auto down_unit = [&](int t, int v, int c) {
    DownUnit d;
    d.valid = v < upg;
    const int vv = d.valid ? v : upg - 1;  // clamped: addresses stay in range
    const Unit2 u = unit2(vv, k, fd_nch);
    const bool sh = (u.slot == k);
    const int sl = sh ? 0 : slot_of(s_ids[t * k + u.slot]);
    const int e = __builtin_amdgcn_readfirstlane(SLOTS && sl < 0 ? 0 : sl);
    const int nu = sh ? nch_s : nch;
    const size_t rec = (static_cast<size_t>(e) * nu + u.chunk) * H + c;
    d.hrow = p.h + (static_cast<size_t>(t) * p.nslots + u.slot) * p.Imax + 32 * u.chunk;
    d.slot = u.slot;
    if constexpr (FP8) {
      const int kb = nu / 4;  // 128-element scale blocks along K
      d.cp = (sh ? p.shared.w2 : p.routed.w2) + rec * 32;
      d.sp = nullptr;
      d.spf = reinterpret_cast<const float*>(sh ? p.shared.w2s : p.routed.w2s) +
              (static_cast<size_t>(e) * (H / 128) + c / 128) * kb + u.chunk / 4;
      d.gdown = 1.0f;
    } else {
      d.cp = (sh ? p.shared.w2 : p.routed.w2) + rec * 16;
      d.sp = (sh ? p.shared.w2s : p.routed.w2s) + rec * 2;
      d.spf = nullptr;
      d.gdown = ld_vmem_f32(sh ? p.shared.gsc : p.routed.gsc, 3 * e + 2);
    }
    d.present = sl >= 0;  // multiplied in at use (a missing expert's term is 0)
    return d;
  };

  uint4 pq[kUD], pq2[FP8 ? kUD : 1];
  uint32_t ps[kUD];
  float psf[FP8 ? kUD : 1];
  DownUnit pdu[kUD];
  const bool have_first = g_first < p.d_groups;
  // issues the loads of this wave's first down units (kept in registers until D).
  // A block with no down group loads group 0's (never used): the loads are not
  // conditional, so the in-order wait counts after them stay exact.
  auto prefetch_down = [&]() {
    const int g0 = have_first ? g_first : 0;
    const int t = fdiv(g0, fd_nrg);
    const int c = (g0 - t * nrg) * kWave + lane;
#pragma unroll
    for (int i = 0; i < kUD; ++i) {
      pdu[i] = down_unit(t, sub + bpg * (wave + kFWaves * i), c);
      pq[i] = *reinterpret_cast<const uint4*>(pdu[i].cp);
      if constexpr (FP8) {
        pq2[i] = *reinterpret_cast<const uint4*>(pdu[i].cp + 16);
        psf[i] = *pdu[i].spf;
        ps[i] = 0;
      } else {
        ps[i] = *reinterpret_cast<const uint16_t*>(pdu[i].sp);
      }
    }
  };

  // ---------------------------------------------------------------- W --
  {
    const int group = lane / LPR, col = lane % LPR;
    const int NG = NW * GPW;
    const int kI = k * p.routed.inter;
    const FastDiv fd_ppt = make_fastdiv(kI + p.shared.inter);
    const FastDiv fd_inter = make_fastdiv(p.routed.inter);
    const int total = T * fd_ppt.d;
    const size_t row_bytes = static_cast<size_t>(H) / 2;
    const size_t srow_bytes = static_cast<size_t>(H) / 16;
    bf16x2 xr[CPL][16];
    auto load_x = [&](int t) {
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
    };
    if (ONE) load_x(0);
    bool prefetched = false;
    for (int j0 = 0; (gw * GPW) + NG * j0 < total; j0 += kUW) {
      Unit13 un[kUW];
      bool present[kUW];
      float g_gate[kUW], g_up[kUW];
      uint4 qg[kUW][CPL], qu[kUW][CPL];
      uint32_t sg[kUW][CPL], su[kUW][CPL];
      uint4 qg2[FP8 ? kUW : 1][CPL], qu2[FP8 ? kUW : 1][CPL];  // FP8: second 16 bytes
      float fsg[FP8 ? kUW : 1][CPL], fsu[FP8 ? kUW : 1][CPL];    // FP8: block scales
#pragma unroll
      for (int jj = 0; jj < kUW; ++jj) {
        un[jj] = unit13(gw * GPW + group + NG * (j0 + jj), total, k, kI, fd_ppt, fd_inter);
        const bool sh = (un[jj].slot == k);
        const int I = sh ? p.shared.inter : p.routed.inter;
        int e = sh ? 0 : slot_of(s_ids[un[jj].t * k + un[jj].slot]);
        present[jj] = true;
        if constexpr (SLOTS) {
          present[jj] = e >= 0;
          e = e < 0 ? 0 : e;
        }
        if (LPR == kWave) e = __builtin_amdgcn_readfirstlane(e);  // one unit per wave
        const size_t rr = static_cast<size_t>(un[jj].r);
        if constexpr (FP8) {
          const uint8_t* __restrict__ codes =
              (sh ? p.shared.w13 : p.routed.w13) + static_cast<size_t>(e) * 2 * I * H;
          const int kb = H / 128;
          const float* __restrict__ sc = reinterpret_cast<const float*>(
                                             sh ? p.shared.w13s : p.routed.w13s) +
                                         static_cast<size_t>(e) * (2 * I / 128) * kb;
          g_gate[jj] = 1.0f;
          g_up[jj] = 1.0f;
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            const int j = col + LPR * c;
            const uint8_t* gr = codes + rr * H + 32 * j;
            const uint8_t* ur = codes + (I + rr) * H + 32 * j;
            qg[jj][c] = *reinterpret_cast<const uint4*>(gr);
            qg2[jj][c] = *reinterpret_cast<const uint4*>(gr + 16);
            qu[jj][c] = *reinterpret_cast<const uint4*>(ur);
            qu2[jj][c] = *reinterpret_cast<const uint4*>(ur + 16);
            fsg[jj][c] = sc[(rr / 128) * kb + j / 4];
            fsu[jj][c] = sc[((I + rr) / 128) * kb + j / 4];
            sg[jj][c] = su[jj][c] = 0;
          }
          continue;
        }
        const uint8_t* __restrict__ codes =
            (sh ? p.shared.w13 : p.routed.w13) + static_cast<size_t>(e) * 2 * I * row_bytes;
        const uint8_t* __restrict__ scales =
            (sh ? p.shared.w13s : p.routed.w13s) + static_cast<size_t>(e) * 2 * I * srow_bytes;
        const float* gsc = sh ? p.shared.gsc : p.routed.gsc;
        g_gate[jj] = ld_vmem_f32(gsc, 3 * e + 0);
        g_up[jj] = ld_vmem_f32(gsc, 3 * e + 1);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int j = col + LPR * c;
          qg[jj][c] = ldnt16(codes + rr * row_bytes + 16 * j);
          qu[jj][c] = ldnt16(codes + (I + rr) * row_bytes + 16 * j);
          if constexpr (LPR == kWave && CPL == 1) {
            // one dword load for both rows' scales: lanes 0..31 read the gate row's
            // 128 bytes, lanes 32..63 the up row's; redistributed at compute time
            const size_t srow = (lane < 32 ? rr : I + rr) * srow_bytes + 4 * (lane & 31);
            sg[jj][c] = *reinterpret_cast<const uint32_t*>(scales + srow);
            su[jj][c] = 0;
          } else {
            sg[jj][c] = *reinterpret_cast<const uint16_t*>(scales + rr * srow_bytes + 2 * j);
            su[jj][c] = *reinterpret_cast<const uint16_t*>(scales + (I + rr) * srow_bytes + 2 * j);
          }
        }
      }
      if (!prefetched) {  // behind the first gate|up loads, ahead of their use
        prefetched = true;
        weights_one_token();
      }
      float hv[kUW];
#pragma unroll
      for (int jj = 0; jj < kUW; ++jj) {
        if (!ONE) load_x(un[jj].t);
        float ag = 0.0f, au = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          if constexpr (FP8) {
            ag += chunk_dot_fp8_bf16(qg[jj][c], qg2[jj][c], xr[c]) * fsg[jj][c];
            au += chunk_dot_fp8_bf16(qu[jj][c], qu2[jj][c], xr[c]) * fsu[jj][c];
            continue;
          }
          if constexpr (LPR == kWave && CPL == 1) {
            const uint32_t d = sg[jj][c];
            const uint32_t gd = static_cast<uint32_t>(
                __builtin_amdgcn_ds_bpermute((lane >> 1) << 2, static_cast<int>(d)));
            const uint32_t ud = static_cast<uint32_t>(
                __builtin_amdgcn_ds_bpermute((32 + (lane >> 1)) << 2, static_cast<int>(d)));
            sg[jj][c] = (gd >> (16 * (lane & 1))) & 0xFFFFu;
            su[jj][c] = (ud >> (16 * (lane & 1))) & 0xFFFFu;
          }
          ag += chunk_dot_bf16(qg[jj][c], sg[jj][c], xr[c]);
          au += chunk_dot_bf16(qu[jj][c], su[jj][c], xr[c]);
        }
        ag = group_sum_last<LPR>(ag);
        au = group_sum_last<LPR>(au);
        hv[jj] = swiglu(p.act, ag * g_gate[jj], au * g_up[jj], p.gate_max, p.up_absmax);
        if constexpr (SLOTS) hv[jj] = present[jj] ? hv[jj] : 0.0f;
      }
      // the batch's h values, published after all of its units are computed: the
      // stores are conditional, and one issued between a unit's loads and their use
      // would make the compiler's in-order wait for that unit cover its
      // acknowledgement
#pragma unroll
      for (int jj = 0; jj < kUW; ++jj) {
        if (col == LPR - 1 && un[jj].valid)
          st_tag(&p.h[(static_cast<size_t>(un[jj].t) * p.nslots + un[jj].slot) * p.Imax +
                      un[jj].r],
                 hv[jj], gen);
      }
    }
    // the down chunks only now: the gate|up stream (which every h, and so every
    // down unit, waits for) has the memory system to itself, and the down loads
    // are in flight while the h values travel between blocks
    prefetch_down();
    weights_one_token();
  }

  // ---------------------------------------------------------------- D --
  gate_one_token();
  bool first = true;
  for (int g = g_first; g < p.d_groups; g += g_step) {
    const int t = fdiv(g, fd_nrg);
    const int rg = g - t * nrg;
    const int c = rg * kWave + lane;
    float acc = 0.0f;
    for (int i0 = 0; sub + bpg * (wave + kFWaves * i0) < upg; i0 += kUD) {
      uint4 q[kUD], q2[FP8 ? kUD : 1];
      uint32_t sc[kUD];
      float scf[FP8 ? kUD : 1];
      DownUnit du[kUD];
      if (first && i0 == 0) {
#pragma unroll
        for (int ii = 0; ii < kUD; ++ii) {
          q[ii] = pq[ii];
          sc[ii] = ps[ii];
          if constexpr (FP8) {
            q2[ii] = pq2[ii];
            scf[ii] = psf[ii];
          }
          du[ii] = pdu[ii];
        }
      } else {
#pragma unroll
        for (int ii = 0; ii < kUD; ++ii) {
          du[ii] = down_unit(t, sub + bpg * (wave + kFWaves * (i0 + ii)), c);
          q[ii] = *reinterpret_cast<const uint4*>(du[ii].cp);
          if constexpr (FP8) {
            q2[ii] = *reinterpret_cast<const uint4*>(du[ii].cp + 16);
            scf[ii] = *du[ii].spf;
            sc[ii] = 0;
          } else {
            sc[ii] = *reinterpret_cast<const uint16_t*>(du[ii].sp);
          }
        }
      }
      {
        const uint64_t* hrow[kUD];
        bool need[kUD];
#pragma unroll
        for (int ii = 0; ii < kUD; ++ii) {
          hrow[ii] = du[ii].hrow;
          need[ii] = du[ii].valid;
        }
        poll_h_batch<kUD>(hrow, need, gen, s_hb[wave], p.spin_limit, p.err);
      }
      wave_lds_sync();
#pragma unroll
      for (int ii = 0; ii < kUD; ++ii) {
        if (du[ii].valid) {
          float hv[32];
          const float4* h4 = reinterpret_cast<const float4*>(&s_hb[wave][32 * ii]);
#pragma unroll
          for (int m = 0; m < 8; ++m) {  // same address in every lane: LDS broadcast
            const float4 v = h4[m];
            hv[4 * m] = v.x;
            hv[4 * m + 1] = v.y;
            hv[4 * m + 2] = v.z;
            hv[4 * m + 3] = v.w;
          }
          const float wgt = slot_weight(t, du[ii].slot) * du[ii].gdown;
          float dot;
          if constexpr (FP8) {
            dot = chunk_dot_fp8_f32(q[ii], q2[ii], hv) * scf[ii];
          } else {
            dot = chunk_dot_f32(q[ii], sc[ii], hv);
          }
          acc = fmaf(dot, (!SLOTS || du[ii].present) ? wgt : 0.0f, acc);
        }
      }
      wave_lds_sync();  // the next batch rewrites s_hb[wave]
    }
    first = false;
    s_red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
      float o = s_red[0][lane];
#pragma unroll
      for (int w = 1; w < kFWaves; ++w) o += s_red[w][lane];
      uint16_t* yout = p.y + static_cast<size_t>(t) * H + c;
      if (bpg == 1) {
        *yout = f32_to_bf16_bits(o);
      } else {
        uint64_t* part = p.part + static_cast<size_t>(g) * bpg * kWave;
        st_tag(&part[sub * kWave + lane], o, gen);
        if (sub == 0) {
          // the group's combining block: every partial, in block order
          float ysum = o;
          for (int s0 = 1; s0 < bpg; s0 += 8) {
            uint64_t pv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) pv[i] = ld_tag(&part[min(s0 + i, bpg - 1) * kWave + lane]);
            for (int spins = 0;; ++spins) {
              bool ok = true;
#pragma unroll
              for (int i = 0; i < 8; ++i) ok = ok && tag_is(pv[i], gen);
              if (__ballot(!ok) == 0) break;
              if (stop_waiting(spins, p.spin_limit, p.err, gen, kWaitPartial)) break;
              __builtin_amdgcn_s_sleep(1);
#pragma unroll
              for (int i = 0; i < 8; ++i)
                if (!tag_is(pv[i], gen)) pv[i] = ld_tag(&part[min(s0 + i, bpg - 1) * kWave + lane]);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
              if (s0 + i < bpg) ysum += tag_value(pv[i]);
          }
          *yout = f32_to_bf16_bits(ysum);
        }
      }
    }
    __syncthreads();
  }
  // one token: the routing side outputs, last (stores issued earlier would enter
  // the in-order wait counts of the loads above)
  if (T == 1 && blockIdx.x == 0 && wave == 0 && lane < k) {
    if (p.ids_out) p.ids_out[lane] = s_ids[lane];
    if (p.w_out) p.w_out[lane] = w1;
  }
  if constexpr (SLOTS) {
    if (blockIdx.x == 0 && p.miss_out) {
      for (int i = threadIdx.x; i < T * k; i += blockDim.x)
        p.miss_out[i] = slot_of(s_ids[i]) < 0 ? s_ids[i] : -1;
    }
  }
}

template <int LPR, bool SLOTS, bool FP8>
static hipError_t launch_fused_lpr(const FusedParams& p, int grid, hipStream_t s) {
  const int cpl = p.H / (32 * LPR);
  dim3 g(grid), b(kFWaves * kWave);
  const bool one = p.T == 1;
  switch (cpl) {
#define FT_FUSED_CPL(C)                                                        \
  case C:                                                                      \
    if (one) moe_decode_fused_kernel<LPR, C, true, SLOTS, FP8><<<g, b, 0, s>>>(p); \
    else moe_decode_fused_kernel<LPR, C, false, SLOTS, FP8><<<g, b, 0, s>>>(p);    \
    break;
    FT_FUSED_CPL(1)
    FT_FUSED_CPL(2)
    FT_FUSED_CPL(3)
    FT_FUSED_CPL(4)
#undef FT_FUSED_CPL
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool SLOTS, bool FP8>
static hipError_t launch_fused(const FusedParams& p, int grid, hipStream_t s) {
  int lpr = 0, cpl = 0;
  gateup_geometry(p.H, &lpr, &cpl);
  switch (lpr) {
    case 64: return launch_fused_lpr<64, SLOTS, FP8>(p, grid, s);
    case 32: return launch_fused_lpr<32, SLOTS, FP8>(p, grid, s);
    case 16: return launch_fused_lpr<16, SLOTS, FP8>(p, grid, s);
    case 8: return launch_fused_lpr<8, SLOTS, FP8>(p, grid, s);
    default: return hipErrorInvalidValue;
  }
}

// slot indirection is for the NVFP4 banks; block-fp8 banks are read directly
hipError_t launch_decode_fused(const FusedParams& p, int grid, hipStream_t s) {
  if (p.fp8) return launch_fused<false, true>(p, grid, s);
  return p.slot_of ? launch_fused<true, false>(p, grid, s) : launch_fused<false, false>(p, grid, s);
}

int fused_block_threads() { return kFWaves * kWave; }

// The fewest blocks per CU that any instantiation of the fused kernel can keep
// resident (the kernel needs one on every CU at once).
hipError_t decode_fused_min_occupancy(int* blocks_per_cu) {
  using K = void (*)(FusedParams);
  static const K kernels[] = {
#define FT_FUSED_LPR(L, S, F)                                                                   \
  moe_decode_fused_kernel<L, 1, true, S, F>, moe_decode_fused_kernel<L, 1, false, S, F>,      \
      moe_decode_fused_kernel<L, 2, true, S, F>, moe_decode_fused_kernel<L, 2, false, S, F>,  \
      moe_decode_fused_kernel<L, 3, true, S, F>, moe_decode_fused_kernel<L, 3, false, S, F>,  \
      moe_decode_fused_kernel<L, 4, true, S, F>, moe_decode_fused_kernel<L, 4, false, S, F>
      FT_FUSED_LPR(64, false, false), FT_FUSED_LPR(32, false, false),
      FT_FUSED_LPR(16, false, false), FT_FUSED_LPR(8, false, false),
      FT_FUSED_LPR(64, true, false), FT_FUSED_LPR(32, true, false),
      FT_FUSED_LPR(16, true, false), FT_FUSED_LPR(8, true, false),
      FT_FUSED_LPR(64, false, true), FT_FUSED_LPR(32, false, true),
      FT_FUSED_LPR(16, false, true), FT_FUSED_LPR(8, false, true)
#undef FT_FUSED_LPR
  };
  int lowest = 1 << 30;
  for (K k : kernels) {
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &n, reinterpret_cast<const void*>(k), kFWaves * kWave, 0);
    if (e != hipSuccess) return e;
    lowest = n < lowest ? n : lowest;
  }
  *blocks_per_cu = lowest;
  return hipSuccess;
}

// Routes of a grouped decode call over a slot bank: expert ids become slot ids; a
// non-resident expert becomes slot 0 with weight 0 (its pair still runs, and
// contributes exactly 0), and its id goes to the miss list.
__global__ __launch_bounds__(256) void map_slots_kernel(int32_t* ids, float* w, int pairs,
                                                        const int32_t* slot_of, int n_slots,
                                                        int32_t* miss_out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= pairs) return;
  const int e = ids[i];
  const int sl = slot_of[e];
  const bool present = sl >= 0 && sl < n_slots;
  ids[i] = present ? sl : 0;
  if (!present) w[i] = 0.0f;
  if (miss_out) miss_out[i] = present ? -1 : e;
}

hipError_t launch_map_slots(int32_t* ids, float* w, int pairs, const int32_t* slot_of,
                            int n_slots, int32_t* miss_out, hipStream_t s) {
  if (pairs <= 0) return hipSuccess;
  map_slots_kernel<<<dim3((pairs + 255) / 256), dim3(256), 0, s>>>(ids, w, pairs, slot_of,
                                                                    n_slots, miss_out);
  return hipGetLastError();
}

// Reads the error word of a decode workspace into *status and clears it.
__global__ void device_status_kernel(uint32_t* err, int32_t* status) {
  if (threadIdx.x == 0) {
    const uint32_t v = __hip_atomic_exchange(err, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *status = static_cast<int32_t>(v);
  }
}

hipError_t launch_device_status(uint32_t* err, int32_t* status, hipStream_t s) {
  device_status_kernel<<<dim3(1), dim3(64), 0, s>>>(err, status);
  return hipGetLastError();
}


}  // namespace ftmoe
