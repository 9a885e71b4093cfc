// decode_fused.hip -- the whole NVFP4 MoE layer at decode time in ONE persistent
// kernel launch on gfx950.
//
// FreeToken fork PR #84 (page 1), bullet on #631: the NVFP4 MoE decode GEMV runs
// in every layer at every decode step.  FreeToken commit log (page 2): MoE router
// and shared-gate kernels, non-power-of-2 top-k, clamped SwiGLU, 512 routed
// experts with top-10 plus a gated shared expert, a "deep-K" decode config.
//
// At batch 1 the layer moves ~24 MB and the HBM floor is ~3 us, the same order
// as a kernel boundary, so the layer runs as one launch of one block per CU:
//
//   R  router rows (fp64 dot products, one per wave) and the shared gate;
//      logits published with device-coherent stores.          -> grid barrier 1
//   S  every block selects the top-k of every token itself (DPP wave reductions,
//      no second barrier) and keeps ids, weights and gates in LDS.
//   W  every wave issues the loads of its down-projection chunks (kept in
//      registers across the next barrier), then streams its gate|up rows:
//      e2m1 -> bf16 in registers, v_dot2_f32_bf16 against bf16 x, per-16 e4m3
//      block scales, global scales, (clamped) SwiGLU; h published.
//                                                              -> grid barrier 2
//   D  down GEMV from the prefetched chunks (lane = output row, K-chunk-major
//      codes, h read as wave-uniform device-coherent loads), weighted by the
//      routing weight / shared gate; blocks of one row group combine through
//      device-coherent partials and a last-arriver counter, in a fixed order.
//
// Grid barriers are device-scope counters polled with a bounded spin (a grid
// that is not co-resident cannot hang: the spin gives up and flags an error).
// Every counter is back at zero when the kernel ends.
#include "ftmoe_device.hpp"
#include "ftmoe_kernels.hpp"

namespace ftmoe {

constexpr int kFWaves = 8;     // waves per block
constexpr int kUW = 3;         // gate|up units per wave and batch
constexpr int kUD = 3;         // down units per wave and batch (first batch prefetched)
constexpr int kMaxTK = 64 * 16;

// 16 bytes at base + byte_off (wave-uniform base and offset), device-coherent.
__device__ __forceinline__ float4 ld_dev_x4_uniform(const float* base, uint32_t byte_off) {
  __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), static_cast<short>(0), 0x7fffffff,
                                        0x00020000);
  typedef int int4v __attribute__((ext_vector_type(4)));
  const int4v v = __builtin_amdgcn_raw_buffer_load_b128(r, 0, static_cast<int>(byte_off), 16);
  return __builtin_bit_cast(float4, v);
}

__device__ __forceinline__ void grid_barrier(uint32_t* counter, uint32_t target, uint32_t* err,
                                             int spin_limit) {
  wait_mem();
  __syncthreads();
  if (threadIdx.x == 0) {
    add_dev(counter, 1u);
    int spins = 0;
    while (ld_dev(counter) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > spin_limit) {
        st_dev(err, 1u);
        break;
      }
    }
  }
  __syncthreads();
}

struct Unit13 {  // one (token, slot, pair) of the gate|up GEMV, for one lane group
  int t, slot, r;
  bool valid;
};

__device__ __forceinline__ Unit13 unit13(const FusedParams& p, int u, int total) {
  Unit13 o;
  o.valid = u < total;
  if (!o.valid) u = 0;
  const int ppt = p.k * p.routed.inter + p.shared.inter;
  o.t = u / ppt;
  const int rem = u - o.t * ppt;
  const int kI = p.k * p.routed.inter;
  if (rem < kI) {
    o.slot = rem / p.routed.inter;
    o.r = rem - o.slot * p.routed.inter;
  } else {
    o.slot = p.k;
    o.r = rem - kI;
  }
  return o;
}

struct Unit2 {  // one (slot, K-chunk) of the down GEMV of one row group
  int slot, chunk;
};

__device__ __forceinline__ Unit2 unit2(const FusedParams& p, int v) {
  const int nch = p.routed.inter / 32;
  Unit2 o;
  if (v < p.k * nch) {
    o.slot = v / nch;
    o.chunk = v - o.slot * nch;
  } else {
    o.slot = p.k;
    o.chunk = v - p.k * nch;
  }
  return o;
}

template <int LPR, int CPL>
__global__ __launch_bounds__(kFWaves* kWave, 1) void moe_decode_fused_kernel(FusedParams p) {
  constexpr int GPW = kWave / LPR;      // lane groups per wave
  constexpr int NC = LPR * CPL / 8;     // float4 pieces of a router row per lane (H / 256)
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = gridDim.x;
  const int gw = blockIdx.x * kFWaves + wave;
  const int NW = G * kFWaves;
  const int H = p.H, E = p.E, T = p.T, k = p.k;
  const int nrg = H / kWave;

  __shared__ int s_ids[kMaxTK];
  __shared__ float s_w[kMaxTK];
  __shared__ float s_gamma[64];
  __shared__ float s_red[kFWaves][kWave];

  // ---------------------------------------------------------------- R --
  // clear the combine counters of this call (used only after barrier 2)
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < p.d_groups; i += G * blockDim.x)
    st_dev(&p.cnt[i], 0u);
  {
    const int rows = E + (p.shared_gate ? 1 : 0);
    for (int row = gw; row < rows; row += NW) {
      if (row < E) {
        const float* __restrict__ wrow = p.wr + static_cast<size_t>(row) * H;
        float4 wv[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c)
          wv[c] = *reinterpret_cast<const float4*>(wrow + 4 * lane + 4 * kWave * c);
        for (int t = 0; t < T; ++t) {
          const uint16_t* __restrict__ xt = p.x + static_cast<size_t>(t) * H;
          double acc = 0.0;
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const uint2 xb = *reinterpret_cast<const uint2*>(xt + 4 * lane + 4 * kWave * c);
            acc = fma(static_cast<double>(wv[c].x), static_cast<double>(bf16_bits_to_f32(xb.x & 0xFFFFu)), acc);
            acc = fma(static_cast<double>(wv[c].y), static_cast<double>(bf16_bits_to_f32(xb.x >> 16)), acc);
            acc = fma(static_cast<double>(wv[c].z), static_cast<double>(bf16_bits_to_f32(xb.y & 0xFFFFu)), acc);
            acc = fma(static_cast<double>(wv[c].w), static_cast<double>(bf16_bits_to_f32(xb.y >> 16)), acc);
          }
          acc = group_sum<kWave>(acc);
          if (lane == 0) {
            if (p.bias) acc += static_cast<double>(p.bias[row]);
            st_dev(&p.logits[static_cast<size_t>(t) * E + row], static_cast<float>(acc));
          }
        }
      } else {
        uint2 gv[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c)
          gv[c] = *reinterpret_cast<const uint2*>(p.shared_gate + 4 * lane + 4 * kWave * c);
        for (int t = 0; t < T; ++t) {
          const uint16_t* __restrict__ xt = p.x + static_cast<size_t>(t) * H;
          double acc = 0.0;
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const uint2 xb = *reinterpret_cast<const uint2*>(xt + 4 * lane + 4 * kWave * c);
            acc = fma(static_cast<double>(bf16_bits_to_f32(gv[c].x & 0xFFFFu)),
                      static_cast<double>(bf16_bits_to_f32(xb.x & 0xFFFFu)), acc);
            acc = fma(static_cast<double>(bf16_bits_to_f32(gv[c].x >> 16)),
                      static_cast<double>(bf16_bits_to_f32(xb.x >> 16)), acc);
            acc = fma(static_cast<double>(bf16_bits_to_f32(gv[c].y & 0xFFFFu)),
                      static_cast<double>(bf16_bits_to_f32(xb.y & 0xFFFFu)), acc);
            acc = fma(static_cast<double>(bf16_bits_to_f32(gv[c].y >> 16)),
                      static_cast<double>(bf16_bits_to_f32(xb.y >> 16)), acc);
          }
          acc = group_sum<kWave>(acc);
          if (lane == 0) st_dev(&p.gamma[t], static_cast<float>(1.0 / (1.0 + exp(-acc))));
        }
      }
    }
  }
  grid_barrier(&p.sync[0], static_cast<uint32_t>(G), &p.sync[3], p.spin_limit);

  // ---------------------------------------------------------------- S --
  for (int t = wave; t < T; t += kFWaves) {
    const float* lg = p.logits + static_cast<size_t>(t) * E;
    auto load = [&](int e) { return ld_dev(lg + e); };
    int id;
    float wt;
    if (E <= 4 * kWave)
      wave_topk<4>(E, k, load, &id, &wt);
    else if (E <= 8 * kWave)
      wave_topk<8>(E, k, load, &id, &wt);
    else
      wave_topk<16>(E, k, load, &id, &wt);
    if (lane < k) {
      s_ids[t * k + lane] = id;
      s_w[t * k + lane] = wt;
      if (blockIdx.x == 0) {
        if (p.ids_out) p.ids_out[t * k + lane] = id;
        if (p.w_out) p.w_out[t * k + lane] = wt;
      }
    }
    if (lane == 0) s_gamma[t] = p.shared_gate ? ld_dev(&p.gamma[t]) : 0.0f;
  }
  __syncthreads();

  // ------------------------------------------------ D assignment (prefetch) --
  const int nch = p.routed.inter / 32;
  const int nch_s = p.shared.inter / 32;
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
  const uint8_t* __restrict__ w2r = p.routed.w2;
  const uint8_t* __restrict__ w2sr = p.routed.w2s;

  auto down_ptrs = [&](int t, int v, int c, const uint8_t*& cp, const uint8_t*& sp, int& nch_u) {
    const Unit2 u = unit2(p, v);
    const bool sh = (u.slot == k);
    const int e = sh ? 0 : s_ids[t * k + u.slot];
    nch_u = sh ? nch_s : nch;
    const size_t rec = (static_cast<size_t>(e) * nch_u + u.chunk) * H + c;
    cp = (sh ? p.shared.w2 : w2r) + rec * 16;
    sp = (sh ? p.shared.w2s : w2sr) + rec * 2;
  };

  uint4 pq[kUD];
  uint32_t ps[kUD];
  const bool have_first = g_first < p.d_groups;
  if (have_first) {
    const int t = g_first / nrg;
    const int c = (g_first - t * nrg) * kWave + lane;
#pragma unroll
    for (int i = 0; i < kUD; ++i) {
      const int v = sub + bpg * (wave + kFWaves * i);
      if (v < upg) {
        const uint8_t *cp, *sp;
        int nu;
        down_ptrs(t, v, c, cp, sp, nu);
        pq[i] = *reinterpret_cast<const uint4*>(cp);
        ps[i] = *reinterpret_cast<const uint16_t*>(sp);
      }
    }
  }

  // ---------------------------------------------------------------- W --
  {
    const int group = lane / LPR, col = lane % LPR;
    const int NG = NW * GPW;
    const int total = T * (k * p.routed.inter + p.shared.inter);
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
    if (T == 1) load_x(0);
    for (int j0 = 0; (gw * GPW) + NG * j0 < total; j0 += kUW) {
      Unit13 un[kUW];
      uint4 qg[kUW][CPL], qu[kUW][CPL];
      uint32_t sg[kUW][CPL], su[kUW][CPL];
#pragma unroll
      for (int jj = 0; jj < kUW; ++jj) {
        un[jj] = unit13(p, gw * GPW + group + NG * (j0 + jj), total);
        const bool sh = (un[jj].slot == k);
        const int I = sh ? p.shared.inter : p.routed.inter;
        const int e = sh ? 0 : s_ids[un[jj].t * k + un[jj].slot];
        const uint8_t* __restrict__ codes =
            (sh ? p.shared.w13 : p.routed.w13) + static_cast<size_t>(e) * 2 * I * row_bytes;
        const uint8_t* __restrict__ scales =
            (sh ? p.shared.w13s : p.routed.w13s) + static_cast<size_t>(e) * 2 * I * srow_bytes;
        const size_t rr = static_cast<size_t>(un[jj].r);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int j = col + LPR * c;
          qg[jj][c] = *reinterpret_cast<const uint4*>(codes + rr * row_bytes + 16 * j);
          qu[jj][c] = *reinterpret_cast<const uint4*>(codes + (I + rr) * row_bytes + 16 * j);
          sg[jj][c] = *reinterpret_cast<const uint16_t*>(scales + rr * srow_bytes + 2 * j);
          su[jj][c] = *reinterpret_cast<const uint16_t*>(scales + (I + rr) * srow_bytes + 2 * j);
        }
      }
#pragma unroll
      for (int jj = 0; jj < kUW; ++jj) {
        if (T != 1) load_x(un[jj].t);
        float ag = 0.0f, au = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          ag += chunk_dot_bf16(qg[jj][c], sg[jj][c], xr[c]);
          au += chunk_dot_bf16(qu[jj][c], su[jj][c], xr[c]);
        }
        ag = group_sum<LPR>(ag);
        au = group_sum<LPR>(au);
        if (col == 0 && un[jj].valid) {
          const bool sh = (un[jj].slot == k);
          const int e = sh ? 0 : s_ids[un[jj].t * k + un[jj].slot];
          const float* gsc = (sh ? p.shared.gsc : p.routed.gsc) + 3 * e;
          const float hv = swiglu(p.act, ag * gsc[0], au * gsc[1], p.gate_max, p.up_absmax);
          st_dev(&p.h[(static_cast<size_t>(un[jj].t) * p.nslots + un[jj].slot) * p.Imax + un[jj].r],
                 hv);
        }
      }
    }
  }
  grid_barrier(&p.sync[1], static_cast<uint32_t>(G), &p.sync[3], p.spin_limit);

  // ---------------------------------------------------------------- D --
  bool first = true;
  for (int g = g_first; g < p.d_groups; g += g_step) {
    const int t = g / nrg;
    const int rg = g - t * nrg;
    const int c = rg * kWave + lane;
    float acc = 0.0f;
    for (int i0 = 0; sub + bpg * (wave + kFWaves * i0) < upg; i0 += kUD) {
      uint4 q[kUD];
      uint32_t sc[kUD];
      if (first && i0 == 0) {
#pragma unroll
        for (int ii = 0; ii < kUD; ++ii) {
          q[ii] = pq[ii];
          sc[ii] = ps[ii];
        }
      } else {
#pragma unroll
        for (int ii = 0; ii < kUD; ++ii) {
          const int v = sub + bpg * (wave + kFWaves * (i0 + ii));
          if (v < upg) {
            const uint8_t *cp, *sp;
            int nu;
            down_ptrs(t, v, c, cp, sp, nu);
            q[ii] = *reinterpret_cast<const uint4*>(cp);
            sc[ii] = *reinterpret_cast<const uint16_t*>(sp);
          }
        }
      }
      float hv[kUD][32];
#pragma unroll
      for (int ii = 0; ii < kUD; ++ii) {
        const int v = sub + bpg * (wave + kFWaves * (i0 + ii));
        if (v < upg) {
          const Unit2 u = unit2(p, v);
          const float* hrow = p.h + (static_cast<size_t>(t) * p.nslots + u.slot) * p.Imax;
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const float4 f =
                ld_dev_x4_uniform(hrow, static_cast<uint32_t>((32 * u.chunk + 4 * m) * 4));
            hv[ii][4 * m + 0] = f.x;
            hv[ii][4 * m + 1] = f.y;
            hv[ii][4 * m + 2] = f.z;
            hv[ii][4 * m + 3] = f.w;
          }
        }
      }
#pragma unroll
      for (int ii = 0; ii < kUD; ++ii) {
        const int v = sub + bpg * (wave + kFWaves * (i0 + ii));
        if (v < upg) {
          const Unit2 u = unit2(p, v);
          const bool sh = (u.slot == k);
          const int e = sh ? 0 : s_ids[t * k + u.slot];
          const float wslot = sh ? s_gamma[t] : s_w[t * k + u.slot];
          const float gd = (sh ? p.shared.gsc : p.routed.gsc)[3 * e + 2];
          acc = fmaf(chunk_dot_f32(q[ii], sc[ii], hv[ii]), wslot * gd, acc);
        }
      }
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
        float* part = p.part + (static_cast<size_t>(g) * bpg) * kWave;
        st_dev(&part[sub * kWave + lane], o);
        wait_mem();
        uint32_t old = 0;
        if (lane == 0) old = add_dev(&p.cnt[g], 1u);
        old = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(old)));
        if (old == static_cast<uint32_t>(bpg - 1)) {
          float ysum = 0.0f;
          for (int s2 = 0; s2 < bpg; ++s2) ysum += ld_dev(&part[s2 * kWave + lane]);
          *yout = f32_to_bf16_bits(ysum);
          if (lane == 0) st_dev(&p.cnt[g], 0u);
        }
      }
    }
    __syncthreads();
  }

  // -------------------------------------------------------------- exit --
  wait_mem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = add_dev(&p.sync[2], 1u);
    if (old == static_cast<uint32_t>(G - 1)) {
      st_dev(&p.sync[0], 0u);
      st_dev(&p.sync[1], 0u);
      st_dev(&p.sync[2], 0u);
    }
  }
}

template <int LPR>
static hipError_t launch_fused_lpr(const FusedParams& p, int grid, hipStream_t s) {
  const int cpl = p.H / (32 * LPR);
  dim3 g(grid), b(kFWaves * kWave);
  switch (cpl) {
    case 1: moe_decode_fused_kernel<LPR, 1><<<g, b, 0, s>>>(p); break;
    case 2: moe_decode_fused_kernel<LPR, 2><<<g, b, 0, s>>>(p); break;
    case 3: moe_decode_fused_kernel<LPR, 3><<<g, b, 0, s>>>(p); break;
    case 4: moe_decode_fused_kernel<LPR, 4><<<g, b, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_fused(const FusedParams& p, int grid, hipStream_t s) {
  int lpr = 0, cpl = 0;
  gateup_geometry(p.H, &lpr, &cpl);
  switch (lpr) {
    case 64: return launch_fused_lpr<64>(p, grid, s);
    case 32: return launch_fused_lpr<32>(p, grid, s);
    case 16: return launch_fused_lpr<16>(p, grid, s);
    case 8: return launch_fused_lpr<8>(p, grid, s);
    default: return hipErrorInvalidValue;
  }
}

int fused_block_threads() { return kFWaves * kWave; }

}  // namespace ftmoe
