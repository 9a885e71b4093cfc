// prefill.hip -- the many-token path: routed (token, slot) pairs grouped by
// expert, then two bf16 MFMA grouped GEMMs per expert and a combine.
//
// FreeToken fork PR #84 (page 1), the bullet on #578: NVFP4 prefill experts are
// dequantised and run as dense products; 1Cat-vLLM PR #525 (page 3) runs NVFP4
// experts as weight-only 4-bit GEMMs with 16-bit activations.  Here the dense
// product is a gfx950 MFMA (v_mfma_f32_16x16x32_bf16).  Every e2m1 x e4m3
// product has at most 6 significant bits, so the dequantised tile values
// code * scale are exact in bf16; the fp32 global scale multiplies the fp32
// accumulator instead.
//
//  1. grouping          per-expert counts, offsets and the work-unit table, and the
//                        pairs scattered into per-expert groups (one block for few
//                        pairs; histogram, scan and scatter kernels for many)
//  2. pf_gateup_kernel   h = SwiGLU(W_gate x, W_up x) per unit of <= 256 tokens
//                        and 64 h columns; h stored as a bf16 (hi, lo) pair
//  3. pf_down_kernel     o = W_down (h_hi + h_lo) per unit and 128 output rows,
//                        times the global scale and the routing weight (or the
//                        shared gate), into a per-(token, slot) buffer
//  4. pf_combine_kernel  y = bf16(sum over slots in slot order)
//
// Work unit: (bank, expert, first sorted position, count <= 256).  The shared
// expert is one more bank whose units take consecutive tokens.  Blocks are
// mapped so that the tiles of one unit land on one XCD (dispatch is round-robin
// over the 8 XCDs), where they share the unit's activation rows in L2.
#include "ftmoe_device.hpp"
#include "ftmoe_kernels.hpp"

namespace ftmoe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

namespace {

constexpr int kPfRows = 128;               // weight rows per block tile
constexpr unsigned kPersistentBlocks = 256;  // one per CU of MI355X (LDS holds one)
constexpr int kPfSlab = 64;                // K elements per LDS slab
constexpr int kLdsRowU4 = kPfSlab / 8 + 1; // 16-byte words per LDS row (one of padding)
// 16-byte words per LDS slab tile: one of padding, so that tiles t and t + 1 start 4 banks
// apart (threads writing the same row of different tiles at once do not collide)
constexpr int kTileU4 = kPfRows * kLdsRowU4 + 1;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma_bf16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
// 16 x 16 x 32 product of 16-bit operands: fp16 (H16) or bf16
template <bool H16>
__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
  if constexpr (H16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return mfma_bf16(a, b, c);
}

// KPT = 16 or 32 consecutive K elements of one row (KPT/2 code bytes, KPT/16 scale
// bytes) -> KPT/8 x 16 B of bf16.
template <int KPT> struct Codes;
template <> struct Codes<16> {
  uint2 q;
  uint32_t s;
  __device__ __forceinline__ void load(const uint8_t* c, const uint8_t* sc) {
    q = *reinterpret_cast<const uint2*>(c);
    s = *sc;
  }
  template <bool H16 = false>
  __device__ __forceinline__ void to_lds(uint4* dst) const {
    const float s0 = e4m3_byte_to_f32<0>(s);
    dst[0] = dequant8_tile<H16>(q.x, s0);
    dst[1] = dequant8_tile<H16>(q.y, s0);
  }
};
template <> struct Codes<32> {
  uint4 q;
  uint32_t s;
  __device__ __forceinline__ void load(const uint8_t* c, const uint8_t* sc) {
    q = *reinterpret_cast<const uint4*>(c);
    s = *reinterpret_cast<const uint16_t*>(sc);
  }
  template <bool H16 = false>
  __device__ __forceinline__ void to_lds(uint4* dst) const {
    const float s0 = e4m3_byte_to_f32<0>(s), s1 = e4m3_byte_to_f32<1>(s);
    dst[0] = dequant8_tile<H16>(q.x, s0);
    dst[1] = dequant8_tile<H16>(q.y, s0);
    dst[2] = dequant8_tile<H16>(q.z, s1);
    dst[3] = dequant8_tile<H16>(q.w, s1);
  }
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Block -> (unit, tile): blocks b = 8 * ntiles * q + 8 * tile + x run unit 8q + x.
__device__ __forceinline__ void unit_tile(int ntiles, int* u, int* tile) {
  const int b = blockIdx.x;
  *u = (b / (8 * ntiles)) * 8 + (b & 7);
  *tile = (b >> 3) % ntiles;
}

}  // namespace

// ------------------------------------------------------------- grouping --
//
// The position of a pair inside its expert's group does not change any result:
// every token is one MFMA column, computed with the same operands and the same K
// order wherever it sits, and the combine sums a token's slots in slot order.  So
// the groups are filled with atomic cursors (any order is as good as another).

namespace {

// Exclusive offsets of the per-expert counts and the work-unit table, by one block
// of kMaxExperts threads; count[e] is thread e's count (0 for e >= E).  Writes
// offset[], cursor[] (= offset) and units[] / nunits.
__device__ void group_units(const PrefillParams& p, int count, int* cursor) {
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_units[kMaxExperts];
  const int e = threadIdx.x;
  const int ut = p.unit_tokens;
  const int nu = (count + ut - 1) / ut;
  // inclusive scans of counts and unit counts: within each wave by lane shuffles,
  // then each wave adds the totals of the waves before it (two block barriers)
  __shared__ int s_wa[kMaxExperts / kWave], s_wb[kMaxExperts / kWave];
  const int lane = e & (kWave - 1), wv = e / kWave;
  int a = count, b = nu;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int ta = __shfl_up(a, off, kWave), tb = __shfl_up(b, off, kWave);
    if (lane >= off) {
      a += ta;
      b += tb;
    }
  }
  if (lane == kWave - 1) {
    s_wa[wv] = a;
    s_wb[wv] = b;
  }
  __syncthreads();
  for (int w = 0; w < wv; ++w) {
    a += s_wa[w];
    b += s_wb[w];
  }
  s_cnt[e] = a;
  s_units[e] = b;
  __syncthreads();
  if (e < p.E) {
    const int off = s_cnt[e] - count;
    const int ubase = s_units[e] - nu;
    p.offset[e] = off;
    cursor[e] = off;
    for (int c = 0; c < nu; ++c) {
      PfUnit un;
      un.bank = 0;
      un.expert = e;
      un.start = off + c * ut;
      un.count = min(ut, count - c * ut);
      p.units[ubase + c] = un;
    }
  }
  if (e == 0) {
    int n = s_units[kMaxExperts - 1];
    if (p.shared.inter > 0) {
      for (int t0 = 0; t0 < p.T; t0 += ut) {
        PfUnit un;
        un.bank = 1;
        un.expert = 0;
        un.start = t0;
        un.count = min(ut, p.T - t0);
        p.units[n++] = un;
      }
    }
    *p.nunits = n;
  }
}

__device__ __forceinline__ int valid_expert(const PrefillParams& p, int pair) {
  const int e = p.ids[pair];
  return (e >= 0 && e < p.E) ? e : -1;
}

}  // namespace

// Whole grouping in one block (few pairs): LDS counts, offsets, LDS cursors.
__global__ __launch_bounds__(kMaxExperts) void pf_group_one_block_kernel(PrefillParams p) {
  constexpr int kPer = kGroupOneBlockPairs / kMaxExperts;  // pairs per thread, at most
  __shared__ int cnt[kMaxExperts];
  __shared__ int cur[kMaxExperts];
  const int tid = threadIdx.x;
  cnt[tid] = 0;
  // every id this thread handles, loaded at once and kept for the scatter (a reload
  // after the unit table's stores would wait for them: vmcnt completes in order)
  int ev[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int pair = tid + j * kMaxExperts;
    ev[j] = pair < p.P ? valid_expert(p, pair) : -1;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (ev[j] >= 0) atomicAdd(&cnt[ev[j]], 1);
  __syncthreads();
  group_units(p, cnt[tid], cur);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (ev[j] >= 0) p.sorted[atomicAdd(&cur[ev[j]], 1)] = tid + j * kMaxExperts;
}

// Many pairs: per-block LDS histograms added into count[] ...
__global__ __launch_bounds__(256) void pf_hist_kernel(PrefillParams p) {
  __shared__ int hist[kMaxExperts];
  for (int e = threadIdx.x; e < p.E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * kGroupPairs;
  for (int i = threadIdx.x; i < kGroupPairs; i += blockDim.x) {
    const int pair = p0 + i;
    if (pair < p.P) {
      const int e = valid_expert(p, pair);
      if (e >= 0) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < p.E; e += blockDim.x)
    if (hist[e]) atomicAdd(&p.count[e], hist[e]);
}

// ... offsets and units by one block, which also clears count[] for the next call ...
__global__ __launch_bounds__(kMaxExperts) void pf_scan_kernel(PrefillParams p) {
  const int e = threadIdx.x;
  int c = 0;
  if (e < p.E) {
    c = p.count[e];
    p.count[e] = 0;
  }
  group_units(p, c, p.cursor);
}

// ... and a scatter through global cursors: a block ranks its kScatterPairs pairs per
// expert in LDS, reserves each expert's run with ONE global atomic (one per pair
// serialised ~160 device-scope atomics on every expert's cursor), and writes its
// pairs there.
constexpr int kScatterPairs = 2048;

__global__ __launch_bounds__(256) void pf_scatter_kernel(PrefillParams p) {
  constexpr int kPer = kScatterPairs / 256;
  __shared__ int cnt[kMaxExperts];
  for (int e = threadIdx.x; e < p.E; e += 256) cnt[e] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * kScatterPairs;
  int ev[kPer], rk[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int pair = p0 + threadIdx.x + 256 * j;
    ev[j] = pair < p.P ? valid_expert(p, pair) : -1;
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) rk[j] = ev[j] >= 0 ? atomicAdd(&cnt[ev[j]], 1) : 0;
  __syncthreads();
  for (int e = threadIdx.x; e < p.E; e += 256) {  // one thread per expert: no race
    const int c = cnt[e];
    cnt[e] = c ? atomicAdd(&p.cursor[e], c) : 0;   // where the block's run of e starts
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (ev[j] >= 0) p.sorted[cnt[ev[j]] + rk[j]] = p0 + threadIdx.x + 256 * j;
}

// --------------------------------------------------------------- GEMMs --
//
// MFMA v_mfma_f32_16x16x32_bf16: A is 16 rows x 32 K, lane l holding row l % 16
// and 8 K values of group l / 16; B is 32 K x 16 columns, lane l holding column
// l % 16 and the same 8 K positions; C lane l holds rows 4 (l / 16) + j, j < 4, of
// column l % 16.  Which 8 of the 32 K positions a lane group holds only has to
// agree between A and B: here group g of a 64-wide slab holds K = 16 g + 8 j .. +8
// in step j (j = 0, 1), so a lane reads 32 contiguous bytes of a token row.
//
// A = dequantised weights: a 128-row x 64-K slab in LDS, written by all threads
// of the block and read by all its waves.  B = token rows straight from global
// memory into registers.  The 16 fragments of 16 tokens of a unit are dealt to
// the W waves round-robin (wave w takes fragments w, w + W, ...), so every wave
// computes a 128-row x (256 / W)-token tile.  Per 64-K slab a CU then reads
// W x 16 KB of A from LDS and 256 x 128 B of B through L1: W = 4 keeps both
// well inside their bandwidth at full MFMA rate.  Token rows run R slabs ahead in
// a register ring and weight codes R slabs ahead.

namespace {

// W waves of up to FR token fragments each: a unit holds up to 16 W FR tokens.
template <int W, int FR>
struct Geometry {
  static constexpr int kThreads = W * kWave;
  static constexpr int kFrags = FR;                      // token fragments per wave
  static constexpr int kUnitTokens = 16 * W * FR;
  static constexpr int kTpr = kThreads / kPfRows;        // dequantising threads per row
  static constexpr int kKpt = kPfSlab / kTpr;            // K elements each per slab
};

// Number of this wave's fragments (<= FR) in a unit of `count` tokens.
template <int W, int FR>
__device__ __forceinline__ int wave_fragments(int count, int wave) {
  const int nf = (count + 15) >> 4;
  return __builtin_amdgcn_readfirstlane(nf > wave ? min(FR, (nf - wave + W - 1) / W) : 0);
}

// Token index (within the unit) of this lane's column in fragment f.
template <int W>
__device__ __forceinline__ int frag_token(int wave, int f, int lane) {
  return (wave + W * f) * 16 + (lane & 15);
}

// The looped K loop of the down GEMM.  NB = 1: B is one 16-bit operand (fp16 h
// with fp16 weight tiles when H16, else bf16); NB = 2: B is a (hi, lo) bf16 pair
// whose two products are accumulated into the same C.
// brow[b][f]: this lane's B row for fragment f (slab 0, lane group offset applied).
// wc / ws: this thread's codes and scales of slab 0 (kKpt K elements of tile row
// drow, part dpart of the slab); wc_step / ws_step: their slab strides.
// Token rows run R - 1 slabs ahead (a ring of R), weight codes RW slabs ahead (a
// ring of RW; RW is a multiple of R and even, and the loop is unrolled RW times so
// that every ring slot and LDS buffer index is a compile-time constant).
template <int W, int FR, int NB, int R, int RW, bool H16>
__device__ __forceinline__ void pf_mainloop(
    const uint8_t* wc, size_t wc_step, const uint8_t* ws, size_t ws_step,
    const uint16_t* const (&brow)[NB][FR], int nfr, int nslab,
    uint4 (*lds)[kTileU4], int drow, int dpart, int lane, f32x4 (&acc)[FR][8]) {
  static_assert(RW % R == 0 && RW % 2 == 0, "ring depths");
  constexpr int KPT = Geometry<W, FR>::kKpt;
  uint4 xr[R][NB][FR][2];
  Codes<KPT> cr[RW];
  // Every load is unconditional (a slab index past the end is clamped to the last
  // slab, a fragment past the unit repeats a valid row): a load under a branch
  // makes the compiler's wait counting fall back to waiting for every load.
  auto clampslab = [&](int s) { return s < nslab ? s : nslab - 1; };
  auto load_b = [&](int s, uint4 (&dst)[NB][FR][2]) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int f = 0; f < FR; ++f) {
        dst[b][f][0] = ld16(brow[b][f] + s * kPfSlab);
        dst[b][f][1] = ld16(brow[b][f] + s * kPfSlab + 8);
      }
  };
  auto load_codes = [&](int s, Codes<KPT>& c) {
    c.load(wc + clampslab(s) * wc_step, ws + clampslab(s) * ws_step);
  };
  uint4* const my0 = &lds[0][drow * kLdsRowU4 + dpart * (KPT / 8)];
  uint4* const my1 = &lds[1][drow * kLdsRowU4 + dpart * (KPT / 8)];

  // prologue: codes of slabs 0 .. RW-1, activations of slabs 0 .. R-2, weights of
  // slab 0.  The loads keep this order (scheduling barriers): the compiler's wait
  // counts at the loop head take the worse of this path and the loop's own, so a
  // late-issued early slab here would make every pass of the loop wait for all
  // loads in flight.
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    load_codes(r, cr[r]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int r = 0; r < R - 1; ++r) {
    load_b(clampslab(r), xr[r]);
    __builtin_amdgcn_sched_barrier(0);
  }
  cr[0].template to_lds<H16>(my0);
  load_codes(RW, cr[0]);
  __builtin_amdgcn_sched_barrier(0);

  // Whole passes of RW slabs; in the last pass the slabs past the end repeat the
  // last slab's loads and dequantisation but add nothing.  (An early exit inside
  // the unrolled pass would give the compiler paths into the loop head with fewer
  // loads in flight, and it would then wait for every load at each pass.)
  for (int s0 = 0; s0 < nslab; s0 += RW) {
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int s = s0 + r;
      const bool live = s < nslab;
      __syncthreads();  // weights of slab s are in LDS; slab s - 1's buffer is free
      load_b(clampslab(s + R - 1), xr[(r + R - 1) % R]);
      const uint4* tile = lds[r & 1];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint4 a[8];
#pragma unroll
        for (int rf = 0; rf < 8; ++rf)
          a[rf] = tile[(rf * 16 + (lane & 15)) * kLdsRowU4 + (lane >> 4) * 2 + j];
        // operand b outermost: consecutive MFMAs write different accumulators
        // (an MFMA right after one into the same accumulator waits for it)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int f = 0; f < FR; ++f) {
            if (live && f < nfr) {
#pragma unroll
              for (int rf = 0; rf < 8; ++rf)
                acc[f][rf] = mfma16<H16>(a[rf], xr[r % R][b][f][j], acc[f][rf]);
            }
          }
      }
      // weights of slab s + 1 (its buffer was last read in iteration s - 1), then
      // the codes of slab s + 1 + RW into the freed ring slot
      const int c = (r + 1) % RW;
      cr[c].template to_lds<H16>((r & 1) ? my0 : my1);
      load_codes(s + 1 + RW, cr[c]);
    }
  }
}

// The gate|up K loop.  Row-major weights are fetched per super-slab of 256 K
// elements: 8 lanes read the 128 code bytes of one row (one whole cache line), so
// a wave load covers 8 rows in full lines, and the HBM stream is line-sized runs
// instead of 32-byte pieces.  Each of the 256 threads fetches 4 such pieces (rows
// (tid >> 3) + 32 i, K segment tid & 7), RS super-slabs ahead in a register ring,
// and dequantises them into the four 64-K slab tiles of the super-slab in LDS.
// Token rows run R - 1 slabs ahead (R divides 4, so every ring slot is a
// compile-time constant in the unrolled loop).
constexpr int kSuperSlab = 4 * kPfSlab;  // 256 K elements: 128 code bytes per row

template <int FR, int R, int RS>
__device__ __forceinline__ void pf_mainloop_rows(
    const uint8_t* wc, const uint8_t* ws, const long long (&rowoff)[4], int H,
    const uint16_t* const (&brow)[1][FR], int nfr, int nslab,
    uint4 (*tiles)[kTileU4], int lane, f32x4 (&acc)[FR][8]) {
  static_assert(4 % R == 0, "token ring depth divides the slabs of a super-slab");
  const int tid = threadIdx.x;
  const int seg = tid & 7;  // 32-K segment of the super-slab
  const int nss = nslab / 4;
  uint4 xr[R][FR][2];
  uint4 qr[RS][4];
  uint32_t sr[RS][4];
  auto clampslab = [&](int s) { return s < nslab ? s : nslab - 1; };
  auto clampss = [&](int ss) { return ss < nss ? ss : nss - 1; };
  // every load unconditional (see pf_mainloop)
  auto load_b = [&](int s, uint4 (&dst)[FR][2]) {
#pragma unroll
    for (int f = 0; f < FR; ++f) {
      dst[f][0] = ld16(brow[0][f] + s * kPfSlab);
      dst[f][1] = ld16(brow[0][f] + s * kPfSlab + 8);
    }
  };
  auto load_w = [&](int ss, uint4 (&q)[4], uint32_t (&sc)[4]) {
    const int c = clampss(ss);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[i] = ld16(wc + rowoff[i] * (H / 2) + c * (kSuperSlab / 2));
      sc[i] = *reinterpret_cast<const uint16_t*>(ws + rowoff[i] * (H / 16) + c * (kSuperSlab / 16));
    }
  };
  auto dequant = [&](const uint4 (&q)[4], const uint32_t (&sc)[4]) {
    uint4* const t = tiles[seg >> 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid >> 3) + 32 * i;
      uint4* dst = t + row * kLdsRowU4 + (seg & 1) * 4;
      const float s0 = e4m3_byte_to_f32<0>(sc[i]), s1 = e4m3_byte_to_f32<1>(sc[i]);
      dst[0] = dequant8_bf16(q[i].x, s0);
      dst[1] = dequant8_bf16(q[i].y, s0);
      dst[2] = dequant8_bf16(q[i].z, s1);
      dst[3] = dequant8_bf16(q[i].w, s1);
    }
  };

  // prologue: weights of super-slabs 0 .. RS-1, token rows of slabs 0 .. R-2, in
  // this order (see pf_mainloop)
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    load_w(r, qr[r], sr[r]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int r = 0; r < R - 1; ++r) {
    load_b(clampslab(r), xr[r]);
    __builtin_amdgcn_sched_barrier(0);
  }

  for (int ss0 = 0; ss0 < nss; ss0 += RS) {
#pragma unroll
    for (int rr = 0; rr < RS; ++rr) {
      const int ss = ss0 + rr;
      const bool live = ss < nss;  // the last pass may run past the end (see pf_mainloop)
      __syncthreads();  // the previous super-slab's MFMAs are done with the tiles
      dequant(qr[rr], sr[rr]);
      load_w(ss + RS, qr[rr], sr[rr]);
      __syncthreads();  // this super-slab's tiles are written
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int s = 4 * ss + j;
        load_b(clampslab(s + R - 1), xr[(j + R - 1) % R]);
        const uint4* tile = tiles[j];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          uint4 a[8];
#pragma unroll
          for (int rf = 0; rf < 8; ++rf)
            a[rf] = tile[(rf * 16 + (lane & 15)) * kLdsRowU4 + (lane >> 4) * 2 + st];
#pragma unroll
          for (int f = 0; f < FR; ++f) {
            if (live && f < nfr) {
#pragma unroll
              for (int rf = 0; rf < 8; ++rf)
                acc[f][rf] = mfma_bf16(a[rf], xr[j % R][f][st], acc[f][rf]);
            }
          }
        }
      }
    }
  }
}

// The down K loop for K = 64 NS with the whole weight tile in LDS: every thread's
// codes of all NS slabs are loaded and dequantised up front (one barrier), then the
// MFMAs run over the NS slabs with no further barrier, token rows (NB operands)
// R - 1 slabs ahead in a ring whose slots are constants (the loop is unrolled).
template <int W, int FR, int NB, int R, int NS, bool H16>
__device__ __forceinline__ void pf_mainloop_whole_a(
    const uint8_t* wc, size_t wc_step, const uint8_t* ws, size_t ws_step,
    const uint16_t* const (&brow)[NB][FR], int nfr, uint4 (*lds)[kTileU4],
    int drow, int dpart, int lane, f32x4 (&acc)[FR][8]) {
  constexpr int KPT = Geometry<W, FR>::kKpt;
  static_assert(R >= 2 && R <= NS, "ring depth");
  Codes<KPT> cr[NS];
  uint4 xr[R][NB][FR][2];
  auto load_b = [&](int s, uint4 (&dst)[NB][FR][2]) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int f = 0; f < FR; ++f) {
        dst[b][f][0] = ld16(brow[b][f] + s * kPfSlab);
        dst[b][f][1] = ld16(brow[b][f] + s * kPfSlab + 8);
      }
  };
#pragma unroll
  for (int s = 0; s < NS; ++s) cr[s].load(wc + s * wc_step, ws + s * ws_step);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < R - 1; ++r) {
    load_b(r, xr[r]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int s = 0; s < NS; ++s)
    cr[s].template to_lds<H16>(&lds[s][drow * kLdsRowU4 + dpart * (KPT / 8)]);
  __syncthreads();
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s + R - 1 < NS) load_b(s + R - 1, xr[(s + R - 1) % R]);
    const uint4* tile = lds[s];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint4 a[8];
#pragma unroll
      for (int rf = 0; rf < 8; ++rf)
        a[rf] = tile[(rf * 16 + (lane & 15)) * kLdsRowU4 + (lane >> 4) * 2 + j];
      // operand b outermost: consecutive MFMAs write different accumulators
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int f = 0; f < FR; ++f) {
          if (f < nfr) {
#pragma unroll
            for (int rf = 0; rf < 8; ++rf)
              acc[f][rf] = mfma16<H16>(a[rf], xr[s % R][b][f][j], acc[f][rf]);
          }
        }
    }
  }
}

// The gate|up K loop for H = 256 NSS, fully unrolled (no loop back edge, so the
// register rings below need no copies and every slot index is a constant): the
// weight tiles are double-buffered in LDS (8 slab tiles), so super-slab ss + 1 is
// dequantised, a quarter before each slab's MFMAs, while super-slab ss is being
// multiplied, with one barrier per super-slab; token rows run R - 1 slabs ahead,
// weight codes RS super-slabs ahead.
template <int NSS, int FR, int R, int RS>
__device__ __forceinline__ void pf_mainloop_rows_unrolled(
    const uint8_t* wc, const uint8_t* ws, const long long (&rowoff)[4], int H,
    const uint16_t* const (&brow)[1][FR], int nfr, uint4 (*tiles)[kTileU4],
    int lane, f32x4 (&acc)[FR][8]) {
  constexpr int NS = 4 * NSS;  // 64-K slabs
  static_assert(RS >= 1 && RS <= NSS && R >= 2, "ring depths");
  const int tid = threadIdx.x;
  const int seg = tid & 7;  // 32-K segment of the super-slab
  uint4 xr[R][FR][2];
  uint4 qr[RS][4];
  uint32_t sr[RS][4];
  auto load_b = [&](int s, uint4 (&dst)[FR][2]) {
#pragma unroll
    for (int f = 0; f < FR; ++f) {
      dst[f][0] = ld16(brow[0][f] + s * kPfSlab);
      dst[f][1] = ld16(brow[0][f] + s * kPfSlab + 8);
    }
  };
  auto load_w = [&](int ss, uint4 (&q)[4], uint32_t (&sc)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[i] = ld16(wc + rowoff[i] * (H / 2) + ss * (kSuperSlab / 2));
      sc[i] = *reinterpret_cast<const uint16_t*>(ws + rowoff[i] * (H / 16) + ss * (kSuperSlab / 16));
    }
  };
  // piece i (tile rows (tid >> 3) + 32 i) of a super-slab into LDS buffer `buf`
  auto dequant_piece = [&](const uint4 (&q)[4], const uint32_t (&sc)[4], int i, int buf) {
    uint4* dst = tiles[4 * buf + (seg >> 1)] + ((tid >> 3) + 32 * i) * kLdsRowU4 + (seg & 1) * 4;
    const float s0 = e4m3_byte_to_f32<0>(sc[i]), s1 = e4m3_byte_to_f32<1>(sc[i]);
    dst[0] = dequant8_bf16(q[i].x, s0);
    dst[1] = dequant8_bf16(q[i].y, s0);
    dst[2] = dequant8_bf16(q[i].z, s1);
    dst[3] = dequant8_bf16(q[i].w, s1);
  };

  // prologue: weights of super-slabs 0 .. RS-1, token rows of slabs 0 .. R-2,
  // super-slab 0 dequantised into buffer 0
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    load_w(r, qr[r], sr[r]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int r = 0; r < R - 1 && r < NS; ++r) {
    load_b(r, xr[r]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) dequant_piece(qr[0], sr[0], i, 0);
  if (RS < NSS) load_w(RS, qr[0], sr[0]);
  __syncthreads();

#pragma unroll
  for (int ss = 0; ss < NSS; ++ss) {
    const int nx = (ss + 1) % RS;  // ring slot of super-slab ss + 1
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = 4 * ss + j;
      if (s + R - 1 < NS) load_b(s + R - 1, xr[(s + R - 1) % R]);
      if (ss + 1 < NSS) dequant_piece(qr[nx], sr[nx], j, (ss + 1) & 1);
      const uint4* tile = tiles[4 * (ss & 1) + j];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        uint4 a[8];
#pragma unroll
        for (int rf = 0; rf < 8; ++rf)
          a[rf] = tile[(rf * 16 + (lane & 15)) * kLdsRowU4 + (lane >> 4) * 2 + st];
#pragma unroll
        for (int f = 0; f < FR; ++f) {
          if (f < nfr) {
#pragma unroll
            for (int rf = 0; rf < 8; ++rf)
              acc[f][rf] = mfma_bf16(a[rf], xr[s % R][f][st], acc[f][rf]);
          }
        }
      }
    }
    if (ss + 1 + RS < NSS) load_w(ss + 1 + RS, qr[nx], sr[nx]);
    __syncthreads();  // buffer (ss + 1) & 1 written; buffer ss & 1 free
  }
}

}  // namespace

// Blocks of 4 waves run two per CU, blocks of 8 waves one per CU.
template <int W>
constexpr int kBlocksPerCu = W == 4 ? 2 : 1;

// NSS > 0: H = 256 NSS with the unrolled K loop (R, RS its ring depths); NSS = 0:
// any H with the looped one.
template <int FR, int R, int RS, int BPC, int NSS>
__global__ __launch_bounds__(256, BPC) void pf_gateup_kernel(PrefillParams p) {
  constexpr int W = 4;
  __shared__ uint4 tiles[NSS > 0 ? 8 : 4][kTileU4];
  int u, tile;
  unit_tile(p.ntiles1, &u, &tile);
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

  // weight fetch: tile rows (tid >> 3) + 32 i (gate rows n0 + (tid >> 3) + 32 i for
  // i < 2, up rows I + n0 + (tid >> 3) + 32 (i - 2)), segment tid & 7; the row
  // offsets of the four pieces are the same for every thread
  const size_t row0 = static_cast<size_t>(un.expert) * 2 * I + n0 + (tid >> 3);
  const uint8_t* wc = bank.w13 + row0 * (H / 2) + (tid & 7) * 16;
  const uint8_t* ws = bank.w13s + row0 * (H / 16) + (tid & 7) * 2;
  const long long rowoff[4] = {0, 32, I, I + 32};

  // B rows: this lane's tokens; columns past the unit's count repeat its last token
  const int nfr = wave_fragments<W, FR>(un.count, wave);
  const uint16_t* brow[1][FR];
#pragma unroll
  for (int f = 0; f < FR; ++f) {
    const int m = min(frag_token<W>(wave, f, lane), un.count - 1);
    const int tq = p.sorted[un.start + m] / p.k;  // read for both banks (in bounds: a
    const int t = un.bank ? un.start + m : tq;    // shared unit's start + m < T <= P)
    brow[0][f] = p.x + static_cast<size_t>(t) * H + (lane >> 4) * 16;
  }

  f32x4 acc[FR][8];
#pragma unroll
  for (int f = 0; f < FR; ++f)
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[f][r] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (NSS > 0)
    pf_mainloop_rows_unrolled<NSS, FR, R, RS>(wc, ws, rowoff, H, brow, nfr, tiles, lane, acc);
  else
    pf_mainloop_rows<FR, R, RS>(wc, ws, rowoff, H, brow, nfr, H / kPfSlab, tiles, lane, acc);

  // epilogue: rows r < 4 are gate columns n0 + 16 r + 4 (lane / 16) + jj, r + 4 the
  // matching up columns
  const float gg = bank.gsc[un.expert * 3 + 0], gu = bank.gsc[un.expert * 3 + 1];
#pragma unroll
  for (int f = 0; f < FR; ++f) {
    const int m = frag_token<W>(wave, f, lane);
    if (f >= nfr || m >= un.count) continue;
    const size_t row = un.bank ? static_cast<size_t>(p.P) + un.start + m
                               : static_cast<size_t>(un.start) + m;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int col = n0 + r * 16 + (lane >> 4) * 4;
      float hv[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        hv[jj] = swiglu(p.act, acc[f][r][jj] * gg, acc[f][r + 4][jj] * gu, p.gate_max, p.up_absmax);
      store_h4(p.hhi, p.hlo, row * p.Imax + col, hv, p.h16);
    }
  }
}

// NS > 0: I = 64 NS for both banks, the whole weight tile in LDS
// (pf_mainloop_whole_a, R its token ring depth); NS = 0: any I, looped.
// H16: h is fp16 (one operand, fp16 weight tiles), else a bf16 (hi, lo) pair.
template <int W, int FR, int R, int RW, int NS, bool H16>
__global__ __launch_bounds__(W * kWave, kBlocksPerCu<W>) void pf_down_kernel(PrefillParams p) {
  using G = Geometry<W, FR>;
  constexpr int NB = H16 ? 1 : 2;
  __shared__ uint4 lds[NS > 0 ? NS : 2][kTileU4];
  int u, tile;
  unit_tile(p.ntiles2, &u, &tile);
  const int nun = *p.nunits;  // both loads issued before either is waited for
  const PfUnit un = p.units[u];  // in bounds: the table has kUnitSlack spare entries
  __asm__ volatile("" ::: "memory");  // keeps them here (not sunk past the check)
  if (u >= nun) return;
  const Bank bank = un.bank ? p.shared : p.routed;
  const int I = bank.inter;
  const int H = p.H;
  const int h0 = tile * kPfRows;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // dequantisation: output row drow of the tile, kKpt K elements at part dpart of
  // each 64-K slab (two 32-K chunks, K-chunk-major: chunk c of row h at
  // ((e * I/32 + c) * H + h) * 16, its two scale bytes at (...) * 2)
  const int drow = tid / G::kTpr, dpart = tid % G::kTpr;
  const int kofs = dpart * G::kKpt;  // K offset within the slab
  const size_t chunk0 = static_cast<size_t>(un.expert) * (I / 32) + (kofs >> 5);
  const uint8_t* wc = bank.w2 + (chunk0 * H + h0 + drow) * 16 + (kofs & 31) / 2;
  const uint8_t* ws = bank.w2s + (chunk0 * H + h0 + drow) * 2 + (kofs & 31) / 16;

  const int nfr = wave_fragments<W, FR>(un.count, wave);
  const uint16_t* brow[NB][FR];
#pragma unroll
  for (int f = 0; f < FR; ++f) {
    const int m = min(frag_token<W>(wave, f, lane), un.count - 1);
    const size_t row = un.bank ? static_cast<size_t>(p.P) + un.start + m
                               : static_cast<size_t>(un.start) + m;
    brow[0][f] = p.hhi + row * p.Imax + (lane >> 4) * 16;
    if constexpr (!H16) brow[NB - 1][f] = p.hlo + row * p.Imax + (lane >> 4) * 16;
  }

  // where each fragment's outputs go, and their weights: looked up before the main
  // loop, so that the epilogue does not wait on a chain of dependent loads
  int ot[FR], oslot[FR];
  float owt[FR];
#pragma unroll
  for (int f = 0; f < FR; ++f) {
    const int m = min(frag_token<W>(wave, f, lane), un.count - 1);
    if (un.bank) {
      ot[f] = un.start + m;
      oslot[f] = p.k;
      owt[f] = p.gamma[ot[f]];
    } else {
      const int pair = p.sorted[un.start + m];
      ot[f] = pair / p.k;
      oslot[f] = pair - ot[f] * p.k;
      owt[f] = p.w[pair];
    }
  }

  f32x4 acc[FR][8];
#pragma unroll
  for (int f = 0; f < FR; ++f)
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[f][r] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (NS > 0)
    pf_mainloop_whole_a<W, FR, NB, R, NS, H16>(wc, static_cast<size_t>(2) * H * 16, ws,
                                               static_cast<size_t>(2) * H * 2, brow, nfr, lds,
                                               drow, dpart, lane, acc);
  else
    pf_mainloop<W, FR, NB, R, RW, H16>(wc, static_cast<size_t>(2) * H * 16, ws,
                                       static_cast<size_t>(2) * H * 2, brow, nfr, I / kPfSlab, lds,
                                       drow, dpart, lane, acc);

  // epilogue: output rows h0 + 16 r + 4 (lane / 16) + jj of token m
  const float gd = bank.gsc[un.expert * 3 + 2];
#pragma unroll
  for (int f = 0; f < FR; ++f) {
    const int m = frag_token<W>(wave, f, lane);
    if (f >= nfr || m >= un.count) continue;
    const int t = ot[f], slot = oslot[f];
    const float wt = owt[f];
    float* dst = p.out + (static_cast<size_t>(t) * p.nslots + slot) * H + h0 + (lane >> 4) * 4;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float4 v;
      v.x = (acc[f][r][0] * gd) * wt;
      v.y = (acc[f][r][1] * gd) * wt;
      v.z = (acc[f][r][2] * gd) * wt;
      v.w = (acc[f][r][3] * gd) * wt;
      *reinterpret_cast<float4*>(dst + r * 16) = v;
    }
  }
}

// y[t] = bf16(sum over slots, in slot order); a pair whose expert id is out of
// range was never computed and makes its token's row NaN.
// The down product for I = 64 NS (both banks) as a persistent kernel: one block
// per CU walks the work items (unit, 128-row tile) in the order of the
// one-block-per-item launch (item b goes to block b mod grid, so a unit's tiles
// stay on one XCD).  The whole weight tile of an item is dequantised into LDS;
// while its MFMAs run, the next item's codes are already being loaded into
// registers, so an item does not start with a memory latency.
template <int NS, int R, bool H16>
__global__ __launch_bounds__(8 * kWave, 1) void pf_down_persistent_kernel(PrefillParams p,
                                                                         int nitems) {
  constexpr int W = 8, FR = 2;
  constexpr int NB = H16 ? 1 : 2;  // h operands: fp16 h, or the bf16 (hi, lo) pair
  using G = Geometry<W, FR>;
  constexpr int KPT = G::kKpt;
  constexpr int kI = 64 * NS;
  __shared__ uint4 lds[NS][kTileU4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = p.H;
  const int nunits = *p.nunits;
  const int drow = tid / G::kTpr, dpart = tid % G::kTpr;
  const int kofs = dpart * G::kKpt;  // K offset within the slab

  auto item_unit = [&](int it, int* u, int* tile) {
    *u = (it / (8 * p.ntiles2)) * 8 + (it & 7);
    *tile = (it >> 3) % p.ntiles2;
  };
  // the first item at or after `it` (stride: the grid) whose unit exists
  auto next_item = [&](int it, int* u, int* tile) {
    for (; it < nitems; it += gridDim.x) {
      item_unit(it, u, tile);
      if (*u < nunits) break;
    }
    // uniform across the block: the unit's descriptor is then a scalar load,
    // which does not wait behind the vector loads in flight
    *u = __builtin_amdgcn_readfirstlane(*u);
    *tile = __builtin_amdgcn_readfirstlane(*tile);
    return __builtin_amdgcn_readfirstlane(it);
  };
  // Loads of an item issued one item ahead.  The memory counter completes in
  // issue order, so the (token, slot) pair indices go first: the dependent weight
  // loads of the next item then wait for them alone, not for the codes.
  Codes<KPT> cr[NS];
  int pr[FR];
  auto load_item = [&](const PfUnit& un, int tile) {
#pragma unroll
    for (int f = 0; f < FR; ++f) {
      const int m = min(frag_token<W>(wave, f, lane), un.count - 1);
      const int sv = p.sorted[un.start + m];  // read for both banks (in bounds: a shared
      pr[f] = un.bank ? 0 : sv;              // unit's start + m < T <= P)
    }
    __builtin_amdgcn_sched_barrier(0);
    const Bank bank = un.bank ? p.shared : p.routed;
    const size_t chunk0 = static_cast<size_t>(un.expert) * (kI / 32) + (kofs >> 5);
    const size_t row = static_cast<size_t>(tile) * kPfRows + drow;
    const uint8_t* wc = bank.w2 + (chunk0 * H + row) * 16 + (kofs & 31) / 2;
    const uint8_t* ws = bank.w2s + (chunk0 * H + row) * 2 + (kofs & 31) / 16;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      cr[s].load(wc + static_cast<size_t>(s) * 2 * H * 16, ws + static_cast<size_t>(s) * 2 * H * 2);
    __builtin_amdgcn_sched_barrier(0);
  };

  int u, tile;
  int it = next_item(blockIdx.x, &u, &tile);
  if (it >= nitems) return;
  PfUnit un = p.units[u];
  load_item(un, tile);
  for (;;) {
    const Bank bank = un.bank ? p.shared : p.routed;
    const int h0 = tile * kPfRows;
    __syncthreads();  // the previous item's MFMAs are done with the tile
#pragma unroll
    for (int s = 0; s < NS; ++s)
      cr[s].template to_lds<H16>(&lds[s][drow * kLdsRowU4 + dpart * (KPT / 8)]);
    // the next item (found before any load goes out: a loop with loads in flight
    // would make the compiler wait for them at its head), this item's output
    // places and weights (from its pair indices), then the next item's loads: all
    // in flight during this item's MFMAs
    int nu = 0, ntile = 0;
    const int nit = next_item(it + gridDim.x, &nu, &ntile);
    // read unconditionally (a valid index), so that it is a scalar load
    const PfUnit nun = p.units[nit < nitems ? nu : u];
    const int nfr = wave_fragments<W, FR>(un.count, wave);
    const uint16_t* brow[NB][FR];
    int ot[FR], oslot[FR];
    float owt[FR];
#pragma unroll
    for (int f = 0; f < FR; ++f) {
      const int m = min(frag_token<W>(wave, f, lane), un.count - 1);
      const size_t row = un.bank ? static_cast<size_t>(p.P) + un.start + m
                                 : static_cast<size_t>(un.start) + m;
      brow[0][f] = p.hhi + row * p.Imax + (lane >> 4) * 16;
      if constexpr (!H16) brow[NB - 1][f] = p.hlo + row * p.Imax + (lane >> 4) * 16;
      if (un.bank) {
        ot[f] = un.start + m;
        oslot[f] = p.k;
        owt[f] = p.gamma[ot[f]];
      } else {
        ot[f] = pr[f] / p.k;
        oslot[f] = pr[f] - ot[f] * p.k;
        owt[f] = p.w[pr[f]];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (nit < nitems) load_item(nun, ntile);

    uint4 xr[R][NB][FR][2];
    auto load_b = [&](int s, uint4 (&dst)[NB][FR][2]) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int f = 0; f < FR; ++f) {
          dst[b][f][0] = ld16(brow[b][f] + s * kPfSlab);
          dst[b][f][1] = ld16(brow[b][f] + s * kPfSlab + 8);
        }
    };
#pragma unroll
    for (int r = 0; r < R - 1; ++r) load_b(r, xr[r]);
    __syncthreads();  // the tile is in LDS

    f32x4 acc[FR][8];
#pragma unroll
    for (int f = 0; f < FR; ++f)
#pragma unroll
      for (int r = 0; r < 8; ++r) acc[f][r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s + R - 1 < NS) load_b(s + R - 1, xr[(s + R - 1) % R]);
      const uint4* t = lds[s];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint4 a[8];
#pragma unroll
        for (int rf = 0; rf < 8; ++rf)
          a[rf] = t[(rf * 16 + (lane & 15)) * kLdsRowU4 + (lane >> 4) * 2 + j];
        // (pair) h_hi products first, then h_lo: consecutive MFMAs write different
        // accumulators (an MFMA right after one into the same accumulator waits)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int f = 0; f < FR; ++f) {
            if (f < nfr) {
#pragma unroll
              for (int rf = 0; rf < 8; ++rf)
                acc[f][rf] = mfma16<H16>(a[rf], xr[s % R][b][f][j], acc[f][rf]);
            }
          }
      }
    }

    // epilogue: output rows h0 + 16 r + 4 (lane / 16) + jj of token m
    const float gd = bank.gsc[un.expert * 3 + 2];
#pragma unroll
    for (int f = 0; f < FR; ++f) {
      const int m = frag_token<W>(wave, f, lane);
      if (f >= nfr || m >= un.count) continue;
      float* dst = p.out + (static_cast<size_t>(ot[f]) * p.nslots + oslot[f]) * H + h0 +
                   (lane >> 4) * 4;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        float4 v;
        v.x = (acc[f][r][0] * gd) * owt[f];
        v.y = (acc[f][r][1] * gd) * owt[f];
        v.z = (acc[f][r][2] * gd) * owt[f];
        v.w = (acc[f][r][3] * gd) * owt[f];
        *reinterpret_cast<float4*>(dst + r * 16) = v;
      }
    }
    if (nit >= nitems) break;
    it = nit;
    u = nu;
    tile = ntile;
    un = nun;
  }
}

__global__ __launch_bounds__(256) void pf_combine_kernel(PrefillParams p) {
  const int H4 = p.H / 4;
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<size_t>(p.T) * H4) return;
  const int t = static_cast<int>(i / H4);
  const int c = static_cast<int>(i - static_cast<size_t>(t) * H4) * 4;
  // Every id and every slot row is loaded before any is used (indices clamped to
  // the token's own entries), then the slots are summed in slot order: a runtime
  // loop would wait for each load in turn, one memory round trip per slot.
  constexpr int kMaxSlots = kTopkMaxK + 1;
  const int32_t* idr = p.ids + static_cast<size_t>(t) * p.k;
  int ev[kTopkMaxK];
#pragma unroll
  for (int s = 0; s < kTopkMaxK; ++s) ev[s] = idr[s < p.k ? s : p.k - 1];
  const float* src = p.out + static_cast<size_t>(t) * p.nslots * p.H + c;
  float4 v[kMaxSlots];
#pragma unroll
  for (int s = 0; s < kMaxSlots; ++s)
    {
      typedef float nt_f4 __attribute__((ext_vector_type(4)));
      const nt_f4 t = __builtin_nontemporal_load(reinterpret_cast<const nt_f4*>(src + static_cast<size_t>(s < p.nslots ? s : p.nslots - 1) * p.H));
      v[s] = make_float4(t.x, t.y, t.z, t.w);
    }
  // nothing that uses a loaded value is scheduled between the loads (it would wait
  // for the earlier loads before the later ones are issued)
  __builtin_amdgcn_sched_barrier(0);
  bool bad = false;
#pragma unroll
  for (int s = 0; s < kTopkMaxK; ++s) bad |= (ev[s] < 0 || ev[s] >= p.E);
  // Every slot is added, a missing one (s >= nslots) masked to +0.0: the sum starts
  // from +0.0 and so is never -0.0, and adding +0.0 leaves it unchanged.  The masks
  // are hidden from the optimiser: a select there becomes a branch that the slot's
  // load is deferred into, behind a wait for every earlier load.
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int s = 0; s < kMaxSlots; ++s) {
    uint32_t keep = s < p.nslots ? 0xFFFFFFFFu : 0u;
    __asm__ volatile("" : "+v"(keep));
    acc.x += __uint_as_float(__float_as_uint(v[s].x) & keep);
    acc.y += __uint_as_float(__float_as_uint(v[s].y) & keep);
    acc.z += __uint_as_float(__float_as_uint(v[s].z) & keep);
    acc.w += __uint_as_float(__float_as_uint(v[s].w) & keep);
  }
  if (bad) acc = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                             __builtin_nanf(""));
  const uint32_t lo = f32_to_bf16_bits(acc.x) | (static_cast<uint32_t>(f32_to_bf16_bits(acc.y)) << 16);
  const uint32_t hi = f32_to_bf16_bits(acc.z) | (static_cast<uint32_t>(f32_to_bf16_bits(acc.w)) << 16);
  *reinterpret_cast<uint2*>(p.y + static_cast<size_t>(t) * p.H + c) = make_uint2(lo, hi);
}

// ------------------------------------------------------------ launchers --


hipError_t launch_prefill(const PrefillParams& p0, hipStream_t s) {
  PrefillParams p = p0;
  const int nblk = prefill_group_blocks(p.T, p.k);
  const int maxu = prefill_max_units(p.E, p.T, p.k, p.shared.inter > 0);
  const int ugroups = (maxu + 7) / 8;
  p.unit_tokens = prefill_unit_tokens(p.T);
  p.ntiles1 = p.Imax / 64;
  p.ntiles2 = p.H / kPfRows;
  if (p.routes_grouped) {
    // units, nunits and sorted were written by the routing kernel
  } else if (p.P <= kGroupOneBlockPairs) {
    pf_group_one_block_kernel<<<1, kMaxExperts, 0, s>>>(p);
  } else {
    pf_hist_kernel<<<nblk, 256, 0, s>>>(p);
    pf_scan_kernel<<<1, kMaxExperts, 0, s>>>(p);
    pf_scatter_kernel<<<(p.P + kScatterPairs - 1) / kScatterPairs, 256, 0, s>>>(p);
  }
  const unsigned g1 = ugroups * 8 * p.ntiles1, g2 = ugroups * 8 * p.ntiles2;
  if (p.unit_tokens == kPfUnitTokens) {
    static_assert(Geometry<4, 4>::kUnitTokens == kPfUnitTokens, "unit size");
    static_assert(Geometry<8, 2>::kUnitTokens == kPfUnitTokens, "unit size");
    switch (p.H) {
      case 1024: pf_gateup_kernel<4, 4, 2, 1, 4><<<g1, 4 * kWave, 0, s>>>(p); break;
      case 2048: pf_gateup_kernel<4, 4, 2, 1, 8><<<g1, 4 * kWave, 0, s>>>(p); break;
      case 4096: pf_gateup_kernel<4, 4, 2, 1, 16><<<g1, 4 * kWave, 0, s>>>(p); break;
      default: pf_gateup_kernel<4, 2, 1, 1, 0><<<g1, 4 * kWave, 0, s>>>(p); break;
    }
    const unsigned gp = g2 < kPersistentBlocks ? g2 : kPersistentBlocks;
    if (p.routed.inter == 512 && (p.shared.inter == 0 || p.shared.inter == 512)) {
      if (p.h16) pf_down_persistent_kernel<8, 2, true><<<gp, 8 * kWave, 0, s>>>(p, static_cast<int>(g2));
      else pf_down_persistent_kernel<8, 2, false><<<gp, 8 * kWave, 0, s>>>(p, static_cast<int>(g2));
    } else {
      if (p.h16) pf_down_kernel<8, 2, 2, 4, 0, true><<<g2, 8 * kWave, 0, s>>>(p);
      else pf_down_kernel<8, 2, 2, 4, 0, false><<<g2, 8 * kWave, 0, s>>>(p);
    }
  } else {
    // few tokens per expert: units of at most 16 tokens, each a separate pass over
    // its expert's weights (the passes of one expert run side by side)
    hipError_t e = launch_grouped_small(p, ugroups, s);
    if (e != hipSuccess) return e;
  }
  const size_t n4 = static_cast<size_t>(p.T) * (p.H / 4);
  // small calls in 64-thread blocks, so that their slot rows are read by every CU
  const unsigned cb = n4 < static_cast<size_t>(256) * 256 ? 64u : 256u;
  pf_combine_kernel<<<static_cast<unsigned>((n4 + cb - 1) / cb), cb, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace ftmoe
