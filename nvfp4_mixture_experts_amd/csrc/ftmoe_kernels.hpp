// ftmoe_kernels.hpp -- internal interface between the C ABI layer (abi.cpp) and
// the gfx950 kernels: parameter blocks and launchers.  Nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "host_layout.hpp"

namespace ftmoe {

// One repacked NVFP4 expert bank (see ft_nvfp4_repack for the layout).
struct Bank {
  const uint8_t* w13;   // [n][2I][H/2] row-major codes
  const uint8_t* w13s;  // [n][2I][H/16] row-major e4m3 scales
  const uint8_t* w2;    // [n][I/32][H][16] K-chunk-major codes
  const uint8_t* w2s;   // [n][I/32][H][2] K-chunk-major e4m3 scales
  const float* gsc;     // [n][3] gate, up, down global scales
  int inter;            // I of this bank (0 = no bank)
};

// Router: logits, the shared expert's gate, and top-k with softmax weights.
struct RouteParams {
  const uint16_t* x;            // bf16 [T][H]
  const float* wr;              // f32 [E][H]
  const float* bias;            // f32 [E] or null
  const uint16_t* shared_gate;  // bf16 [H] or null
  int T, E, H, k;
  float* logits;                // f32 [T][E]
  float* gamma;                 // f32 [T] (sigmoid of the shared gate) or null
  int32_t* ids;                 // i32 [T][k]
  float* w;                     // f32 [T][k]
  int32_t* ids_copy;            // optional second copy of ids (caller's side output)
  float* w_copy;                // optional second copy of w
  uint32_t* counter;            // last-arriver counter for the fused top-k
  int tok_tile;                 // tokens per wave (set by the launcher)
  double* part;                 // split-K router: f64 [ksplit][T][E + 1] partial sums
  int ksplit;                   // K splits (set by the launcher)
  uint16_t* wsplit;             // many-token router: bf16 [E][2][H] pieces of each row
  float* wnorm;                 // many-token router: f32 [E] 2-norm of each row, rounded up
};

// The whole decode layer in one persistent launch (one block per CU).  Values
// handed from one block to another are "tagged": an 8-byte word holding the fp32
// value in its low half and the call's generation number in its high half,
// written and read with single 8-byte device-coherent accesses.

struct FusedParams {
  const uint16_t* x;            // bf16 [T][H]
  const float* wr;              // f32 [E][H]
  const float* bias;            // f32 [E] or null
  const uint16_t* shared_gate;  // bf16 [H] or null
  int T, E, H, k, act;
  float gate_max, up_absmax;
  Bank routed, shared;          // shared.inter == 0: no shared expert
  int nslots, Imax;
  uint16_t* y;                  // bf16 [T][H]
  int32_t* ids_out;             // optional i32 [T][k]
  float* w_out;                 // optional f32 [T][k]
  uint64_t* logits;             // tagged [kLogitCopies][T][E + 1] (column E: shared gate)
  uint64_t* h;                  // tagged [T][nslots][Imax]
  uint64_t* part;               // tagged [d_groups][blocks_per_group][64]
  uint32_t* gen;                // per-block call counters [grid]
  uint32_t* err;                // [0] reasons of give-ups (the result is then invalid),
                                // [1] generation of the latest call that gave up
  int d_groups;                 // T * H / 64 (token, row group) pairs of the down GEMV
  int blocks_per_group;         // blocks sharing one group when d_groups < grid
  int spin_limit;               // polls of one value before giving up
  const int32_t* slot_of;       // optional [E] expert -> slot of `routed` (null: identity)
  int n_slots;                  // slots of `routed` when slot_of is set
  int32_t* miss_out;            // optional [T][k]: id of a non-resident selected expert, or -1
  int fp8;                      // 1: both banks are block-fp8 (w13s / w2s point at fp32 block
                                // scales, gsc unused), 0: NVFP4
};


// The routing of a decode batch in one launch (route_group.hip).
struct RouteGroupParams {
  const uint16_t* x;            // bf16 [T][H]
  const float* wr;              // f32 [E][H]
  const float* bias;            // f32 [E] or null
  const uint16_t* shared_gate;  // bf16 [H] or null
  int T, E, H, k;
  int ksplit;                   // K splits of the router product (route_group_splits)
  int32_t* ids;                 // i32 [T][k] expert ids (slot ids over a slot bank)
  float* w;                     // f32 [T][k] routing weights (0 for a non-resident expert)
  float* gamma;                 // f32 [T] shared gate, or null
  int32_t* ids_copy;            // optional i32 [T][k]: the expert ids
  float* w_copy;                // optional f32 [T][k]: the softmax weights
  const int32_t* slot_of;       // optional [E] expert -> slot
  int n_slots;
  int32_t* miss_out;            // optional [T][k]: non-resident selected expert, or -1
  int group;                    // 1: also group the pairs (units, nunits, sorted)
  int n_group;                  // experts (or slots) of the grouping, <= kMaxExperts
  int unit_tokens;              // tokens per work unit
  int shared_units;             // 1: append the shared expert's units
  PfUnit* units;
  int32_t* nunits;
  int32_t* sorted;
  uint64_t* part;               // tagged [ksplit][E / 16 tiles][16][T][2]: partial sums (low, high)
  uint64_t* lg;                 // tagged [T][E]: fp32 logits (bias added)
  uint64_t* tids;               // tagged [T * k]: the ids, for the grouping block
  uint32_t* gen;                // per-block call counters [grid] (shared with the decode kernel)
  uint32_t* err;                // error word (as FusedParams::err)
  int spin_limit;
};

struct PrefillParams {
  const uint16_t* x;       // bf16 [T][H]
  int T, H, k, E, P;       // P = T * k routed pairs; pair = t * k + slot
  Bank routed, shared;
  const int32_t* ids;      // i32 [T][k]
  const float* w;          // f32 [T][k]
  const float* gamma;      // f32 [T] shared-expert gate, or null
  int32_t* count;          // i32 [E] pairs per expert (zero between calls)
  int32_t* cursor;         // i32 [E] fill positions of the groups
  int32_t* offset;         // i32 [E] first sorted position of each expert
  int32_t* sorted;         // i32 [P] pairs grouped by expert (in no particular order within one)
  PfUnit* units;           // [max units]
  int32_t* nunits;         // number of valid units
  int Imax;                // row stride of hhi / hlo
  int h16;                 // 1: h travels as fp16 in hhi (hlo unused); 0: as a bf16 pair
  int routes_grouped;      // 1: units, nunits and sorted are already written (by the routing
                           // kernel of a decode batch): the grouping kernels are skipped
  uint16_t* hhi;           // [P + T][Imax] h in fp16 (h16), or h rounded to bf16 ...
  uint16_t* hlo;           // bf16 [P + T][Imax] ... and the rounded remainder (h16 = 0)
  float* out;              // f32 [T][nslots][H] weighted expert outputs
  int nslots;              // k (+1 with a shared expert)
  int act;
  float gate_max, up_absmax;
  int ntiles1, ntiles2;    // column tiles per unit of the two GEMMs (set by the launcher)
  int unit_tokens;         // tokens per work unit (set by the launcher)
  uint16_t* y;             // bf16 [T][H]
};

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s);
// expert GEMMs of the grouped path for few tokens (after grouping, before combine)
hipError_t launch_grouped_small(const PrefillParams& p, int ugroups, hipStream_t s);

// Launchers: return the launch status (hipGetLastError after the launch).
hipError_t launch_decode_fused(const FusedParams& p, int grid, hipStream_t s);
int fused_block_threads();
hipError_t decode_fused_min_occupancy(int* blocks_per_cu);
hipError_t launch_route_group(const RouteGroupParams& p, int grid, hipStream_t s);
hipError_t route_group_min_occupancy(int* blocks_per_cu);
// copies the error word err[0] of a decode workspace to *status and clears it
hipError_t launch_device_status(uint32_t* err, int32_t* status, hipStream_t s);
// Rewrites routes [T*k] in place from expert ids to slot ids (a non-resident expert:
// slot 0 and weight 0) and writes the miss list (expert id or -1) when given.
hipError_t launch_map_slots(int32_t* ids, float* w, int pairs, const int32_t* slot_of,
                            int n_slots, int32_t* miss_out, hipStream_t s);
hipError_t launch_route(const RouteParams& p, bool fuse_topk, hipStream_t s);
int route_fused_topk_tokens();  // the fused top-k handles at most this many tokens
hipError_t launch_route_split(const RouteParams& p, hipStream_t s);
hipError_t launch_topk(const RouteParams& p, hipStream_t s);
// logits only (no shared gate, no top-k), as an fp64 MFMA product; H % 64 == 0
hipError_t launch_route_mfma(const RouteParams& p, hipStream_t s);
// many tokens: approximate logits by a bf16 MFMA product with a rigorous error bound,
// then per token the exact fp64 logits of the experts the bound cannot rule out and
// the top-k among them (ids, w and their copies); p.wsplit / p.wnorm are scratch
hipError_t launch_route_bounded(const RouteParams& p, hipStream_t s);
hipError_t launch_repack_w2(int H, int I, int n, const uint8_t* w2, const uint8_t* w2s,
                            uint8_t* out_w2, uint8_t* out_w2s, hipStream_t s);
hipError_t launch_dequant(int H, int I, const Bank& b, int expert, int tensor, int out_dtype,
                          void* out, hipStream_t s);
// per-tensor FP8 W8A8 linear: workspace bytes (codes, amax partials, scale), the
// activation quantisation (sets *xq and *s_x to their places in ws) and the GEMM
// (row_scale [N] when set, else `scale` for every row; y columns col0.. of stride ldy)
// Quantisation and GEMV in one launch for few, short activation rows (row-wise scales).
bool fp8_linear_fused_fits(int64_t M, int64_t K);
hipError_t launch_fp8_linear_fused(const uint16_t* x, const uint8_t* w, int M, int N, int K,
                                   const float* row_scale, uint16_t* y, int ldy, int col0,
                                   hipStream_t s);
size_t fp8_linear_workspace(int64_t M, int64_t K);
hipError_t launch_fp8_quantize(const uint16_t* x, int64_t M, int64_t K, void* ws, uint8_t** xq,
                               float** s_x, hipStream_t s);
hipError_t launch_fp8_gemm(const uint8_t* xq, const uint8_t* w, int M, int N, int K,
                           const float* s_x, const float* row_scale, float scale, uint16_t* y,
                           int ldy, int col0, hipStream_t s);
// extend attention over a KV-cache prefix (format 0 bf16, 1 e4m3, 2 NVFP4) and the
// new tokens (bf16), causal, optional window
struct AttnParams {
  int n_new, prefix, Hq, Hkv, D, window, format;
  const uint16_t* q;        // [n_new][Hq][D]
  const uint16_t* k_new;    // [n_new][Hkv][D]
  const uint16_t* v_new;
  const void* k_cache;      // [prefix][Hkv][D] bf16 / e4m3, or [prefix][Hkv][D/2] e2m1
  const void* v_cache;
  const uint8_t* k_bscale;  // NVFP4: e4m3 [prefix][Hkv][D/16]
  const uint8_t* v_bscale;
  float k_scale, v_scale;   // fp8 / NVFP4 tensor scales (on the dot outputs)
  float sm_scale;           // 1 / sqrt(D)
  uint16_t* out;            // [n_new][Hq][D]
};
hipError_t launch_attn_extend(const AttnParams& p, hipStream_t s);
// block-fp8 banks (Bank.w13s / w2s hold fp32 block scales; gsc unused)
hipError_t launch_repack_fp8_w2(int H, int I, int n, const uint8_t* w2, uint8_t* out_w2,
                                hipStream_t s);
hipError_t launch_fp8_dequant(int H, int I, const Bank& b, int expert, int tensor, int mode,
                              float* out, hipStream_t s);

}  // namespace ftmoe
