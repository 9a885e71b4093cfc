// ftmoe_kernels.hpp -- internal interface between the C ABI layer (abi.cpp) and
// the gfx950 kernels: parameter blocks and launchers.  Nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

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
  uint32_t* zero;               // counters of later kernels of the same call, cleared here
  int nzero;
};

// Gate|up GEMV with in-register dequantisation and (clamped) SwiGLU.
struct GateUpParams {
  const uint16_t* x;  // bf16 [T][H]
  int T, H, k;
  int E;              // routed experts: an id outside [0, E) yields NaN, never a load
  Bank routed, shared;
  const int32_t* ids; // i32 [T][k]
  float* h;           // f32 [T][k+1][Imax]
  int Imax;
  int act;
  float gate_max, up_absmax;
};

// Down GEMV, weighted combine over the selected experts and the shared expert.
struct DownParams {
  int T, H, k, nslots;  // nslots = k (+1 with a shared expert)
  int E;                // routed experts: an id outside [0, E) yields NaN, never a load
  Bank routed, shared;
  const int32_t* ids;   // i32 [T][k]
  const float* w;       // f32 [T][k]
  const float* gamma;   // f32 [T] or null
  const float* h;       // f32 [T][k+1][Imax]
  int Imax;
  float* part;          // f32 [T][H/64][nslots][64] per-slot partial outputs
  uint32_t* cnt;        // u32 [T][H/64] last-arriver counters
  uint16_t* y;          // bf16 [T][H]
};

// The whole decode layer in one persistent launch (one block per CU).  Values
// handed from one block to another are "tagged": an 8-byte word holding the fp32
// value in its low half and the call's generation number in its high half,
// written and read with single 8-byte device-coherent accesses.
constexpr int kLogitCopies = 16;    // replicas of the router logits (spreads the reads)
constexpr int kMaxFusedGrid = 1024;

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
  uint32_t* err;                // set when a poll gives up (the result is then invalid)
  int d_groups;                 // T * H / 64 (token, row group) pairs of the down GEMV
  int blocks_per_group;         // blocks sharing one group when d_groups < grid
  int spin_limit;               // polls of one value before giving up
};

// Launchers: return the launch status (hipGetLastError after the launch).
hipError_t launch_decode_fused(const FusedParams& p, int grid, hipStream_t s);
int fused_block_threads();
hipError_t launch_route(const RouteParams& p, bool fuse_topk, hipStream_t s);
hipError_t launch_topk(const RouteParams& p, hipStream_t s);
hipError_t launch_gateup(const GateUpParams& p, hipStream_t s);
void gateup_geometry(int H, int* lpr, int* cpl);  // supported when lpr > 0 and 1 <= cpl <= 4
hipError_t launch_down(const DownParams& p, hipStream_t s);
hipError_t launch_repack_w2(int H, int I, int n, const uint8_t* w2, const uint8_t* w2s,
                            uint8_t* out_w2, uint8_t* out_w2s, hipStream_t s);
hipError_t launch_dequant(int H, int I, const Bank& b, int expert, int tensor, int out_dtype,
                          void* out, hipStream_t s);

}  // namespace ftmoe
