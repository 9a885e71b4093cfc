// abi.cpp -- the exported C ABI of libftmoe.so (declared in include/ftmoe.h):
// argument validation, workspace layout and kernel dispatch.  Everything here
// runs on the host; compute calls only enqueue kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <cfloat>
#include <cmath>

#include "abi_internal.hpp"
#include "ftmoe.h"
#include "ftmoe_kernels.hpp"

using namespace ftmoe;

namespace {

thread_local char g_err[512] = "";

ft_status fail(ft_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

ft_status ok() {
  g_err[0] = '\0';
  return FT_OK;
}

ft_status hip_fail(hipError_t e, const char* what) {
  return fail(FT_EHIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxDevices = 64;
constexpr int kSpinLimit = 1 << 20;  // polls of one value (~1 s) before the kernel gives up

// Polls of one value before a wait of the fused decode kernel gives up; 0 = kSpinLimit.
// Set only through ft_set_wait_limit (a test and diagnostic hook).
std::atomic<int> g_wait_limit{0};

int wait_limit() {
  const int v = g_wait_limit.load(std::memory_order_relaxed);
  return v > 0 ? v : kSpinLimit;
}

// Per-device launch geometry of the fused decode kernel (one block per CU), set
// once the device is known to keep one block of every instantiation resident per
// CU (the kernel's blocks wait for each other, so all of them must run at once).
int g_fused_grid[kMaxDevices] = {0};

ft_status fused_grid(int* grid) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(FT_EUNSUPPORTED, "device index %d", dev);
  if (g_fused_grid[dev] == 0) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    if (cus <= 0) return fail(FT_EHIP, "device reports %d compute units", cus);
    int per_cu = 0;
    e = decode_fused_min_occupancy(&per_cu);
    if (e != hipSuccess) return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
    if (per_cu < 1)
      return fail(FT_EUNSUPPORTED,
                  "the fused decode kernel cannot keep a block resident on a compute unit");
    e = route_group_min_occupancy(&per_cu);
    if (e != hipSuccess) return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
    if (per_cu < 1)
      return fail(FT_EUNSUPPORTED,
                  "the decode routing kernel cannot keep a block resident on a compute unit");
    g_fused_grid[dev] = cus < kMaxFusedGrid ? cus : kMaxFusedGrid;
  }
  *grid = g_fused_grid[dev];
  return FT_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }



ft_status check_desc(const ft_moe_desc* d) {
  char msg[160];
  const ft_status st = desc_problem(d, msg, sizeof msg);
  return st == FT_OK ? FT_OK : fail(st, "%s", msg);
}

ft_status check_bank(const ft_nvfp4_experts* b, const char* name) {
  if (!b) return fail(FT_EINVAL, "%s bank is NULL", name);
  if (!b->w13 || !b->w13_scale || !b->w2 || !b->w2_scale || !b->global_scale)
    return fail(FT_EINVAL, "%s bank has a NULL pointer", name);
  if (!aligned16(b->w13) || !aligned16(b->w13_scale) || !aligned16(b->w2) ||
      !aligned16(b->w2_scale) || !aligned16(b->global_scale))
    return fail(FT_EINVAL, "%s bank pointers must be 16-byte aligned", name);
  return FT_OK;
}

Bank to_bank(const ft_nvfp4_experts* b, int inter) {
  Bank r{};
  if (b) {
    r.w13 = b->w13;
    r.w13s = b->w13_scale;
    r.w2 = b->w2;
    r.w2s = b->w2_scale;
    r.gsc = b->global_scale;
    r.inter = inter;
  }
  return r;
}


ft_status check_ws(const ft_moe_desc* d, int64_t T, int path, void* ws, size_t ws_bytes,
                          Layout* L) {
  *L = layout(*d, T, path);
  if (!ws) return fail(FT_EWORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) & 255u)
    return fail(FT_EWORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < L->total)
    return fail(FT_EWORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, L->total);
  return FT_OK;
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

ft_status check_layer_args(const ft_moe_desc* desc, const uint16_t* x,
                                  const ft_nvfp4_experts* routed, const ft_nvfp4_experts* shared,
                                  const uint16_t* shared_gate, const uint16_t* y) {
  ft_status st;
  if (!x || !y) return fail(FT_EINVAL, "x or y is NULL");
  if (!aligned16(x)) return fail(FT_EINVAL, "x must be 16-byte aligned");
  if (!aligned16(y)) return fail(FT_EINVAL, "y must be 16-byte aligned");
  if ((st = check_bank(routed, "routed")) != FT_OK) return st;
  if (desc->shared_inter > 0) {
    if ((st = check_bank(shared, "shared")) != FT_OK) return st;
    if (!shared_gate) return fail(FT_EINVAL, "shared_gate is NULL with a shared expert");
    if (!aligned16(shared_gate)) return fail(FT_EINVAL, "shared_gate must be 16-byte aligned");
  }
  return FT_OK;
}

ft_status check_fp8_bank(const ft_fp8_experts* b, const char* name) {
  if (!b) return fail(FT_EINVAL, "%s fp8 bank is NULL", name);
  if (!b->w13 || !b->w13_scale || !b->w2 || !b->w2_scale)
    return fail(FT_EINVAL, "%s fp8 bank has a NULL pointer", name);
  if (!aligned16(b->w13) || !aligned16(b->w13_scale) || !aligned16(b->w2) ||
      !aligned16(b->w2_scale))
    return fail(FT_EINVAL, "%s fp8 bank pointers must be 16-byte aligned", name);
  return FT_OK;
}

Bank to_bank_fp8(const ft_fp8_experts* b, int inter) {
  Bank r{};
  if (b) {
    r.w13 = b->w13;
    r.w13s = reinterpret_cast<const uint8_t*>(b->w13_scale);
    r.w2 = b->w2;
    r.w2s = reinterpret_cast<const uint8_t*>(b->w2_scale);
    r.gsc = nullptr;
    r.inter = inter;
  }
  return r;
}

// Router logits (fp64, one fp32 rounding), the shared gate when `gamma` is set,
// and top-k with softmax weights into ids / w (and the optional copies).
ft_status run_route(const ft_moe_desc* desc, int T, const uint16_t* x, const float* w_router,
                    const float* bias, const uint16_t* shared_gate, float* logits, float* gamma,
                    int32_t* ids, float* w, int32_t* ids_copy, float* w_copy, uint32_t* counter,
                    double* split_part, uint16_t* wsplit, float* wnorm, hipStream_t s) {
  RouteParams p{};
  p.x = x;
  p.wr = w_router;
  p.bias = bias;
  p.shared_gate = gamma ? shared_gate : nullptr;
  p.T = T;
  p.E = desc->num_experts;
  p.H = desc->hidden;
  p.k = desc->top_k;
  p.logits = logits;
  p.gamma = gamma;
  p.ids = ids;
  p.w = w;
  p.ids_copy = ids_copy;
  p.w_copy = w_copy;
  p.counter = counter;
  hipError_t e;
  if (T >= kRouteMfmaMinTokens) {
    // many tokens: bf16 MFMA approximations with a rigorous error bound, the exact
    // fp64 logits of the experts the bound leaves in play and the top-k among them
    // (with the row pieces and norms in the workspace); the shared gate by the row
    // kernel (as its only row).  Without that scratch (callers other than
    // ft_moe_route): the fp64 MFMA product of every logit, then the top-k kernel.
    if (wsplit && wnorm) {
      p.wsplit = wsplit;
      p.wnorm = wnorm;
      e = launch_route_bounded(p, s);
      if (e != hipSuccess) return hip_fail(e, "bounded router kernels");
    } else {
      e = launch_route_mfma(p, s);
      if (e != hipSuccess) return hip_fail(e, "route kernel");
    }
    if (gamma) {
      RouteParams q = p;
      q.E = 0;
      e = launch_route(q, false, s);
      if (e != hipSuccess) return hip_fail(e, "shared gate kernel");
    }
    if (!(wsplit && wnorm)) {
      e = launch_topk(p, s);
      if (e != hipSuccess) return hip_fail(e, "top-k kernel");
    }
    return FT_OK;
  }
  if (T >= kRouteSplitMinTokens) {
    // split-K fp64 MFMA partial sums, then a block per token sums them (in split
    // order), rounds once to fp32 and selects
    p.part = split_part;
    e = launch_route_split(p, s);
    if (e != hipSuccess) return hip_fail(e, "split router kernels");
    return FT_OK;
  }
  // the last block to finish selects the experts when it has a wave per token;
  // otherwise a top-k kernel follows (a block per token up to 256 tokens, else a
  // wave per token)
  const bool fuse = T <= route_fused_topk_tokens();
  e = launch_route(p, fuse, s);
  if (e != hipSuccess) return hip_fail(e, "route kernel");
  if (!fuse) {
    e = launch_topk(p, s);
    if (e != hipSuccess) return hip_fail(e, "top-k kernel");
  }
  return FT_OK;
}

// Grouped experts: pairs grouped by expert, gate|up and down grouped GEMMs, combine.
// gamma (the shared gate) must already be in the workspace when there is a shared expert.
ft_status run_grouped(const ft_moe_desc* desc, int T, const uint16_t* x, const int32_t* ids,
                      const float* w, const ft_nvfp4_experts* routed,
                      const ft_nvfp4_experts* shared, uint16_t* y, void* workspace,
                      const Layout& L, hipStream_t s, bool routes_grouped = false) {
  const bool has_shared = desc->shared_inter > 0;
  PrefillParams p{};
  p.x = x;
  p.T = T;
  p.H = desc->hidden;
  p.k = desc->top_k;
  p.E = desc->num_experts;
  p.P = T * desc->top_k;
  p.routed = to_bank(routed, desc->inter);
  p.shared = has_shared ? to_bank(shared, desc->shared_inter) : Bank{};
  p.ids = ids;
  p.w = w;
  p.gamma = has_shared ? at<float>(workspace, L.gamma) : nullptr;
  p.count = at<int32_t>(workspace, L.count);
  p.cursor = at<int32_t>(workspace, L.cursor);
  p.offset = at<int32_t>(workspace, L.offset);
  p.sorted = at<int32_t>(workspace, L.sorted);
  p.units = at<PfUnit>(workspace, L.units);
  p.nunits = at<int32_t>(workspace, L.nunits);
  p.Imax = desc->inter > desc->shared_inter ? desc->inter : desc->shared_inter;
  p.hhi = at<uint16_t>(workspace, L.hhi);
  p.hlo = at<uint16_t>(workspace, L.hlo);
  p.out = at<float>(workspace, L.out);
  p.nslots = desc->top_k + (has_shared ? 1 : 0);
  p.act = desc->act;
  p.gate_max = desc->gate_max;
  p.up_absmax = desc->up_absmax;
  p.h16 = prefill_h16(desc->act, desc->gate_max, desc->up_absmax) ? 1 : 0;
  p.routes_grouped = routes_grouped ? 1 : 0;
  p.y = y;
  hipError_t e = launch_prefill(p, s);
  if (e != hipSuccess) return hip_fail(e, "grouped expert kernels");
  return FT_OK;
}

}  // namespace

namespace ftmoe {
ft_status abi_fail(ft_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}
ft_status abi_hip_fail(hipError_t e, const char* what) { return hip_fail(e, what); }
}  // namespace ftmoe

extern "C" {

int32_t ft_abi_version(void) { return FT_ABI_VERSION; }

const char* ft_last_error(void) { return g_err; }

ft_status ft_init(int32_t device) {
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
  if (device < 0 || device >= n) return fail(FT_EINVAL, "device %d out of range [0, %d)", device, n);
  e = hipSetDevice(device);
  if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(FT_EUNSUPPORTED, "device %d is %s; this library is built for gfx950", device,
                prop.gcnArchName);
  int grid = 0;
  ft_status st = fused_grid(&grid);
  if (st != FT_OK) return st;
  st = scratch_setup(device);
  if (st != FT_OK) return st;
  return ok();
}

size_t ft_nvfp4_repacked_bytes(int32_t hidden, int32_t inter, int32_t n_experts, int32_t part) {
  if (hidden <= 0 || inter <= 0 || n_experts <= 0 || hidden % 32 || inter % 32) return 0;
  const size_t n = static_cast<size_t>(n_experts), H = static_cast<size_t>(hidden),
               I = static_cast<size_t>(inter);
  switch (part) {
    case 0: return n * 2 * I * H / 2;
    case 1: return n * 2 * I * H / 16;
    case 2: return n * H * I / 2;
    case 3: return n * H * I / 16;
    default: return 0;
  }
}

ft_status ft_nvfp4_repack(int32_t hidden, int32_t inter, int32_t n_experts, const uint8_t* w13,
                          const uint8_t* w13_scale, const uint8_t* w2, const uint8_t* w2_scale,
                          uint8_t* out_w13, uint8_t* out_w13_scale, uint8_t* out_w2,
                          uint8_t* out_w2_scale, void* stream) {
  if (hidden <= 0 || inter <= 0 || n_experts <= 0)
    return fail(FT_EINVAL, "repack: non-positive size");
  if (hidden % 256 || !inter_ok(inter))
    return fail(FT_EUNSUPPORTED, "repack: hidden %d / inter %d unsupported", hidden, inter);
  const void* ptrs[8] = {w13, w13_scale, w2, w2_scale, out_w13, out_w13_scale, out_w2, out_w2_scale};
  for (const void* p : ptrs) {
    if (!p) return fail(FT_EINVAL, "repack: NULL pointer");
    if (!aligned16(p)) return fail(FT_EINVAL, "repack: pointers must be 16-byte aligned");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(out_w13, w13, ft_nvfp4_repacked_bytes(hidden, inter, n_experts, 0),
                                hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "repack w13");
  e = hipMemcpyAsync(out_w13_scale, w13_scale, ft_nvfp4_repacked_bytes(hidden, inter, n_experts, 1),
                     hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "repack w13 scales");
  e = launch_repack_w2(hidden, inter, n_experts, w2, w2_scale, out_w2, out_w2_scale, s);
  if (e != hipSuccess) return hip_fail(e, "repack w2");
  return ok();
}

size_t ft_moe_workspace_bytes(const ft_moe_desc* desc, int64_t tokens, int32_t path) {
  if (check_desc(desc) != FT_OK || tokens < 0 || path < 0 || path > 2) return 0;
  return layout(*desc, tokens, path).total;
}

ft_status ft_moe_route(const ft_moe_desc* desc, int64_t tokens, const uint16_t* x,
                       const float* w_router, const float* bias, int32_t* topk_ids, float* topk_w,
                       void* workspace, size_t workspace_bytes, void* stream) {
  ft_status st = check_desc(desc);
  if (st != FT_OK) return st;
  if (tokens < 0) return fail(FT_EINVAL, "tokens < 0");
  // the router grids carry tokens / 64 in their y dimension (at most 65535)
  if (tokens > (1 << 21)) return fail(FT_EUNSUPPORTED, "route takes at most 2^21 tokens per call");
  if (!x || !w_router || !topk_ids || !topk_w) return fail(FT_EINVAL, "route: NULL pointer");
  if (!aligned16(x) || !aligned16(w_router))
    return fail(FT_EINVAL, "route: x and w_router must be 16-byte aligned");
  Layout L;
  if ((st = check_ws(desc, tokens, 0, workspace, workspace_bytes, &L)) != FT_OK) return st;
  if (tokens == 0) return ok();
  st = run_route(desc, static_cast<int>(tokens), x, w_router, bias, nullptr,
                 at<float>(workspace, L.logits), nullptr, topk_ids, topk_w, nullptr, nullptr,
                 at<uint32_t>(workspace, L.sync) + kRouteCounterWord,
                 at<double>(workspace, L.rsplit),
                 tokens >= kRouteMfmaMinTokens ? at<uint16_t>(workspace, L.wsplit) : nullptr,
                 tokens >= kRouteMfmaMinTokens ? at<float>(workspace, L.wnorm) : nullptr,
                 static_cast<hipStream_t>(stream));
  if (st != FT_OK) return st;
  return ok();
}

}  // extern "C"

namespace {

// The one-launch decode kernel (1..7 tokens) on banks already converted to Bank.
ft_status run_fused(const ft_moe_desc* desc, int T, const uint16_t* x, const float* w_router,
                    const float* bias, const Bank& routed, const Bank& shared,
                    const uint16_t* shared_gate, int32_t* topk_ids_out, float* topk_w_out,
                    uint16_t* y, void* workspace, const Layout& L, int grid,
                    const int32_t* slot_of, int32_t n_slots, int32_t* miss_out, int fp8,
                    hipStream_t s) {
  const bool has_shared = desc->shared_inter > 0;
  const int nrg = desc->hidden / kRowGroup;
  FusedParams p{};
  p.x = x;
  p.wr = w_router;
  p.bias = bias;
  p.shared_gate = has_shared ? shared_gate : nullptr;
  p.T = T;
  p.E = desc->num_experts;
  p.H = desc->hidden;
  p.k = desc->top_k;
  p.act = desc->act;
  p.gate_max = desc->gate_max;
  p.up_absmax = desc->up_absmax;
  p.routed = routed;
  p.shared = has_shared ? shared : Bank{};
  p.nslots = desc->top_k + (has_shared ? 1 : 0);
  p.Imax = desc->inter > desc->shared_inter ? desc->inter : desc->shared_inter;
  p.y = y;
  p.ids_out = topk_ids_out;
  p.w_out = topk_w_out;
  p.logits = at<uint64_t>(workspace, L.logits);
  p.h = at<uint64_t>(workspace, L.h);
  p.part = at<uint64_t>(workspace, L.part);
  p.gen = at<uint32_t>(workspace, L.gen);
  p.err = at<uint32_t>(workspace, L.sync) + kErrorWord;
  p.d_groups = T * nrg;
  const int upg = desc->top_k * (desc->inter / 32) + desc->shared_inter / 32;
  p.blocks_per_group = p.d_groups >= grid ? 1 : std::min(grid / p.d_groups, upg);
  p.spin_limit = wait_limit();
  p.slot_of = slot_of;
  p.n_slots = n_slots;
  p.miss_out = miss_out;
  p.fp8 = fp8;
  hipError_t e = launch_decode_fused(p, grid, s);
  if (e != hipSuccess) return hip_fail(e, "fused decode kernel");
  return ok();
}

// The decode call; with slot_of set, `routed` is a bank of n_slots expert slots.
ft_status decode_impl(const ft_moe_desc* desc, int64_t tokens, const uint16_t* x,
                      const float* w_router, const float* bias, const ft_nvfp4_experts* routed,
                      const int32_t* slot_of, int32_t n_slots, int32_t* miss_out,
                      const ft_nvfp4_experts* shared, const uint16_t* shared_gate,
                      int32_t* topk_ids_out, float* topk_w_out, uint16_t* y, void* workspace,
                      size_t workspace_bytes, void* stream) {
  ft_status st = check_desc(desc);
  if (st != FT_OK) return st;
  if (tokens < 1 || tokens > kMaxDecodeTokens)
    return fail(tokens < 1 ? FT_EINVAL : FT_EUNSUPPORTED, "decode takes 1..%d tokens, got %lld",
                kMaxDecodeTokens, static_cast<long long>(tokens));
  if (!w_router) return fail(FT_EINVAL, "w_router is NULL");
  if (!aligned16(w_router)) return fail(FT_EINVAL, "w_router must be 16-byte aligned");
  if ((st = check_layer_args(desc, x, routed, shared, shared_gate, y)) != FT_OK) return st;
  Layout L;
  if ((st = check_ws(desc, tokens, 1, workspace, workspace_bytes, &L)) != FT_OK) return st;
  int grid = 0;
  if ((st = fused_grid(&grid)) != FT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool has_shared = desc->shared_inter > 0;
  const int T = static_cast<int>(tokens);
  if (T >= kGroupedDecodeMinTokens) {
    int32_t* ids = at<int32_t>(workspace, L.ids);
    float* wts = at<float>(workspace, L.w);
    const int n_group = slot_of ? n_slots : desc->num_experts;
    if (route_group_fits(*desc, T, grid, n_group)) {
      // routing, selection and grouping in one launch (one block per CU)
      RouteGroupParams q{};
      q.x = x;
      q.wr = w_router;
      q.bias = bias;
      q.shared_gate = has_shared ? shared_gate : nullptr;
      q.T = T;
      q.E = desc->num_experts;
      q.H = desc->hidden;
      q.k = desc->top_k;
      q.ksplit = route_group_splits(desc->num_experts, desc->hidden, grid);
      q.ids = ids;
      q.w = wts;
      q.gamma = has_shared ? at<float>(workspace, L.gamma) : nullptr;
      q.ids_copy = topk_ids_out;
      q.w_copy = topk_w_out;
      q.slot_of = slot_of;
      q.n_slots = n_slots;
      q.miss_out = miss_out;
      q.group = 1;
      q.n_group = n_group;
      q.unit_tokens = prefill_unit_tokens(T);
      q.shared_units = has_shared ? 1 : 0;
      q.units = at<PfUnit>(workspace, L.units);
      q.nunits = at<int32_t>(workspace, L.nunits);
      q.sorted = at<int32_t>(workspace, L.sorted);
      q.part = at<uint64_t>(workspace, L.logits);
      q.lg = at<uint64_t>(workspace, L.part);
      q.tids = at<uint64_t>(workspace, L.h);
      q.gen = at<uint32_t>(workspace, L.gen);
      q.err = at<uint32_t>(workspace, L.sync) + kErrorWord;
      q.spin_limit = wait_limit();
      hipError_t e = launch_route_group(q, grid, s);
      if (e != hipSuccess) return hip_fail(e, "decode routing kernel");
      ft_moe_desc gd = *desc;
      gd.num_experts = n_group;
      st = run_grouped(&gd, T, x, ids, wts, routed, shared, y, workspace, L, s, true);
      if (st != FT_OK) return st;
      return ok();
    }
    st = run_route(desc, T, x, w_router, bias, shared_gate, at<float>(workspace, L.logits),
                   has_shared ? at<float>(workspace, L.gamma) : nullptr, ids, wts, topk_ids_out,
                   topk_w_out, at<uint32_t>(workspace, L.sync) + kRouteCounterWord,
                   at<double>(workspace, L.rsplit), nullptr, nullptr, s);
    if (st != FT_OK) return st;
    ft_moe_desc gd = *desc;
    if (slot_of) {
      // routes -> slot ids (a missing expert: slot 0, weight 0); group by slot
      hipError_t e = launch_map_slots(ids, wts, T * desc->top_k, slot_of, n_slots, miss_out, s);
      if (e != hipSuccess) return hip_fail(e, "slot map kernel");
      gd.num_experts = n_slots;
    }
    st = run_grouped(&gd, T, x, ids, wts, routed, shared, y, workspace, L, s);
    if (st != FT_OK) return st;
    return ok();
  }

  return run_fused(desc, T, x, w_router, bias, to_bank(routed, desc->inter),
                   has_shared ? to_bank(shared, desc->shared_inter) : Bank{}, shared_gate,
                   topk_ids_out, topk_w_out, y, workspace, L, grid, slot_of, n_slots, miss_out, 0,
                   s);
}

}  // namespace

extern "C" {

ft_status ft_moe_nvfp4_decode(const ft_moe_desc* desc, int64_t tokens, const uint16_t* x,
                              const float* w_router, const float* bias,
                              const ft_nvfp4_experts* routed, const ft_nvfp4_experts* shared,
                              const uint16_t* shared_gate, int32_t* topk_ids_out,
                              float* topk_w_out, uint16_t* y, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return decode_impl(desc, tokens, x, w_router, bias, routed, nullptr, 0, nullptr, shared,
                     shared_gate, topk_ids_out, topk_w_out, y, workspace, workspace_bytes, stream);
}

ft_status ft_moe_nvfp4_decode_slots(const ft_moe_desc* desc, int64_t tokens, const uint16_t* x,
                                    const float* w_router, const float* bias,
                                    const ft_nvfp4_experts* slots, int32_t n_slots,
                                    const int32_t* slot_of, const ft_nvfp4_experts* shared,
                                    const uint16_t* shared_gate, int32_t* topk_ids_out,
                                    float* topk_w_out, int32_t* miss_out, uint16_t* y,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  ft_status st = check_desc(desc);
  if (st != FT_OK) return st;
  if (!slot_of) return fail(FT_EINVAL, "slot_of is NULL");
  if (reinterpret_cast<uintptr_t>(slot_of) & 3u) return fail(FT_EINVAL, "slot_of must be 4-byte aligned");
  if (miss_out && (reinterpret_cast<uintptr_t>(miss_out) & 3u))
    return fail(FT_EINVAL, "miss_out must be 4-byte aligned");
  if (n_slots < 1) return fail(FT_EINVAL, "n_slots must be >= 1");
  if (tokens >= kGroupedDecodeMinTokens && n_slots > desc->num_experts)
    return fail(FT_EUNSUPPORTED,
                "decode_slots with %d or more tokens needs n_slots <= num_experts (%d > %d)",
                kGroupedDecodeMinTokens, n_slots, desc->num_experts);
  return decode_impl(desc, tokens, x, w_router, bias, slots, slot_of, n_slots, miss_out, shared,
                     shared_gate, topk_ids_out, topk_w_out, y, workspace, workspace_bytes, stream);
}

size_t ft_fp8_repacked_bytes(int32_t hidden, int32_t inter, int32_t n_experts, int32_t part) {
  if (hidden <= 0 || inter <= 0 || n_experts <= 0 || hidden % 128 || inter % 128) return 0;
  const size_t n = static_cast<size_t>(n_experts), H = static_cast<size_t>(hidden),
               I = static_cast<size_t>(inter);
  switch (part) {
    case 0: return n * 2 * I * H;
    case 1: return n * (2 * I / 128) * (H / 128) * 4;
    case 2: return n * H * I;
    case 3: return n * (H / 128) * (I / 128) * 4;
    default: return 0;
  }
}

ft_status ft_fp8_repack(int32_t hidden, int32_t inter, int32_t n_experts, const uint8_t* w13,
                        const float* w13_scale, const uint8_t* w2, const float* w2_scale,
                        uint8_t* out_w13, float* out_w13_scale, uint8_t* out_w2,
                        float* out_w2_scale, void* stream) {
  if (hidden <= 0 || inter <= 0 || n_experts <= 0)
    return fail(FT_EINVAL, "fp8 repack: non-positive size");
  if (hidden % 256 || inter % 128 || inter > 4096)
    return fail(FT_EUNSUPPORTED, "fp8 repack: hidden %d / inter %d unsupported (hidden %% 256, "
                "inter %% 128)", hidden, inter);
  const void* ptrs[8] = {w13, w13_scale, w2, w2_scale, out_w13, out_w13_scale, out_w2, out_w2_scale};
  for (const void* p : ptrs) {
    if (!p) return fail(FT_EINVAL, "fp8 repack: NULL pointer");
    if (!aligned16(p)) return fail(FT_EINVAL, "fp8 repack: pointers must be 16-byte aligned");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t b0 = ft_fp8_repacked_bytes(hidden, inter, n_experts, 0);
  const size_t b1 = ft_fp8_repacked_bytes(hidden, inter, n_experts, 1);
  const size_t b3 = ft_fp8_repacked_bytes(hidden, inter, n_experts, 3);
  hipError_t e = hipMemcpyAsync(out_w13, w13, b0, hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "fp8 repack w13");
  e = hipMemcpyAsync(out_w13_scale, w13_scale, b1, hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "fp8 repack w13 scales");
  e = hipMemcpyAsync(out_w2_scale, w2_scale, b3, hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "fp8 repack w2 scales");
  e = launch_repack_fp8_w2(hidden, inter, n_experts, w2, out_w2, s);
  if (e != hipSuccess) return hip_fail(e, "fp8 repack w2");
  return ok();
}

ft_status ft_moe_fp8_decode(const ft_moe_desc* desc, int64_t tokens, const uint16_t* x,
                            const float* w_router, const float* bias, const ft_fp8_experts* routed,
                            const ft_fp8_experts* shared, const uint16_t* shared_gate,
                            int32_t* topk_ids_out, float* topk_w_out, uint16_t* y,
                            void* workspace, size_t workspace_bytes, void* stream) {
  ft_status st = check_desc(desc);
  if (st != FT_OK) return st;
  if (tokens < 1 || tokens >= kGroupedDecodeMinTokens)
    return fail(tokens < 1 ? FT_EINVAL : FT_EUNSUPPORTED,
                "fp8 decode takes 1..%d tokens, got %lld", kGroupedDecodeMinTokens - 1,
                static_cast<long long>(tokens));
  if (desc->inter % 128 || desc->shared_inter % 128)
    return fail(FT_EUNSUPPORTED, "fp8 decode needs inter and shared_inter multiples of 128");
  if (!w_router) return fail(FT_EINVAL, "w_router is NULL");
  if (!aligned16(w_router)) return fail(FT_EINVAL, "w_router must be 16-byte aligned");
  if (!x || !y) return fail(FT_EINVAL, "x or y is NULL");
  if (!aligned16(x) || !aligned16(y)) return fail(FT_EINVAL, "x and y must be 16-byte aligned");
  if ((st = check_fp8_bank(routed, "routed")) != FT_OK) return st;
  const bool has_shared = desc->shared_inter > 0;
  if (has_shared) {
    if ((st = check_fp8_bank(shared, "shared")) != FT_OK) return st;
    if (!shared_gate) return fail(FT_EINVAL, "shared_gate is NULL with a shared expert");
    if (!aligned16(shared_gate)) return fail(FT_EINVAL, "shared_gate must be 16-byte aligned");
  }
  Layout L;
  if ((st = check_ws(desc, tokens, 1, workspace, workspace_bytes, &L)) != FT_OK) return st;
  int grid = 0;
  if ((st = fused_grid(&grid)) != FT_OK) return st;
  return run_fused(desc, static_cast<int>(tokens), x, w_router, bias,
                   to_bank_fp8(routed, desc->inter),
                   has_shared ? to_bank_fp8(shared, desc->shared_inter) : Bank{}, shared_gate,
                   topk_ids_out, topk_w_out, y, workspace, L, grid, nullptr, 0, nullptr, 1,
                   static_cast<hipStream_t>(stream));
}

ft_status ft_fp8_dequant(int32_t hidden, int32_t inter, int32_t n_experts,
                         const ft_fp8_experts* bank, int32_t expert, int32_t tensor, int32_t mode,
                         float* out, void* stream) {
  if (hidden <= 0 || inter <= 0 || n_experts <= 0) return fail(FT_EINVAL, "fp8 dequant: bad size");
  if (hidden % 256 || inter % 128 || inter > 4096)
    return fail(FT_EUNSUPPORTED, "fp8 dequant: hidden %d / inter %d unsupported", hidden, inter);
  if (expert < 0 || expert >= n_experts) return fail(FT_EINVAL, "fp8 dequant: expert out of range");
  if (tensor < 0 || tensor > 2) return fail(FT_EINVAL, "fp8 dequant: tensor must be 0, 1 or 2");
  if (mode != 0 && mode != 1) return fail(FT_EINVAL, "fp8 dequant: mode must be 0 or 1");
  if (!out || !aligned16(out)) return fail(FT_EINVAL, "fp8 dequant: out NULL or misaligned");
  ft_status st = check_fp8_bank(bank, "dequant");
  if (st != FT_OK) return st;
  hipError_t e = launch_fp8_dequant(hidden, inter, to_bank_fp8(bank, inter), expert, tensor, mode,
                                    out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fp8 dequant kernel");
  return ok();
}

size_t ft_fp8_linear_workspace_bytes(int64_t M, int64_t K) {
  if (M < 0 || K <= 0 || K % 64 || M > (1LL << 30) || K > (1 << 20)) return 0;
  return fp8_linear_workspace(M, K);
}

namespace {
ft_status check_fp8_linear(int64_t M, int64_t K, const uint16_t* x, const uint8_t* w,
                           const uint16_t* y, void* ws, size_t ws_bytes) {
  if (M < 0 || K <= 0) return fail(FT_EINVAL, "fp8 linear: M < 0 or K <= 0");
  if (K % 64 || M > (1LL << 30) || K > (1 << 20) || M * K > (1LL << 34))
    return fail(FT_EUNSUPPORTED, "fp8 linear: K must be a multiple of 64 (M %lld, K %lld)",
                static_cast<long long>(M), static_cast<long long>(K));
  if (!x || !w || !y) return fail(FT_EINVAL, "fp8 linear: NULL pointer");
  if (!aligned16(x) || !aligned16(w)) return fail(FT_EINVAL, "fp8 linear: x, w must be 16-byte aligned");
  if (!ws) return fail(FT_EWORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) & 255u)
    return fail(FT_EWORKSPACE, "workspace must be 256-byte aligned");
  const size_t need = fp8_linear_workspace(M, K);
  if (ws_bytes < need) return fail(FT_EWORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  return FT_OK;
}
}  // namespace

ft_status ft_fp8_quantize(int64_t M, int64_t K, const uint16_t* x, uint8_t* xq, float* x_scale,
                          void* workspace, size_t workspace_bytes, void* stream) {
  ft_status st = check_fp8_linear(M, K, x, xq, reinterpret_cast<const uint16_t*>(x_scale),
                                  workspace, workspace_bytes);
  if (st != FT_OK) return st;
  if (M == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* q = nullptr;
  float* sx = nullptr;
  hipError_t e = launch_fp8_quantize(x, M, K, workspace, &q, &sx, s);
  if (e != hipSuccess) return hip_fail(e, "fp8 quantise kernels");
  e = hipMemcpyAsync(xq, q, static_cast<size_t>(M) * K, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(x_scale, sx, sizeof(float), hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "fp8 quantise copy-out");
  return ok();
}

ft_status ft_fp8_linear(int64_t M, int64_t N, int64_t K, const uint16_t* x, const uint8_t* w,
                        const float* w_scale_rows, uint16_t* y, void* workspace,
                        size_t workspace_bytes, void* stream) {
  ft_status st = check_fp8_linear(M, K, x, w, y, workspace, workspace_bytes);
  if (st != FT_OK) return st;
  if (N <= 0 || N > (1 << 30)) return fail(FT_EINVAL, "fp8 linear: N must be in [1, 2^30]");
  if (!w_scale_rows) return fail(FT_EINVAL, "fp8 linear: w_scale_rows is NULL");
  if (M == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fp8_linear_fused_fits(M, K)) {  // one launch: codes of x formed in every block
    const hipError_t e = launch_fp8_linear_fused(x, w, static_cast<int>(M), static_cast<int>(N),
                                                 static_cast<int>(K), w_scale_rows, y,
                                                 static_cast<int>(N), 0, s);
    if (e != hipSuccess) return hip_fail(e, "fp8 fused quantise + GEMV kernel");
    return ok();
  }
  uint8_t* q = nullptr;
  float* sx = nullptr;
  hipError_t e = launch_fp8_quantize(x, M, K, workspace, &q, &sx, s);
  if (e != hipSuccess) return hip_fail(e, "fp8 quantise kernels");
  e = launch_fp8_gemm(q, w, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), sx,
                      w_scale_rows, 0.0f, y, static_cast<int>(N), 0, s);
  if (e != hipSuccess) return hip_fail(e, "fp8 gemm kernel");
  return ok();
}

ft_status ft_fp8_linear_parts(int64_t M, int64_t K, const uint16_t* x, const uint8_t* w,
                              int32_t n_parts, const int64_t* part_rows, const float* part_scales,
                              uint16_t* y, void* workspace, size_t workspace_bytes,
                              void* stream) {
  ft_status st = check_fp8_linear(M, K, x, w, y, workspace, workspace_bytes);
  if (st != FT_OK) return st;
  if (n_parts < 1 || !part_rows || !part_scales)
    return fail(FT_EINVAL, "fp8 linear parts: need n_parts >= 1 and host part arrays");
  if (part_rows[0] != 0) return fail(FT_EINVAL, "fp8 linear parts: part_rows[0] must be 0");
  for (int32_t p = 0; p < n_parts; ++p)
    if (part_rows[p + 1] <= part_rows[p])
      return fail(FT_EINVAL, "fp8 linear parts: part %d is empty or reversed", p);
  const int64_t N = part_rows[n_parts];
  if (N > (1 << 30)) return fail(FT_EINVAL, "fp8 linear parts: too many rows");
  if (M == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* q = nullptr;
  float* sx = nullptr;
  hipError_t e = launch_fp8_quantize(x, M, K, workspace, &q, &sx, s);
  if (e != hipSuccess) return hip_fail(e, "fp8 quantise kernels");
  for (int32_t p = 0; p < n_parts; ++p) {
    const int64_t r0 = part_rows[p], r1 = part_rows[p + 1];
    e = launch_fp8_gemm(q, w + r0 * K, static_cast<int>(M), static_cast<int>(r1 - r0),
                        static_cast<int>(K), sx, nullptr, part_scales[p], y, static_cast<int>(N),
                        static_cast<int>(r0), s);
    if (e != hipSuccess) return hip_fail(e, "fp8 gemm kernel (part)");
  }
  return ok();
}

int32_t ft_fp8_scale_runs(const float* w_scale_rows, int64_t N, int64_t* part_rows,
                          float* part_scales, int32_t max_parts) {
  if (!w_scale_rows || N <= 0 || !part_rows || !part_scales || max_parts < 1) return -1;
  int32_t n = 0;
  part_rows[0] = 0;
  for (int64_t r = 0; r < N; ++r) {
    const bool starts = r == 0 || std::memcmp(&w_scale_rows[r], &w_scale_rows[r - 1], 4) != 0;
    if (starts) {
      if (n == max_parts) return -1;
      part_scales[n] = w_scale_rows[r];
      if (n > 0) part_rows[n] = r;
      ++n;
    }
  }
  part_rows[n] = N;
  return n;
}

ft_status ft_attn_extend(int32_t n_new, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                         int32_t window, const uint16_t* q, const uint16_t* k_new,
                         const uint16_t* v_new, const ft_kv_cache* cache, uint16_t* out,
                         void* stream) {
  if (n_new < 0 || window < 0 || q_heads <= 0 || kv_heads <= 0 || q_heads % kv_heads)
    return fail(FT_EINVAL, "attn: bad n_new / window / head counts");
  if (head_dim != 64 && head_dim != 128)
    return fail(FT_EUNSUPPORTED, "attn: head_dim %d (64 or 128)", head_dim);
  if (!cache) return fail(FT_EINVAL, "attn: cache is NULL");
  if (cache->prefix < 0 || cache->format < 0 || cache->format > 2)
    return fail(FT_EINVAL, "attn: bad cache prefix or format");
  if (static_cast<int64_t>(n_new) * q_heads > (1LL << 30) || cache->prefix > (1 << 28))
    return fail(FT_EUNSUPPORTED, "attn: too many tokens");
  if (n_new == 0) return ok();
  if (!q || !k_new || !v_new || !out) return fail(FT_EINVAL, "attn: NULL pointer");
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out))
    return fail(FT_EINVAL, "attn: q, k_new, v_new and out must be 16-byte aligned");
  if (cache->prefix > 0) {
    if (!cache->k || !cache->v) return fail(FT_EINVAL, "attn: cache k / v NULL");
    if (!aligned16(cache->k) || !aligned16(cache->v))
      return fail(FT_EINVAL, "attn: cache k / v must be 16-byte aligned");
    if (cache->format == 2 && (!cache->k_block_scale || !cache->v_block_scale))
      return fail(FT_EINVAL, "attn: NVFP4 cache needs its block scales");
    if (cache->format != 0 && !(cache->k_scale > 0.0f && cache->k_scale <= FLT_MAX &&
                                cache->v_scale > 0.0f && cache->v_scale <= FLT_MAX))
      return fail(FT_EINVAL, "attn: k_scale and v_scale must be positive and finite");
  }
  AttnParams p{};
  p.n_new = n_new;
  p.prefix = cache->prefix;
  p.Hq = q_heads;
  p.Hkv = kv_heads;
  p.D = head_dim;
  p.window = window;
  p.format = cache->format;
  p.q = q;
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_cache = cache->k;
  p.v_cache = cache->v;
  p.k_bscale = cache->k_block_scale;
  p.v_bscale = cache->v_block_scale;
  p.k_scale = cache->k_scale;
  p.v_scale = cache->v_scale;
  p.sm_scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(head_dim)));
  p.out = out;
  hipError_t e = launch_attn_extend(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attention kernel");
  return ok();
}

ft_status ft_moe_nvfp4_prefill(const ft_moe_desc* desc, int64_t tokens, const uint16_t* x,
                               const int32_t* topk_ids, const float* topk_w,
                               const ft_nvfp4_experts* routed, const ft_nvfp4_experts* shared,
                               const uint16_t* shared_gate, uint16_t* y, void* workspace,
                               size_t workspace_bytes, void* stream) {
  ft_status st = check_desc(desc);
  if (st != FT_OK) return st;
  if (tokens < 0) return fail(FT_EINVAL, "tokens < 0");
  if (tokens > 65535) return fail(FT_EUNSUPPORTED, "prefill takes at most 65535 tokens per call");
  if (!topk_ids || !topk_w) return fail(FT_EINVAL, "topk_ids or topk_w is NULL");
  if ((st = check_layer_args(desc, x, routed, shared, shared_gate, y)) != FT_OK) return st;
  Layout L;
  if ((st = check_ws(desc, tokens, 2, workspace, workspace_bytes, &L)) != FT_OK) return st;
  if (tokens == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = static_cast<int>(tokens);
  if (desc->shared_inter > 0) {
    // sigmoid of the shared expert's gate for every token
    RouteParams p{};
    p.x = x;
    p.shared_gate = shared_gate;
    p.T = T;
    p.E = 0;
    p.H = desc->hidden;
    p.k = desc->top_k;
    p.gamma = at<float>(workspace, L.gamma);
    hipError_t e = launch_route(p, false, s);
    if (e != hipSuccess) return hip_fail(e, "shared gate kernel");
  }
  st = run_grouped(desc, T, x, topk_ids, topk_w, routed, shared, y, workspace, L, s);
  if (st != FT_OK) return st;
  return ok();
}

ft_status ft_moe_device_status(void* workspace, size_t workspace_bytes, int32_t* status,
                               void* stream) {
  if (!workspace || !status) return fail(FT_EINVAL, "device_status: NULL pointer");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(FT_EWORKSPACE, "workspace must be 256-byte aligned");
  if (workspace_bytes < 256) return fail(FT_EWORKSPACE, "workspace has %zu bytes", workspace_bytes);
  if (reinterpret_cast<uintptr_t>(status) & 3u)
    return fail(FT_EINVAL, "device_status: status must be 4-byte aligned");
  hipError_t e = launch_device_status(at<uint32_t>(workspace, 0) + kErrorWord, status,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "device status kernel");
  return ok();
}

ft_status ft_set_wait_limit(int32_t polls) {
  if (polls < 0) return fail(FT_EINVAL, "wait limit must be >= 0");
  g_wait_limit.store(polls, std::memory_order_relaxed);
  return ok();
}

ft_status ft_nvfp4_dequant(int32_t hidden, int32_t inter, int32_t n_experts,
                           const ft_nvfp4_experts* bank, int32_t expert, int32_t tensor,
                           int32_t out_dtype, void* out, void* stream) {
  if (hidden <= 0 || inter <= 0 || n_experts <= 0) return fail(FT_EINVAL, "dequant: bad size");
  if (hidden % 256 || !inter_ok(inter))
    return fail(FT_EUNSUPPORTED, "dequant: hidden %d / inter %d unsupported", hidden, inter);
  if (expert < 0 || expert >= n_experts) return fail(FT_EINVAL, "dequant: expert out of range");
  if (tensor < 0 || tensor > 2) return fail(FT_EINVAL, "dequant: tensor must be 0, 1 or 2");
  if (out_dtype < 0 || out_dtype > 4) return fail(FT_EINVAL, "dequant: out_dtype must be 0..4");
  if (!aligned16(out)) return fail(FT_EINVAL, "dequant: out must be 16-byte aligned");
  if (!out) return fail(FT_EINVAL, "dequant: out is NULL");
  ft_status st = check_bank(bank, "dequant");
  if (st != FT_OK) return st;
  hipError_t e = launch_dequant(hidden, inter, to_bank(bank, inter), expert, tensor, out_dtype, out,
                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "dequant kernel");
  return ok();
}

}  // extern "C"
