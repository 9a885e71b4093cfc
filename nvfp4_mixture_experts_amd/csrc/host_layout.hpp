// host_layout.hpp -- host-only arithmetic of libftmoe: descriptor checks, the
// launch-shape helpers that size workspace regions, and the workspace layout of
// every entry point.  Plain C++ (no HIP): abi.cpp and the kernel sources use it,
// and it is compiled on its own, with the address and undefined-behaviour
// sanitizers, by a CPU test that sweeps shapes and token counts.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <stdio.h>

#include "ftmoe.h"

namespace ftmoe {

// ------------------------------------------------------------ constants --

constexpr int kLogitCopies = 16;      // replicas of the router logits (spreads the reads)
constexpr int kMaxFusedGrid = 1024;   // blocks of the one-launch decode kernel, at most
constexpr int kRowGroup = 64;         // output rows of one down-GEMV group (one per lane)
constexpr int kMaxTopK = 16;
constexpr int kMaxDecodeTokens = 64;
constexpr int kGroupedDecodeMinTokens = 8;  // decode calls from here on take the grouped path
constexpr int kRouteMfmaMinTokens = 1024;   // router calls from here on: unsplit fp64 MFMA
constexpr int kRouteSplitMinTokens = 24;    // ... and from here on: split-K fp64 MFMA

constexpr int kMaxExperts = 1024;   // experts per bank supported by the grouping kernels
constexpr int kGroupPairs = 1024;   // pairs per histogram block
constexpr int kGroupOneBlockPairs = 16384;  // up to this many pairs are grouped by one block
constexpr int kPfUnitTokens = 256;    // tokens per work unit of a many-token call
constexpr int kSmallCallTokens = 64;  // calls of at most this many tokens take the few-token
constexpr int kSmallUnitTokens = 16;  // kernels, with units of at most this many tokens (one
                                      // MFMA column block: a unit's tokens share one weight pass)
// Spare entries after the last possible unit of the unit table: the expert kernels
// read units[u] (u < 8 * ceil(units / 8)) together with the unit count, before
// checking u against it.
constexpr int kUnitSlack = 8;

// Split-K fp64 MFMA router: tokens per block, target blocks, most K splits.
constexpr int kRouteSplitTokens = 32;
constexpr int kRouteSplitTargetBlocks = 512;
constexpr int kRouteMaxSplits = 32;

struct PfUnit {
  int bank;    // 0 routed, 1 shared
  int expert;  // routed expert id (0 for the shared bank)
  int start;   // routed: first position in `sorted`; shared: first token
  int count;   // 1 .. unit_tokens
};

// ------------------------------------------------------- launch shapes --

// The widest power of two <= 64 lanes per row that divides the H/32 chunks of a
// gate|up row, and the chunks each lane then owns (supported: lpr > 0, cpl 1..4).
inline void gateup_geometry(int H, int* lpr, int* cpl) {
  const int chunks = H / 32;
  int l = 64;
  while (l > 8 && chunks % l != 0) l >>= 1;
  *lpr = (chunks % l == 0) ? l : 0;
  *cpl = (*lpr > 0) ? chunks / l : 0;
}

inline int prefill_unit_tokens(int T) {
  return T <= kSmallCallTokens ? kSmallUnitTokens : kPfUnitTokens;
}

// sum over experts of ceil(n_e / ut) <= (experts with a pair) + P / ut, plus the
// shared expert's units
inline int prefill_max_units(int E, int T, int k, bool shared) {
  const long long P = static_cast<long long>(T) * k;
  const int ut = prefill_unit_tokens(T);
  const long long n = (P < E ? P : E) + P / ut + (shared ? (T + ut - 1) / ut : 0);
  return static_cast<int>(n);
}

inline int prefill_group_blocks(int T, int k) {
  const long long P = static_cast<long long>(T) * k;
  return static_cast<int>((P + kGroupPairs - 1) / kGroupPairs);
}

// K splits of the split-K router for (E, T, H): the largest power of two that
// divides H / 64 and keeps about kRouteSplitTargetBlocks blocks (chosen as for
// 64-row blocks whatever the block's wave count: more splits add partial sums for
// the top-k to read, measured slower at 64 tokens).
inline int route_split_k(int E, int T, int H) {
  const int nrb = (E + 1 + 63) / 64;
  const int ntb = (T + kRouteSplitTokens - 1) / kRouteSplitTokens;
  const int kmax = H / 64;  // 64-K steps
  int ks = 1;
  while ((kmax % (2 * ks)) == 0 && 2 * ks <= kRouteMaxSplits &&
         nrb * ntb * 2 * ks <= kRouteSplitTargetBlocks)
    ks *= 2;
  return ks;
}

inline size_t route_split_bytes(int E, int T, int H) {
  return static_cast<size_t>(route_split_k(E, T, H)) * T * (E + 1) * sizeof(double);
}

// The one-launch routing of a decode batch (8..64 tokens): K splits of its fp64
// router product, the largest power of two up to kRouteGroupMaxSplits that keeps
// one (16-row tile, split) task per block of a `grid`-block launch, a whole number
// of 16-K pieces for each of the block's 8 waves, and the partial sums (16 bytes
// per row of every 16-row tile, token and split) inside the tagged logits region
// of the decode workspace (kLogitCopies * T * (E + 1) words).
constexpr int kRouteGroupMaxSplits = 8;

inline int route_group_splits(int E, int H, int grid) {
  const int nrt = (E + 15) / 16;
  int ks = 1;
  while (2 * ks <= kRouteGroupMaxSplits && nrt * 2 * ks <= grid && H % (128 * 2 * ks) == 0 &&
         2 * (2 * ks) * nrt <= E + 1)
    ks *= 2;
  return ks;
}

// Whether a decode call of T tokens takes the one-launch routing: a block per
// token for the selection and another for its shared gate fit the grid, the
// partial sums fit the tagged logits region, the logits the partial-output region
// and the ids the h region (path-1 layout).
inline bool route_group_fits(const ft_moe_desc& d, int64_t T, int grid, int n_group) {
  if (T < kGroupedDecodeMinTokens || T > kMaxDecodeTokens || 2 * T > grid) return false;
  if (n_group < 1 || n_group > kMaxExperts || d.hidden % 128 != 0) return false;
  const size_t t = static_cast<size_t>(T), E = static_cast<size_t>(d.num_experts);
  const size_t ks = static_cast<size_t>(route_group_splits(d.num_experts, d.hidden, grid));
  const size_t logits_bytes = static_cast<size_t>(kLogitCopies) * t * (E + 1) * 8;
  const size_t imax = static_cast<size_t>(d.inter > d.shared_inter ? d.inter : d.shared_inter);
  const size_t nslots = static_cast<size_t>(d.top_k) + (d.shared_inter > 0 ? 1 : 0);
  const size_t part_bytes = static_cast<size_t>(kMaxFusedGrid) * kRowGroup * 8;
  const size_t nrt = (E + 15) / 16;
  return ks * nrt * 16 * t * 16 <= logits_bytes && t * E * 8 <= part_bytes &&
         t * static_cast<size_t>(d.top_k) * 8 <= t * nslots * imax * 8;
}

// -------------------------------------------------------- descriptors --

// Whether the grouped expert GEMMs hand h from the gate|up product to the down
// product in fp16 (one MFMA operand) rather than as a bf16 (hi, lo) pair (two):
// only when the activation bounds |h| well inside fp16's range.  The clamped SwiGLU
// gives |h| <= max(gate_max, 0.2785) * |up_absmax| (|silu(g)| < 0.2785 for g <= 0,
// silu(g) < g for g > 0); the plain SwiGLU is unbounded.  NaN limits give the pair.
inline bool prefill_h16(int act, float gate_max, float up_absmax) {
  if (act != 1) return false;
  const float gm = gate_max > 0.2785f ? gate_max : 0.2785f;
  const float ua = up_absmax < 0.0f ? -up_absmax : up_absmax;
  return gm * ua <= 32768.0f;
}

inline bool inter_ok(int I) { return I >= 64 && I <= 4096 && I % 64 == 0; }

// FT_OK, or the status of the first problem of the descriptor, with its message
// formatted into buf[n].
inline ft_status desc_problem(const ft_moe_desc* d, char* buf, size_t n) {
  if (!d) {
    snprintf(buf, n, "desc is NULL");
    return FT_EINVAL;
  }
  if (d->num_experts <= 0 || d->hidden <= 0 || d->inter <= 0 || d->top_k <= 0 ||
      d->shared_inter < 0) {
    snprintf(buf, n, "desc has a non-positive size");
    return FT_EINVAL;
  }
  if (d->top_k > d->num_experts) {
    snprintf(buf, n, "top_k %d exceeds num_experts %d", d->top_k, d->num_experts);
    return FT_EINVAL;
  }
  if (d->act != 0 && d->act != 1) {
    snprintf(buf, n, "act must be 0 or 1");
    return FT_EINVAL;
  }
  if (d->num_experts > kMaxExperts) {
    snprintf(buf, n, "num_experts %d > %d", d->num_experts, kMaxExperts);
    return FT_EUNSUPPORTED;
  }
  if (d->top_k > kMaxTopK) {
    snprintf(buf, n, "top_k %d > %d", d->top_k, kMaxTopK);
    return FT_EUNSUPPORTED;
  }
  int lpr = 0, cpl = 0;
  gateup_geometry(d->hidden, &lpr, &cpl);
  if (d->hidden % 256 != 0 || d->hidden > 8192 || lpr == 0 || cpl < 1 || cpl > 4) {
    snprintf(buf, n, "hidden %d unsupported (multiple of 256, <= 8192)", d->hidden);
    return FT_EUNSUPPORTED;
  }
  if (!inter_ok(d->inter)) {
    snprintf(buf, n, "inter %d unsupported (multiple of 64 in [64, 4096])", d->inter);
    return FT_EUNSUPPORTED;
  }
  if (d->shared_inter != 0 && !inter_ok(d->shared_inter)) {
    snprintf(buf, n, "shared_inter %d unsupported", d->shared_inter);
    return FT_EUNSUPPORTED;
  }
  return FT_OK;
}

// ---------------------------------------------------------- workspace --

// Workspace regions (byte offsets, each 256-byte aligned).  The sync region at
// offset 0 holds the route counter (word 0, reset by the kernel that uses it) and
// the decode error word (words 32, 33).
struct Layout {
  size_t sync, gen, logits, h, part;  // route / one-launch decode
  size_t rsplit;                      // split-K router partials
  size_t wsplit, wnorm;               // many-token router: row pieces and norms
  size_t ids, w;                      // routes of a grouped decode
  size_t gamma, count, cursor, offset, units, nunits, sorted, hhi, hlo, out;  // grouped experts
  size_t total;
};

constexpr int kRouteCounterWord = 0;  // in the sync region
constexpr int kErrorWord = 32;        // in the sync region (its own cache line): reasons,
                                      // then the generation of the latest give-up

inline size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

// Bytes of the split router's partial sums for up to T tokens (the largest over
// every token count it serves, so that a workspace for T serves smaller T).
inline size_t route_split_cap(const ft_moe_desc& d, int64_t T) {
  size_t cap = 0;
  const int64_t hi = T < kRouteMfmaMinTokens ? T : kRouteMfmaMinTokens - 1;
  for (int64_t t = kRouteSplitMinTokens; t <= hi; ++t) {
    const size_t b = route_split_bytes(d.num_experts, static_cast<int>(t), d.hidden);
    cap = b > cap ? b : cap;
  }
  return cap;
}

// Layout of the workspace of path 0 (ft_moe_route), 1 (ft_moe_nvfp4_decode) or
// 2 (ft_moe_nvfp4_prefill) for T tokens; `d` must have passed desc_problem.
inline Layout layout(const ft_moe_desc& d, int64_t T, int path) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t t = static_cast<size_t>(T);
  const size_t k = static_cast<size_t>(d.top_k);
  const size_t E = static_cast<size_t>(d.num_experts);
  const size_t H = static_cast<size_t>(d.hidden);
  const size_t imax = static_cast<size_t>(d.inter > d.shared_inter ? d.inter : d.shared_inter);
  const size_t nslots = k + (d.shared_inter > 0 ? 1 : 0);
  L.sync = take(256);  // route counter, error word
  auto grouped = [&]() {
    const int Ti = static_cast<int>(T), ki = d.top_k;
    const size_t P = t * k;
    L.gamma = take(t * 4);
    L.count = take(E * 4);
    L.cursor = take(E * 4);
    L.offset = take(E * 4);
    L.units = take(static_cast<size_t>(prefill_max_units(d.num_experts, Ti, ki,
                                                         d.shared_inter > 0) + kUnitSlack) *
                   sizeof(PfUnit));
    L.nunits = take(4);
    L.sorted = take(P * 4);
    L.hhi = take((P + t) * imax * 2);
    L.hlo = take((P + t) * imax * 2);
    L.out = take(t * nslots * H * 4);
  };
  if (path == 0) {
    L.logits = take(t * E * 4);
    L.rsplit = take(route_split_cap(d, T));
    if (T >= kRouteMfmaMinTokens) {
      L.wsplit = take(E * H * 4);
      L.wnorm = take(E * 4);
    }
  } else if (path == 1) {
    // the one-launch kernel's regions, then (for token counts that take the
    // grouped path) router logits, routes and the grouped regions
    L.gen = take(static_cast<size_t>(kMaxFusedGrid) * 4);
    const size_t fused_logits = static_cast<size_t>(kLogitCopies) * t * (E + 1) * 8;
    const size_t route_logits = t * E * 4;
    L.logits = take(fused_logits > route_logits ? fused_logits : route_logits);
    L.h = take(t * nslots * imax * 8);
    L.part = take(static_cast<size_t>(kMaxFusedGrid) * kRowGroup * 8);
    if (T >= kGroupedDecodeMinTokens) {
      L.ids = take(t * k * 4);
      L.w = take(t * k * 4);
      L.rsplit = take(route_split_cap(d, T));
      grouped();
    }
  } else {
    grouped();
  }
  L.total = off;
  return L;
}

}  // namespace ftmoe
