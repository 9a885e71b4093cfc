// host_layout_check.cpp -- sweeps libftmoe's host-side workspace arithmetic
// (host_layout.hpp) over descriptors and token counts, built with the address and
// undefined-behaviour sanitizers by tests/test_sanitizers.py.
//
// For every accepted descriptor, path and token count it recomputes, written out
// here independently, the bytes each workspace region must hold, and checks that
// every region is 256-byte aligned, holds at least that, overlaps no other region
// and ends inside the total; and that the total never shrinks as tokens grow (a
// workspace sized for T serves every smaller T).  Prints "ok" and exits 0, or
// prints the first violation and exits 1.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "host_layout.hpp"

using namespace ftmoe;

namespace {

struct Region {
  const char* name;
  size_t off, need;
};

int g_fail = 0;

void violation(const char* what, const ft_moe_desc& d, long long T, int path, const char* r) {
  if (g_fail++ < 5)
    std::printf("VIOLATION %s: region %s, E=%d H=%d I=%d k=%d shared=%d T=%lld path=%d\n", what, r,
                d.num_experts, d.hidden, d.inter, d.top_k, d.shared_inter, T, path);
}

size_t split_need(const ft_moe_desc& d, long long T) {
  size_t need = 0;  // partial sums of every token count the split router serves
  for (long long t = kRouteSplitMinTokens; t <= T && t < kRouteMfmaMinTokens; ++t) {
    int ks = 1;  // K splits: a power of two dividing H/64, at most 32, ~512 blocks
    const long long nrb = (d.num_experts + 1 + 63) / 64, ntb = (t + 31) / 32;
    while ((d.hidden / 64) % (2 * ks) == 0 && 2 * ks <= 32 && nrb * ntb * 2 * ks <= 512) ks *= 2;
    need = std::max(need, static_cast<size_t>(ks) * static_cast<size_t>(t) *
                              static_cast<size_t>(d.num_experts + 1) * 8);
  }
  return need;
}

std::vector<Region> regions(const ft_moe_desc& d, long long T, int path, const Layout& L) {
  const size_t t = T, k = d.top_k, E = d.num_experts, H = d.hidden;
  const size_t imax = std::max(d.inter, d.shared_inter);
  const size_t nslots = k + (d.shared_inter > 0);
  const size_t ut = T <= 64 ? 16 : 256;
  const size_t P = t * k;
  const size_t units = std::min(P, E) + P / ut + (d.shared_inter > 0 ? (t + ut - 1) / ut : 0) + 8;
  std::vector<Region> r = {{"sync", L.sync, 34 * 4}};  // route counter; error words 32, 33
  auto grouped = [&]() {
    r.push_back({"gamma", L.gamma, t * 4});
    r.push_back({"count", L.count, E * 4});
    r.push_back({"cursor", L.cursor, E * 4});
    r.push_back({"offset", L.offset, E * 4});
    r.push_back({"units", L.units, units * 16});
    r.push_back({"nunits", L.nunits, 4});
    r.push_back({"sorted", L.sorted, P * 4});
    r.push_back({"hhi", L.hhi, (P + t) * imax * 2});
    r.push_back({"hlo", L.hlo, (P + t) * imax * 2});
    r.push_back({"out", L.out, t * nslots * H * 4});
  };
  if (path == 0) {
    r.push_back({"logits", L.logits, t * E * 4});
    r.push_back({"rsplit", L.rsplit, split_need(d, T)});
  } else if (path == 1) {
    r.push_back({"gen", L.gen, 1024 * 4});
    r.push_back({"logits", L.logits, std::max(16 * t * (E + 1) * 8, t * E * 4)});
    r.push_back({"h", L.h, t * nslots * imax * 8});
    r.push_back({"part", L.part, 1024 * 64 * 8});
    if (T >= 8) {
      r.push_back({"ids", L.ids, t * k * 4});
      r.push_back({"w", L.w, t * k * 4});
      r.push_back({"rsplit", L.rsplit, split_need(d, T)});
      grouped();
    }
  } else {
    grouped();
  }
  return r;
}

void check(const ft_moe_desc& d, long long T, int path) {
  const Layout L = layout(d, T, path);
  std::vector<Region> r = regions(d, T, path, L);
  for (const Region& a : r) {
    if (a.off % 256) violation("misaligned", d, T, path, a.name);
    if (a.off + a.need > L.total) violation("past the total", d, T, path, a.name);
    for (const Region& b : r) {
      if (&a == &b || a.need == 0 || b.need == 0) continue;
      if (a.off < b.off + b.need && b.off < a.off + a.need) violation("overlap", d, T, path, a.name);
    }
  }
}

// The one-launch routing of a decode batch: every region its kernel writes lies
// inside the decode layout's region it borrows, and the split count keeps whole
// 16-K pieces per wave and one task per block.
void check_route_group(const ft_moe_desc& d, long long T) {
  const Layout L = layout(d, T, 1);
  const std::vector<Region> r = regions(d, T, 1, L);
  auto need_of = [&](const char* name) -> size_t {
    for (const Region& a : r)
      if (std::string(a.name) == name) return a.need;
    return 0;
  };
  for (int grid : {16, 64, 128, 256, 304, 1024}) {
    if (!route_group_fits(d, T, grid, d.num_experts)) continue;
    const size_t t = static_cast<size_t>(T), E = static_cast<size_t>(d.num_experts);
    const int ks = route_group_splits(d.num_experts, d.hidden, grid);
    const size_t nrt = (E + 15) / 16;
    if (ks < 1 || ks > kRouteGroupMaxSplits || (ks & (ks - 1)) != 0)
      violation("route split count", d, T, 1, "ksplit");
    if (ks > 1 && static_cast<int>(nrt) * ks > grid) violation("route tasks > grid", d, T, 1, "ksplit");
    if (d.hidden % (128 * ks) != 0) violation("route pieces", d, T, 1, "ksplit");
    if (2 * T > grid) violation("route blocks", d, T, 1, "grid");
    if (static_cast<size_t>(ks) * nrt * 16 * t * 16 > need_of("logits"))
      violation("route partial sums", d, T, 1, "logits");
    if (t * E * 8 > need_of("part")) violation("route logits", d, T, 1, "part");
    if (t * static_cast<size_t>(d.top_k) * 8 > need_of("h")) violation("route ids", d, T, 1, "h");
  }
}

}  // namespace

int main() {
  const int Es[] = {1, 2, 8, 16, 100, 288, 512, 1000, 1024, 1025};
  const int Hs[] = {128, 256, 1024, 2048, 3072, 4096, 8192, 8448};
  const int Is[] = {32, 64, 128, 512, 768, 4096, 4160};
  const int ks[] = {1, 2, 8, 10, 16, 17};
  const int shs[] = {0, 64, 512, 4096};
  const long long Ts[] = {0,   1,    2,    7,    8,    16,   23,    24,      25,     31,
                          32,  33,   63,   64,   65,   255,  256,   1023,    1024,   1025,
                          4096, 8192, 65535, 1 << 21};
  long long accepted = 0, rejected = 0, checked = 0;
  for (int E : Es)
    for (int H : Hs)
      for (int I : Is)
        for (int k : ks)
          for (int sh : shs) {
            ft_moe_desc d{E, H, I, k, 1, 7.0f, 7.0f, sh};
            char msg[160];
            if (desc_problem(&d, msg, sizeof msg) != FT_OK) {
              ++rejected;
              continue;
            }
            ++accepted;
            for (int path = 0; path < 3; ++path) {
              const long long tmax = path == 0 ? (1 << 21) : (path == 1 ? 64 : 65535);
              size_t prev = 0;
              for (long long T : Ts) {
                if (T > tmax) continue;
                check(d, T, path);
                if (path == 1 && T >= 8) check_route_group(d, T);
                ++checked;
                const size_t tot = layout(d, T, path).total;
                if (tot < prev) violation("total shrank", d, T, path, "total");
                prev = tot;
              }
            }
          }
  std::printf("descriptors accepted %lld rejected %lld, layouts checked %lld\n", accepted, rejected,
              checked);
  if (g_fail) return 1;
  std::printf("ok\n");
  return 0;
}
