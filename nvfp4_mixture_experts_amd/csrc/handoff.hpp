// handoff.hpp -- generation-tagged words: how the persistent kernels of libftmoe
// hand values from one block to another without grid barriers.  A value sits in
// the low half of an 8-byte word and the call's generation in the high half; it
// is written and read with single device-coherent 8-byte accesses, and a consumer
// polls until the tag carries its own generation.  Every poll is bounded: a wait
// that gives up records why in the workspace's error word.
#pragma once

#include "ftmoe_device.hpp"

namespace ftmoe {

// ------------------------------------------------------------ tagged words --

__device__ __forceinline__ uint64_t tagged(float v, uint32_t gen) {
  return (static_cast<uint64_t>(gen) << 32) | __float_as_uint(v);
}
__device__ __forceinline__ void st_tag(uint64_t* p, float v, uint32_t gen) {
  __hip_atomic_store(p, tagged(v, gen), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tag(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_is(uint64_t w, uint32_t gen) {
  return static_cast<uint32_t>(w >> 32) == gen;
}
__device__ __forceinline__ float tag_value(uint64_t w) {
  return __uint_as_float(static_cast<uint32_t>(w));
}

// ------------------------------------------------------------ give-ups --
//
// err[0] collects the reasons (kWait* bits) of every wait that gave up since the
// caller last read the status (ft_moe_device_status reads and clears it); err[1]
// holds the generation of the latest call with a give-up, so that every other
// wait of that call stops within 16 polls instead of running to its own limit.
enum : uint32_t { kWaitLogits = 1u, kWaitGate = 2u, kWaitH = 4u, kWaitPartial = 8u,
                  kWaitRoutes = 16u };

__device__ __forceinline__ void give_up(uint32_t* err, uint32_t gen, uint32_t why) {
  __hip_atomic_fetch_or(err, why, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  st_dev(err + 1, gen);
}

// True when the wait has polled `spin_limit` times, or (checked every 16th poll)
// another wait of this call has already given up; records the first case.
__device__ __forceinline__ bool stop_waiting(int spins, int spin_limit, uint32_t* err,
                                             uint32_t gen, uint32_t why) {
  if (spins >= spin_limit) {
    give_up(err, gen, why);
    return true;
  }
  return (spins & 15) == 15 && ld_dev(err + 1) == gen;
}

// Reads one tagged word per lane, polling until every lane's word carries `gen`.
__device__ __forceinline__ uint64_t poll_tag(const uint64_t* p, uint32_t gen, int spin_limit,
                                             uint32_t* err) {
  uint64_t wd = ld_tag(p);
  for (int spins = 0; __ballot(!tag_is(wd, gen)) != 0; ++spins) {
    if (stop_waiting(spins, spin_limit, err, gen, kWaitLogits)) break;
    __builtin_amdgcn_s_sleep(1);
    if (!tag_is(wd, gen)) wd = ld_tag(p);
  }
  return wd;
}

}  // namespace ftmoe
