// noalloc.hip -- ft_moe_nvfp4_decode_noalloc: the one-launch decode call for
// callers that cannot allocate device memory (code under HIP graph capture that
// may not call hipMalloc, tight serving loops, harnesses that forbid allocation).
//
// The call runs the same kernel as ft_moe_nvfp4_decode for 1..7 tokens; its
// workspace is `scratch`, a fixed array in device memory that every GPU the
// library runs on holds for the life of the process.  Its device address is
// taken once per device at set-up (ft_init, with that device current) and kept;
// host code never passes the array's own name to a kernel (on the host that name
// stands for a host-side shadow, not device memory).
//
// Why reuse across calls of different shapes is safe: only the one-launch decode
// kernel ever uses this memory, and everything that kernel reads back from it is
// a tagged word (value plus the generation of the call that wrote it) or its own
// per-block call counter at a fixed offset.  The counters only grow, so a word
// left by any earlier call, whatever its layer shape, carries an older
// generation and is never taken for the current call's.  The array starts at zero.
#include <hip/hip_runtime.h>

#include <mutex>

#include "abi_internal.hpp"
#include "ftmoe.h"
#include "ftmoe_kernels.hpp"

namespace ftmoe {
constexpr size_t kScratchBytes = size_t(4) << 20;  // 4 MiB: the workloads need at most 1.3 MiB
}

// The no-allocation call's workspace (one copy per GPU).
static __device__ __align__(256) unsigned char scratch[ftmoe::kScratchBytes];

namespace ftmoe {
namespace {

constexpr int kScratchDevices = 64;
void* g_scratch_ptr[kScratchDevices] = {};
std::mutex g_scratch_mu;

__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* p, size_t n16) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

void* scratch_of(int device) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_ptr[device];
}

}  // namespace

// Once per device, with `device` current (ft_init): the array's device address,
// and a zero fill (a kernel, then a wait for it).
ft_status scratch_setup(int device) {
  if (device < 0 || device >= kScratchDevices)
    return abi_fail(FT_EUNSUPPORTED, "device index %d", device);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device]) return FT_OK;
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return abi_hip_fail(e, "hipGetSymbolAddress(scratch)");
  if (!ptr || (reinterpret_cast<uintptr_t>(ptr) & 255u))
    return abi_fail(FT_EHIP, "scratch address %p is not 256-byte aligned", ptr);
  zero_fill_kernel<<<dim3(256), dim3(256), 0, nullptr>>>(static_cast<uint4*>(ptr),
                                                         kScratchBytes / 16);
  e = hipGetLastError();
  if (e != hipSuccess) return abi_hip_fail(e, "scratch zero fill");
  e = hipDeviceSynchronize();
  if (e != hipSuccess) return abi_hip_fail(e, "scratch zero fill");
  g_scratch_ptr[device] = ptr;
  return FT_OK;
}

}  // namespace ftmoe

extern "C" ft_status ft_moe_nvfp4_decode_noalloc(
    const ft_moe_desc* desc, int64_t tokens, const uint16_t* x, const float* w_router,
    const float* bias, const ft_nvfp4_experts* routed, const ft_nvfp4_experts* shared,
    const uint16_t* shared_gate, int32_t* topk_ids_out, float* topk_w_out, uint16_t* y,
    int32_t* status, void* stream) {
  using namespace ftmoe;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return abi_hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kScratchDevices) return abi_fail(FT_EUNSUPPORTED, "device index %d", dev);
  void* ptr = scratch_of(dev);
  if (!ptr) return abi_fail(FT_EINVAL, "ft_init(%d) has not been called on this device", dev);
  if (tokens < 1 || tokens >= kNoallocMaxTokens + 1)
    return abi_fail(tokens < 1 ? FT_EINVAL : FT_EUNSUPPORTED,
                    "decode_noalloc takes 1..%d tokens, got %lld", kNoallocMaxTokens,
                    static_cast<long long>(tokens));
  // an invalid descriptor gives 0 here and is reported by ft_moe_nvfp4_decode below
  const size_t need = ft_moe_workspace_bytes(desc, tokens, 1);
  if (need > kScratchBytes)
    return abi_fail(FT_EWORKSPACE, "decode_noalloc: the call needs %zu bytes of scratch, the "
                    "static scratch holds %zu", need, kScratchBytes);
  if (status && (reinterpret_cast<uintptr_t>(status) & 3u))
    return abi_fail(FT_EINVAL, "decode_noalloc: status must be 4-byte aligned");
  ft_status st = ft_moe_nvfp4_decode(desc, tokens, x, w_router, bias, routed, shared, shared_gate,
                                     topk_ids_out, topk_w_out, y, ptr, kScratchBytes, stream);
  if (st != FT_OK || !status) return st;
  return ft_moe_device_status(ptr, kScratchBytes, status, stream);
}
