// abi_internal.hpp -- host helpers shared by the C ABI sources (abi.cpp,
// noalloc.hip): the thread-local error message and the static scratch set-up.
#pragma once

#include <hip/hip_runtime.h>

#include "ftmoe.h"
#include "host_layout.hpp"

namespace ftmoe {

// Sets ft_last_error() to the formatted message and returns `code`.
ft_status abi_fail(ft_status code, const char* fmt, ...);
// FT_EHIP with "what: <HIP error string>".
ft_status abi_hip_fail(hipError_t e, const char* what);

// ft_moe_nvfp4_decode_noalloc runs the one-launch kernel only (fewer tokens than
// kGroupedDecodeMinTokens).
constexpr int kNoallocMaxTokens = kGroupedDecodeMinTokens - 1;

// Address and zero fill of the no-allocation call's static scratch on `device`
// (current); once per device, from ft_init.
ft_status scratch_setup(int device);

}  // namespace ftmoe
