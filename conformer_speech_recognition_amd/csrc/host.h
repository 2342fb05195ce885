// Host-side helpers shared by the C-ABI translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gigaam.h"

namespace gg {

// Record a printf-style message for gigaam_last_error() and return `code`.
int fail(int code, const char* fmt, ...);

// Round-to-nearest-even fp32 -> fp16 / bf16 bit patterns.
uint16_t f32_to_f16_bits(float v);
uint16_t f32_to_bf16_bits(float v);

}  // namespace gg

#define HIP_TRY(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess)                                                               \
      return gg::fail(GIGAAM_E_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));   \
  } while (0)
