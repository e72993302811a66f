// Internal helpers shared by the HIP sources of libpsb (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "psb.h"

#define PSB_API extern "C" __attribute__((visibility("default")))

// Launch-error check: maps a failed launch to PSB_ERR_HIP.
#define PSB_LAUNCH_CHECK()                              \
  do {                                                  \
    if (hipGetLastError() != hipSuccess) return PSB_ERR_HIP; \
  } while (0)

namespace psb {

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Wavefront size of gfx950.
constexpr int kWave = 64;

}  // namespace psb
