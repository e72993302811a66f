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

// Largest i in [0, n) with c[i] <= p, or -1 (c non-decreasing).
__device__ inline int32_t last_le(const int32_t* c, int32_t n, int32_t p) {
  int32_t lo = 0, hi = n;  // search in [lo, hi)
  while (lo < hi) {
    const int32_t mid = (lo + hi) >> 1;
    if (c[mid] <= p) lo = mid + 1; else hi = mid;
  }
  return lo - 1;
}

// Enqueues the check that every non-padding id of doc_ids [B, S] (row stride row_stride)
// forms one contiguous run per row; ORs PSB_DATA_DOC_NOT_CONTIGUOUS into *status_word
// when not.  Argument errors are returned before anything is enqueued.
psb_status launch_contiguity_check(const int32_t* doc_ids, int64_t B, int64_t S, int64_t row_stride,
                                   int32_t* status_word, hipStream_t stream);

}  // namespace psb
