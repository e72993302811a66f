// Status strings and version of the psb C ABI (host-only).
#include "psb.h"

#define PSB_API extern "C" __attribute__((visibility("default")))

PSB_API const char* psb_status_string(psb_status status) {
  switch (status) {
    case PSB_OK: return "ok";
    case PSB_ERR_INVALID_ARG: return "invalid argument (null pointer, negative size, misalignment or non-finite scale)";
    case PSB_ERR_SHAPE: return "inconsistent shapes, strides or query shard range";
    case PSB_ERR_UNSUPPORTED: return "unsupported head dimension (64 and 128 are built)";
    case PSB_ERR_CAPACITY: return "output or workspace buffer too small";
    case PSB_ERR_HIP: return "HIP runtime error (kernel launch failed)";
    case PSB_ERR_SCRATCH_LIMIT:
      return "problem needs more scheduler memory than the no-allocation entry point's static buffer holds";
    default: return "unknown status";
  }
}

PSB_API int32_t psb_version(void) { return 100; }
