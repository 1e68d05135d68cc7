// Host-side helpers shared by the libpagedattn entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedattn.h"

namespace pa {

// Element size of a pa_dtype in bytes; 0 for an unknown code.
inline int elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
    default: return 0;
  }
}

// Whether a cache pa_dtype holds 8-bit codes with scales (INT8 or FP8).
inline bool is_q8(int32_t dtype) { return dtype == PA_I8 || dtype == PA_FP8; }

inline bool aligned16(const void* p) { return p && ((uintptr_t)p & 15u) == 0; }

// Status of the launches just made (clears HIP's sticky launch error).
inline pa_status launch_status() {
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa
