// Internal helpers shared by the libpa translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

inline int elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
    default: return 0;
  }
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Status of the launches just enqueued.
inline int launch_status() { return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP; }

}  // namespace pa
