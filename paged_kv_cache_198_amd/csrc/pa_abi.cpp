// Library-wide entry points of libpa: version and status text.
#include "pa.h"

extern "C" int pa_version(void) { return 100; }  // 0.1.0

extern "C" const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID: return "invalid argument";
    case PA_ERR_OOM: return "out of KV blocks";
    case PA_ERR_HIP: return "HIP launch error";
    case PA_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case PA_ERR_UNSUPPORTED: return "shape or type outside the compiled set";
    case PA_ERR_TOO_LARGE: return "workspace needed exceeds the static scratch";
    default: return "unknown status";
  }
}
