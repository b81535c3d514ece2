// Status strings and version of the rbq C ABI.
#include "../../include/rbq.h"

extern "C" const char* rbq_status_string(rbq_status s) {
  switch (s) {
    case RBQ_OK: return "RBQ_OK";
    case RBQ_EINVAL: return "RBQ_EINVAL: invalid argument";
    case RBQ_ENOTSUP: return "RBQ_ENOTSUP: unsupported shape or dtype combination";
    case RBQ_EHIP: return "RBQ_EHIP: HIP launch failed";
  }
  return "RBQ_UNKNOWN";
}

extern "C" const char* rbq_version(void) { return "rbq 0.1.0 (gfx950)"; }
