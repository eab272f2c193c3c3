// Status strings and version of the C ABI.
#include "common.h"

MOE_API const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported shape or dtype";
    case MOE_EWORKSPACE: return "workspace missing or too small";
    case MOE_EHIP: return "HIP runtime error";
    case MOE_ESCRATCH: return "problem needs more scratch than the no-allocation entry point holds (4 MiB)";
    default: return "unknown status";
  }
}

MOE_API int moe_version(void) { return 100; }
