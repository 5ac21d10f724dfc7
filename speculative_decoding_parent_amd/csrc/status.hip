// Version and status strings of the eagle.h C ABI.
#include "common.h"

extern "C" int eagle_abi_version(void) { return EAGLE_ABI_VERSION; }

extern "C" const char* eagle_status_string(int status) {
  switch (status) {
    case EAGLE_OK: return "ok";
    case EAGLE_EINVAL: return "invalid argument";
    case EAGLE_EUNSUPPORTED: return "unsupported shape or type";
    case EAGLE_EWORKSPACE: return "workspace too small";
    case EAGLE_EHIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}
