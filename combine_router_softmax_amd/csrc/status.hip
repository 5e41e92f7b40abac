// Version and status strings of the C ABI.
#include "moe_common.hpp"

MOE_API int moe_abi_version(void) { return MOE_ABI_VERSION; }

MOE_API const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported by this build";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP runtime or launch failure";
  }
  return "unknown status";
}
