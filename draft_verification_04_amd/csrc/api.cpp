// Version and status strings of the libspecverify C ABI.
#include "spec_verify.h"

extern "C" int32_t spec_abi_version(void) { return SPEC_ABI_VERSION; }

extern "C" const char* spec_status_string(int32_t status) {
  switch (status) {
    case SPEC_OK: return "ok";
    case SPEC_ERR_INVALID_ARG: return "invalid argument";
    case SPEC_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case SPEC_ERR_UNSUPPORTED: return "unsupported by this library";
    case SPEC_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}
