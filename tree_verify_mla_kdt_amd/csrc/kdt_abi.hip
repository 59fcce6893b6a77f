// Version and status-string entry points of the kdt C ABI.
#include "kdt_common.hpp"

extern "C" int kdt_abi_version(void) { return KDT_ABI_VERSION; }

extern "C" const char* kdt_status_str(int code) {
  switch (code) {
    case KDT_OK: return "ok";
    case KDT_ERR_INVALID_ARG: return "invalid argument";
    case KDT_ERR_UNSUPPORTED: return "unsupported shape, dtype or alignment";
    case KDT_ERR_WORKSPACE: return "workspace missing or too small";
    case KDT_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}
