// Small host-side helpers of the C ABI.
#include "sv_common.h"

extern "C" const char* sv_status_string(sv_status s) {
  switch (s) {
    case SV_OK: return "ok";
    case SV_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SV_ERR_UNSUPPORTED: return "unsupported shape or type";
    case SV_ERR_BAD_TREE: return "validation found a data error (see the status array)";
    case SV_ERR_HIP: return "HIP launch error";
    case SV_ERR_SCRATCH_LIMIT: return "workspace larger than the library's scratch array";
    default: return "unknown status";
  }
}

extern "C" int32_t sv_version(void) { return 100; }
