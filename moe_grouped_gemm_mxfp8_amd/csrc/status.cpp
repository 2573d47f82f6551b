// Status strings of the C ABI.
#include "../../include/moe_gg.h"

extern "C" MOE_GG_API const char *moe_gg_status_string(int status) {
  switch (status) {
    case MOE_GG_OK: return "ok";
    case MOE_GG_EINVAL: return "invalid argument (null pointer, non-positive or misaligned size)";
    case MOE_GG_EUNSUPPORTED: return "unsupported shape for these kernels";
    case MOE_GG_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}
