// Status-code names of the C ABI (declared in include/hybrid_attn.h).  Host
// code only, built with the host compiler like the step generator.
#include "hybrid_attn.h"

extern "C" const char* ha_status_string(ha_status status) {
  switch (status) {
    case HA_OK: return "HA_OK";
    case HA_ERR_INVALID_ARGUMENT: return "HA_ERR_INVALID_ARGUMENT";
    case HA_ERR_UNSUPPORTED: return "HA_ERR_UNSUPPORTED";
    case HA_ERR_WORKSPACE_TOO_SMALL: return "HA_ERR_WORKSPACE_TOO_SMALL";
    case HA_ERR_HIP: return "HA_ERR_HIP";
  }
  return "HA_ERR_UNKNOWN";
}
