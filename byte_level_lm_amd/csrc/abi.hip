// Library-wide entry points of the C ABI: version and status strings.
#include "common.h"

extern "C" int bllm_version(void) { return BLLM_VERSION_NUMBER; }

extern "C" const char* bllm_status_string(int code) {
  switch (code) {
    case BLLM_OK: return "ok";
    case BLLM_E_INVAL: return "invalid argument";
    case BLLM_E_NOTSUP: return "unsupported shape, dtype or alignment";
    case BLLM_E_WS: return "workspace missing or too small";
    case BLLM_E_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}
