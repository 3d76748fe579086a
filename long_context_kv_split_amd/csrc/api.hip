// Status strings and version of the C ABI declared in sd.h.
#include "sd.h"

extern "C" const char *sd_status_string(sd_status status) {
  switch (status) {
    case SD_OK: return "SD_OK";
    case SD_ERR_INVALID_ARG: return "SD_ERR_INVALID_ARG: invalid argument";
    case SD_ERR_UNSUPPORTED: return "SD_ERR_UNSUPPORTED: shape or dtype not supported";
    case SD_ERR_WORKSPACE: return "SD_ERR_WORKSPACE: workspace missing or too small";
    case SD_ERR_HIP: return "SD_ERR_HIP: HIP runtime error at launch";
  }
  return "SD_ERR_UNKNOWN";
}

extern "C" int32_t sd_version(void) { return 223; }
