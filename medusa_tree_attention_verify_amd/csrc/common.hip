// Library-wide entry points: status strings, device check, version.

#include <string.h>

#include "mv_host.h"

extern "C" {

MV_API const char* mv_status_string(int status) {
  switch (status) {
    case MV_OK: return "ok";
    case MV_ERR_INVALID_ARG: return "invalid argument";
    case MV_ERR_INVALID_TREE: return "invalid tree specification";
    case MV_ERR_UNSUPPORTED: return "unsupported size or dtype";
    case MV_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MV_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

MV_API int mv_device_check(int device) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n) return MV_ERR_HIP;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return MV_ERR_HIP;
  return strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? MV_OK : MV_ERR_UNSUPPORTED;
}

MV_API int mv_version(void) { return 100; }

}  // extern "C"
