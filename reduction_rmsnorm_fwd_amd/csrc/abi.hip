// Library-level calls of the C ABI: status strings, ABI version, device check.
#include <string.h>

#include "fo_common.hpp"

extern "C" const char* fo_status_str(int s) {
  switch (s) {
    case FO_OK: return "FO_OK";
    case FO_ERR_NULL: return "FO_ERR_NULL: a required pointer is NULL";
    case FO_ERR_SHAPE: return "FO_ERR_SHAPE: a size is out of range";
    case FO_ERR_DTYPE: return "FO_ERR_DTYPE: dtype not supported by this op";
    case FO_ERR_STRIDE: return "FO_ERR_STRIDE: row stride too small or misaligned";
    case FO_ERR_WORKSPACE: return "FO_ERR_WORKSPACE: workspace missing or too small";
    case FO_ERR_DEVICE: return "FO_ERR_DEVICE: no gfx950 device";
    case FO_ERR_HIP: return "FO_ERR_HIP: a HIP launch failed";
    default: return "unknown fo status";
  }
}

extern "C" int fo_abi_version(void) { return FO_ABI_VERSION; }

extern "C" int fo_device_supported(int dev) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || dev < 0 || dev >= n) return FO_ERR_DEVICE;
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) != hipSuccess) return FO_ERR_DEVICE;
  return strncmp(p.gcnArchName, "gfx950", 6) == 0 ? FO_OK : FO_ERR_DEVICE;
}
