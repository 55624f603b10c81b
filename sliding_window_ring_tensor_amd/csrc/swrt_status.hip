// swrt_status.hip -- status strings and ABI version of libswrt.
#include "swrt.h"

extern "C" const char *swrt_status_string(int status) {
  switch (status) {
    case SWRT_OK: return "ok";
    case SWRT_E_INVALID_ARG: return "invalid argument (nothing launched)";
    case SWRT_E_UNSUPPORTED: return "unsupported size or element layout (nothing launched)";
    case SWRT_E_LAUNCH: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

extern "C" int swrt_abi_version(void) { return SWRT_ABI_VERSION; }
