// Status strings and ABI version of the library behind tt.h.
#include "common.h"

extern "C" const char* tt_status_string(int status) {
  switch (status) {
    case TT_OK: return "TT_OK";
    case TT_ERR_ARG: return "TT_ERR_ARG: invalid argument";
    case TT_ERR_UNSUPPORTED: return "TT_ERR_UNSUPPORTED: outside the implemented shapes or dtypes";
    case TT_ERR_WORKSPACE: return "TT_ERR_WORKSPACE: workspace smaller than required";
    case TT_ERR_HIP: return "TT_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown status";
  }
}

extern "C" int tt_abi_version(void) { return (1 << 16) | 2; }
