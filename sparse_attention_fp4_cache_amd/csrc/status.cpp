// status.cpp -- status-code names of the C ABI.
#include "csa2fp4.h"

extern "C" const char* csa2_status_string(int status) {
  switch (status) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_NULL: return "null pointer argument";
    case CSA2_ERR_SHAPE: return "size or count out of range";
    case CSA2_ERR_UNSUPPORTED: return "unsupported configuration";
    case CSA2_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA2_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}
