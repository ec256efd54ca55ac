// status.cpp -- text for libfp8q status codes.
#include "fp8q.h"

extern "C" const char* fp8_status_string(int status) {
  switch (status) {
    case FP8Q_OK: return "ok";
    case FP8Q_EINVAL: return "invalid argument (nothing was enqueued)";
    case FP8Q_EUNSUPPORTED: return "unsupported request";
    case FP8Q_EHIP: return "HIP runtime call or kernel launch failed";
    default: return "unknown status";
  }
}
