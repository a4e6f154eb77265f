// Return-code names and ABI version of libech.
#include "ech.h"

extern "C" const char* ech_status_str(int code) {
  switch (code) {
    case ECH_OK: return "ok";
    case ECH_EINVAL: return "invalid argument (size, pointer, alignment or unsupported shape)";
    case ECH_ENOSPC: return "selection demand exceeds the device cache size";
    case ECH_EUNSUPPORTED: return "unsupported key dtype or device";
    case ECH_EHIP: return "HIP launch or runtime error";
    case ECH_ESCRATCH: return "the call needs more than the static scratch array holds";
    default: return "unknown error code";
  }
}

extern "C" int ech_version(void) { return 300; }   // 3.0: the live copier takes the FINAL list too
