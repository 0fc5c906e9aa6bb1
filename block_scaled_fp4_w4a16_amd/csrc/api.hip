// Version and status strings of the C ABI (host only).
#include <stdint.h>
#include "fp4w4a16.h"

extern "C" int fp4_abi_version(void) { return FP4W4A16_ABI_VERSION; }

extern "C" const char* fp4_status_string(int status) {
  switch (status) {
    case FP4_OK: return "ok";
    case FP4_ERR_ARG: return "invalid argument (null pointer or unknown format)";
    case FP4_ERR_SHAPE: return "invalid shape (M, N or K out of range, or K not a multiple of the block size)";
    case FP4_ERR_ALIGN: return "misaligned pointer (planes and x need 16-byte alignment, y 4-byte)";
    case FP4_ERR_UNSUPPORTED: return "unsupported shape for this entry point";
    case FP4_ERR_HIP: return "the HIP runtime rejected a kernel launch";
    default: return "unknown status";
  }
}
