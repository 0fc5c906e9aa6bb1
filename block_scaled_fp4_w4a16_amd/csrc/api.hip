// Version and status strings of the C ABI, the tuning overrides and the device facts shared by the
// entry points (host only).
#include <stdint.h>
#include <stdlib.h>
#include <atomic>
#include "fp4w4a16.h"
#include "launch.h"

extern "C" int fp4_abi_version(void) { return FP4W4A16_ABI_VERSION; }

extern "C" const char* fp4_status_string(int status) {
  switch (status) {
    case FP4_OK: return "ok";
    case FP4_ERR_ARG: return "invalid argument (null pointer or unknown format)";
    case FP4_ERR_SHAPE: return "invalid shape (M, N or K out of range, or K not a multiple of the block size)";
    case FP4_ERR_ALIGN: return "misaligned pointer (planes and x need 16-byte alignment, y 4-byte)";
    case FP4_ERR_UNSUPPORTED: return "unsupported shape for this entry point";
    case FP4_ERR_INVALID_SCALE: return "invalid scale: a scale code is NaN or infinite";
    case FP4_ERR_HIP: return "the HIP runtime rejected a kernel launch or a copy";
    default: return "unknown status";
  }
}

static int env_int(const char* name) {
  const char* e = getenv(name);
  if (!e || !*e) return -1;
  return atoi(e);
}

const Fp4Tuning& fp4_tuning() {
  static const Fp4Tuning t = {env_int("FP4_GEMV_WAVES"), env_int("FP4_GEMV_U"),      env_int("FP4_GEMV_ONE"),
                              env_int("FP4_GEMV_RING"),  env_int("FP4_MIDM_WAVES"),  env_int("FP4_GEMM_SHORT"),
                              env_int("FP4_GEMM_SPLIT"), env_int("FP4_GEMM_BAND_ROWS"),
                              env_int("FP4_GEMM_NARROW"),  env_int("FP4_QUANT_EXHAUSTIVE"),
                              env_int("FP4_ONE_BATCH"),  env_int("FP4_GEMM_SETS"),   env_int("FP4_GEMM_PARTS")};
  return t;
}

int fp4_device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int c = cus[dev].load(std::memory_order_relaxed);
  if (c <= 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
    cus[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}
