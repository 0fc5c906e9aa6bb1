// Host-side argument checks shared by the entry points.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <atomic>

static inline bool fp4_valid_format(int f) { return f >= 1 && f <= 4; }

static inline bool fp4_aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// N, K checks common to every entry point: returns 0 or a negative status.
static inline int fp4_check_nk(int fmt, int64_t N, int64_t K) {
  if (N < 1 || K < 1) return -2;
  if (N > (1LL << 30) || K > (1LL << 30)) return -4;
  const int64_t kmul = (fmt == 1) ? 16 : 32;
  if (K % kmul) return -2;
  return 0;
}

// Launch status of the last kernel enqueued by this thread.
static inline int fp4_launch_status() { return hipGetLastError() == hipSuccess ? 0 : -6; }

// A kernel's dynamic-LDS limit raised to `bytes` once per device: the attribute is set for the device
// current at the call, so a process that launches on several GPUs needs it on each. One static object
// per kernel instantiation; a race only repeats the call.
struct Fp4LdsLimit {
  std::atomic<int> done[64];
  void ensure(const void* fn, int bytes) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
      (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
      return;
    }
    if (done[dev].load(std::memory_order_acquire)) return;
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess)
      done[dev].store(1, std::memory_order_release);
  }
};
