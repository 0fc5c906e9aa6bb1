// Host-side helpers shared by the entry points: argument checks, checked launches, the tuning
// overrides and per-device caches.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <atomic>
#include <tuple>
#include <utility>

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

// Launches kernel `k` through hipLaunchKernel and returns 0, or FP4_ERR_HIP (-6) when the runtime
// rejects this launch. The status is the launch's own return value: an error left behind by an
// earlier, unrelated HIP call is neither reported nor cleared here. Each argument is converted to
// the kernel's parameter type before its address is passed.
template <typename... P, typename... A, size_t... I>
static inline int fp4_launch_impl(void (*k)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t st,
                                  std::index_sequence<I...>, A&&... a) {
  std::tuple<P...> args(static_cast<P>(std::forward<A>(a))...);
  void* ptrs[sizeof...(P) > 0 ? sizeof...(P) : 1] = {static_cast<void*>(&std::get<I>(args))...};
  return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, ptrs, lds, st) == hipSuccess ? 0 : -6;
}

template <typename... P, typename... A>
static inline int fp4_launch(void (*k)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t st, A&&... a) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  return fp4_launch_impl(k, grid, block, lds, st, std::index_sequence_for<P...>{}, std::forward<A>(a)...);
}

// Tuning overrides, read once from the environment at the first call that needs them (a
// thread-safe static initialisation in api.hip) and fixed for the life of the process. -1 = unset.
// They exist for A/B timing and for tests that force one path; nothing sets them by default.
struct Fp4Tuning {
  int gemv_waves;      // FP4_GEMV_WAVES: 1..16 waves per GEMV workgroup
  int gemv_u;          // FP4_GEMV_U: 2..4 chunk slots per wave (M = 1)
  int gemv_one;        // FP4_GEMV_ONE=0: batch loop with prefetch instead of one batch per wave
  int gemv_ring;       // FP4_GEMV_RING=0/1: never / whenever it applies, the long-K ring kernel
  int midm_waves;      // FP4_MIDM_WAVES: waves per mid-M workgroup
  int gemm_short;      // FP4_GEMM_SHORT=0: 256-row tiles only
  int gemm_split;      // FP4_GEMM_SPLIT=0: whole K per workgroup; =1: two-set tiles split K wherever the grid allows
  int gemm_band_rows;  // FP4_GEMM_BAND_ROWS=0: 256-row tiles at M <= 192
  int gemm_narrow;     // FP4_GEMM_NARROW=0: no 128-column tiles on small grids
  int quant_exhaustive;  // FP4_QUANT_EXHAUSTIVE=1: the ROCmFP4 packer scores every candidate (no pruning)
  int one_batch;       // FP4_ONE_BATCH=0: no one-batch GEMV for 2 <= M <= 8 (batch loop, or mid-M kernel from M = 5)
  int gemm_sets;       // FP4_GEMM_SETS=1: one set of 4 waves per workgroup on 128-row small-grid tiles too
  int gemm_parts;      // FP4_GEMM_PARTS: K parts of a two-set grid with a workspace, where they fit (1: none)
};
const Fp4Tuning& fp4_tuning();

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

// Compute units of the current device (queried once per device).
int fp4_device_cus();
