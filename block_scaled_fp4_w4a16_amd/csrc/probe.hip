// Measurement probe for the benchmark (built into libfp4probe.so, separate from the library and its C
// ABI; nothing in the library calls it).
//  * fp4probe_read: a kernel that only streams `bytes` from HBM, with the GEMV's load form (16-byte
//    nontemporal buffer loads, four per lane, 256-lane workgroups, one 16 KiB slice per workgroup). Its
//    rate at a given size is the ceiling that launch cost and memory latency leave for any kernel that
//    must read those bytes once.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

constexpr int PROBE_THREADS = 256;
constexpr int PROBE_SLICE = PROBE_THREADS * 64;  // bytes per workgroup

// Workgroup b reads bytes [b * 16 KiB, (b + 1) * 16 KiB): load i of lane t at 4096 i + 16 t (each load
// instruction of a wave covers 1 KiB contiguously). Past the end the buffer loads return zeros. The XOR
// of everything read is stored only if it equals a value the data would have to be built for, so the
// loads stay and almost nothing is written.
__global__ __launch_bounds__(PROBE_THREADS) void read_probe_kernel(const uint8_t* __restrict__ p, uint64_t bytes,
                                                                   uint32_t* __restrict__ sink) {
  const uint64_t base = (uint64_t)blockIdx.x * PROBE_SLICE;
  const uint64_t left = bytes - base;
  const __amdgpu_buffer_rsrc_t r = rsrc(p + base, (uint32_t)(left < PROBE_SLICE ? left : PROBE_SLICE));
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 4096 * i + 16 * threadIdx.x, 0, 2));
  const u32x4 a = v[0] ^ v[1] ^ v[2] ^ v[3];
  const uint32_t x = a[0] ^ a[1] ^ a[2] ^ a[3];
  if (x == 0x9E3779B9u) sink[threadIdx.x] = x;
}

}  // namespace

extern "C" int fp4probe_read(const void* p, uint64_t bytes, void* sink, void* stream) {
  if (!p || !sink || bytes == 0 || ((uintptr_t)p & 15)) return -1;
  const uint64_t blocks = (bytes + PROBE_SLICE - 1) / PROBE_SLICE;
  if (blocks > 0x7fffffffULL) return -1;
  void* args[] = {&p, &bytes, &sink};
  return hipLaunchKernel(reinterpret_cast<const void*>(&read_probe_kernel), dim3((unsigned)blocks),
                         dim3(PROBE_THREADS), args, 0, (hipStream_t)stream) == hipSuccess ? 0 : -6;
}
