// Load-time repack (canonical -> kernel layout) and the FP32 dequantizer of the kernel layout.
#include "common.h"
#include "launch.h"
#include "fp4w4a16.h"
#include <atomic>
#include <mutex>

namespace fp4 {

// One thread per 16-byte lane piece of the nibble plane, plus the scale bytes of its row.
template <int F>
__global__ void pack_layout_kernel(int N, int K, int nchunk, int64_t npieces,
                                   const uint8_t* __restrict__ src_q, const uint8_t* __restrict__ src_s,
                                   uint8_t* __restrict__ dst_q, uint8_t* __restrict__ dst_s) {
  int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= npieces) return;
  const int lane = (int)(p & 63);
  const int64_t unit = p >> 6;            // tile * nchunk + chunk
  const int chunk = (int)(unit % nchunk);
  const int64_t tile = unit / nchunk;
  const int n = lane & 15, g = lane >> 4;
  const int64_t row = tile * TILE_N + n;
  const bool row_ok = row < N;

  uint8_t out[16];
#pragma unroll
  for (int b = 0; b < 16; ++b) out[b] = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int k = chunk * CHUNK_K + kmap(F, g, i);
    uint32_t code = 0;
    if (row_ok && k < K) {
      if (F == NVFP4) {
        uint8_t b = src_q[row * (K / 2) + k / 2];
        code = (k & 1) ? (b >> 4) : (b & 15);
      } else {
        // the nibble bytes follow the block's scale field: 2 bytes (Dual, Q4_0) or 1 (FAST)
        const int bb = (F == FAST) ? 17 : 18, ns = (F == FAST) ? 1 : 2;
        const int blk = k >> 5, j = k & 31;
        uint8_t b = src_q[(row * (K / 32) + blk) * bb + ns + (j & 15)];
        code = (j >= 16) ? (b >> 4) : (b & 15);
      }
    }
    out[nib_byte(F, i)] |= (uint8_t)(code << (4 * nib_high(F, i)));
  }
  u32x4 v;
  __builtin_memcpy(&v, out, 16);
  *reinterpret_cast<u32x4*>(dst_q + p * 16) = v;

  // lane group 0 writes this row's scale bytes for the chunk
  if (g == 0) {
    constexpr int sbytes = scale_bytes_row_chunk(F);
    uint8_t sb[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < scales_per_row_chunk(F); ++j) {
      const int k0 = chunk * CHUNK_K + j * group_size(F);
      if (row_ok && k0 < K) {
        if (F == NVFP4) {
          sb[j] = src_s[row * (K / 16) + k0 / 16];
        } else if (F == DUAL) {
          sb[j] = src_q[(row * (K / 32) + (k0 >> 5)) * 18 + ((k0 >> 4) & 1)] & 0x7F;
        } else if (F == FAST) {
          sb[j] = src_q[(row * (K / 32) + (k0 >> 5)) * 17] & 0x7F;
        } else {  // Q4_0: the FP16 scale, little-endian
          sb[2 * j] = src_q[(row * (K / 32) + (k0 >> 5)) * 18];
          sb[2 * j + 1] = src_q[(row * (K / 32) + (k0 >> 5)) * 18 + 1];
        }
      }
    }
    uint8_t* d = dst_s + unit * unit_s(F) + n * sbytes;
#pragma unroll
    for (int j = 0; j < sbytes; ++j) d[j] = sb[j];
  }
}

template <int F>
__device__ __forceinline__ float level_of(uint32_t code) {
  if (F == Q4_0) return (float)((int)code - 8);
  const uint32_t m = code & 7;
  float mag;
  if (F == NVFP4)  // E2M1: 0, .5, 1, 1.5, then 2, 3, 4, 6 = 2^((m>>1)-1) * (1 or 1.5)
    mag = m < 4 ? 0.5f * (float)m : (float)((1u << (m >> 1)) >> 1) * ((m & 1) ? 1.5f : 1.0f);
  else             // Codebook10: 0, 1, 2, 3, 4, 6, 8, 10
    mag = m < 5 ? (float)m : (float)(m == 5 ? 6 : m == 6 ? 8 : 10);
  return (code & 8) ? -mag : mag;
}

// One thread per 16-byte lane piece: 32 weights -> fl32(fl32(level*scale)*g).
template <int F>
__global__ void dequant_kernel(int N, int K, int nchunk, int64_t npieces, const uint8_t* __restrict__ q,
                               const uint8_t* __restrict__ s, float gscale, float* __restrict__ w) {
  int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= npieces) return;
  const int lane = (int)(p & 63);
  const int64_t unit = p >> 6;
  const int chunk = (int)(unit % nchunk);
  const int64_t tile = unit / nchunk;
  const int n = lane & 15, g = lane >> 4;
  const int64_t row = tile * TILE_N + n;
  if (row >= N) return;
  const u32x4 qv = *reinterpret_cast<const u32x4*>(q + p * 16);
  uint8_t qb[16];
  __builtin_memcpy(qb, &qv, 16);
  const uint8_t* srow = s + unit * unit_s(F) + n * scale_bytes_row_chunk(F);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int kk = kmap(F, g, i);
    const int k = chunk * CHUNK_K + kk;
    if (k >= K) continue;
    const uint32_t code = (qb[nib_byte(F, i)] >> (4 * nib_high(F, i))) & 15u;
    const float level = level_of<F>(code);
    const int j = kk / group_size(F);
    float sc;
    if (F == Q4_0) {
      const uint16_t hb = (uint16_t)(srow[2 * j] | (srow[2 * j + 1] << 8));
      sc = (float)__builtin_bit_cast(_Float16, hb);
    } else {
      sc = __builtin_amdgcn_cvt_f32_fp8(srow[j], 0);
    }
    const float prod = level * sc;  // exact: at most 3 + 4 (or, for Q4_0, 4 + 11) significant bits
    w[row * (int64_t)K + k] = prod * gscale;
  }
}

// Scale validation (fp4_pack_layout with validate != 0): one thread per scale of the canonical input.
// A NaN E4M3 / UE4M3 code (low 7 bits all ones; UE4M3's bit 7 is ignored as on decode) or a Q4_0 FP16
// scale with an all-ones exponent sets *bad. Every writer stores the same value, so the races are benign.
template <int F>
__global__ void validate_scales_kernel(int64_t nscales, const uint8_t* __restrict__ src_q,
                                       const uint8_t* __restrict__ src_s, unsigned int* __restrict__ bad) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nscales; i += (int64_t)gridDim.x * blockDim.x) {
    bool nonfinite;
    if (F == NVFP4) {
      nonfinite = (src_s[i] & 0x7F) == 0x7F;
    } else if (F == DUAL) {           // two scale bytes at the head of each 18-byte block
      nonfinite = (src_q[(i >> 1) * 18 + (i & 1)] & 0x7F) == 0x7F;
    } else if (F == FAST) {           // one scale byte at the head of each 17-byte block
      nonfinite = (src_q[i * 17] & 0x7F) == 0x7F;
    } else {                          // Q4_0: FP16 scale, little-endian, at the head of each 18-byte block
      const unsigned hi = src_q[i * 18 + 1];
      nonfinite = ((hi >> 2) & 31) == 31;
    }
    if (nonfinite) *bad = 1u;
  }
}

__global__ void clear_word_kernel(unsigned int* w) { *w = 0u; }

// One 4-byte word per device for the validation result. In host code `fp4_bad_scale_word` is only a
// stand-in for the symbol: its device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned int fp4_bad_scale_word;

}  // namespace fp4

using namespace fp4;

namespace {
std::mutex g_validate_lock[64];
std::atomic<unsigned int*> g_validate_word[64];

// The device address of the validation word on the current device (or nullptr).
unsigned int* validate_word(int dev) {
  unsigned int* p = g_validate_word[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* a = nullptr;
  if (hipGetSymbolAddress(&a, HIP_SYMBOL(fp4::fp4_bad_scale_word)) != hipSuccess || !a) return nullptr;
  p = static_cast<unsigned int*>(a);
  g_validate_word[dev].store(p, std::memory_order_release);
  return p;
}

template <int F>
int validate_scales(int64_t N, int64_t K, const uint8_t* sq, const uint8_t* ss, hipStream_t st) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -6;
  std::lock_guard<std::mutex> guard(g_validate_lock[dev]);
  unsigned int* word = validate_word(dev);
  if (!word) return -6;
  const int64_t nscales = (F == NVFP4) ? N * (K / 16) : (F == DUAL ? 2 : 1) * N * (K / 32);
  const int threads = 256;
  const int64_t want = (nscales + threads - 1) / threads;
  const unsigned blocks = (unsigned)(want < 4096 ? (want > 0 ? want : 1) : 4096);
  int rc = fp4_launch(clear_word_kernel, dim3(1), dim3(1), 0, st, word);
  if (rc) return rc;
  rc = fp4_launch(validate_scales_kernel<F>, dim3(blocks), dim3(threads), 0, st, nscales, sq, ss, word);
  if (rc) return rc;
  unsigned int host = 0;
  if (hipMemcpyAsync(&host, word, sizeof(host), hipMemcpyDeviceToHost, st) != hipSuccess) return -6;
  if (hipStreamSynchronize(st) != hipSuccess) return -6;
  return host ? -5 : 0;
}
}  // namespace

extern "C" int fp4_layout_bytes(int fmt, int64_t N, int64_t K, size_t* q_bytes, size_t* s_bytes) {
  if (!fp4_valid_format(fmt) || !q_bytes || !s_bytes) return -1;
  int rc = fp4_check_nk(fmt, N, K);
  if (rc) return rc;
  const int64_t tiles = (N + TILE_N - 1) / TILE_N, nchunk = (K + CHUNK_K - 1) / CHUNK_K;
  *q_bytes = (size_t)(tiles * nchunk * UNIT_Q);
  *s_bytes = (size_t)(tiles * nchunk * unit_s(fmt));
  return 0;
}

extern "C" int fp4_pack_layout(int fmt, int64_t N, int64_t K, const void* src_q, const void* src_s,
                               void* dst_q, void* dst_s, int validate, void* stream) {
  if (!fp4_valid_format(fmt) || !src_q || !dst_q || !dst_s) return -1;
  if (fmt == NVFP4 && !src_s) return -1;
  if (fmt != NVFP4 && src_s) return -1;
  int rc = fp4_check_nk(fmt, N, K);
  if (rc) return rc;
  if (!fp4_aligned(dst_q, 16) || !fp4_aligned(dst_s, 16)) return -3;
  const int64_t tiles = (N + TILE_N - 1) / TILE_N;
  const int nchunk = (int)((K + CHUNK_K - 1) / CHUNK_K);
  const int64_t npieces = tiles * nchunk * 64;
  const int threads = 256;
  const int64_t blocks = (npieces + threads - 1) / threads;
  if (blocks > 0x7fffffffLL) return -4;
  hipStream_t st = (hipStream_t)stream;
  const uint8_t* sq = (const uint8_t*)src_q;
  const uint8_t* ss = (const uint8_t*)src_s;
  uint8_t* dq = (uint8_t*)dst_q;
  uint8_t* ds = (uint8_t*)dst_s;
  if (validate) {
    switch (fmt) {
      case NVFP4: rc = validate_scales<NVFP4>(N, K, sq, ss, st); break;
      case DUAL:  rc = validate_scales<DUAL>(N, K, sq, ss, st); break;
      case FAST:  rc = validate_scales<FAST>(N, K, sq, ss, st); break;
      default:    rc = validate_scales<Q4_0>(N, K, sq, ss, st); break;
    }
    if (rc) return rc;
  }
  const dim3 grid((unsigned)blocks), block(threads);
  switch (fmt) {
    case NVFP4: return fp4_launch(pack_layout_kernel<NVFP4>, grid, block, 0, st, (int)N, (int)K, nchunk, npieces, sq, ss, dq, ds);
    case DUAL:  return fp4_launch(pack_layout_kernel<DUAL>, grid, block, 0, st, (int)N, (int)K, nchunk, npieces, sq, ss, dq, ds);
    case FAST:  return fp4_launch(pack_layout_kernel<FAST>, grid, block, 0, st, (int)N, (int)K, nchunk, npieces, sq, ss, dq, ds);
    default:    return fp4_launch(pack_layout_kernel<Q4_0>, grid, block, 0, st, (int)N, (int)K, nchunk, npieces, sq, ss, dq, ds);
  }
}

extern "C" int fp4_dequant_f32(int fmt, int64_t N, int64_t K, const void* q, const void* s, float global_scale,
                               float* w, void* stream) {
  if (!fp4_valid_format(fmt) || !q || !s || !w) return -1;
  int rc = fp4_check_nk(fmt, N, K);
  if (rc) return rc;
  if (!fp4_aligned(q, 16) || !fp4_aligned(s, 16) || !fp4_aligned(w, 4)) return -3;
  const int64_t tiles = (N + TILE_N - 1) / TILE_N;
  const int nchunk = (int)((K + CHUNK_K - 1) / CHUNK_K);
  const int64_t npieces = tiles * nchunk * 64;
  const int threads = 256;
  const int64_t blocks = (npieces + threads - 1) / threads;
  if (blocks > 0x7fffffffLL) return -4;
  hipStream_t st = (hipStream_t)stream;
  const uint8_t* qq = (const uint8_t*)q;
  const uint8_t* sp = (const uint8_t*)s;
  const dim3 grid((unsigned)blocks), block(threads);
  switch (fmt) {
    case NVFP4: return fp4_launch(dequant_kernel<NVFP4>, grid, block, 0, st, (int)N, (int)K, nchunk, npieces, qq, sp, global_scale, w);
    case DUAL:  return fp4_launch(dequant_kernel<DUAL>, grid, block, 0, st, (int)N, (int)K, nchunk, npieces, qq, sp, global_scale, w);
    case FAST:  return fp4_launch(dequant_kernel<FAST>, grid, block, 0, st, (int)N, (int)K, nchunk, npieces, qq, sp, global_scale, w);
    default:    return fp4_launch(dequant_kernel<Q4_0>, grid, block, 0, st, (int)N, (int)K, nchunk, npieces, qq, sp, global_scale, w);
  }
}
