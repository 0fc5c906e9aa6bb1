// Device packers: fp32 weights -> canonical packed bytes.
//
// NVFP4, data-free round-to-nearest (Nanbeige4.2-3B-NVFP4A16 card, "Creation"; EdgeRock-4B-NVFP4
// card, description): global amax -> g = fl32(amax / 2688); per 16-weight block an E4M3 scale,
// rounded to nearest-even from blockmax / (6 g) in FP64; per weight the nearest E2M1 magnitude.
//
// ROCmFP4, finite-UE4M3 MSE search (ROCmFP4 design page, section 03): for each scale group (two
// 16-weight halves for Dual, the whole block for FAST) the winner among the 127 candidate codes is the
// smallest error E(c) (FP64, terms summed in index order), ties broken by distance to the start code
// (E4M3 RNE of max|w| / 10) and then by the lower code. The default kernel runs one thread per block and
// visits the candidates outward from the start with safe pruning (below); the exhaustive kernel (one wave
// per block, the 64 lanes scoring two candidates each, then a wave reduction) is kept for comparison.
//
// Q4_0, signed abs-max (ROCmFP4 design page, comparison table, stock Q4_0 reference scale): one thread
// per 32-weight block; m = the first weight of largest magnitude, d = m / -8 (exact), stored as FP16
// (RNE); each code is floor(w / d + 8.5) clipped to 0..15, computed in FP64 with the unrounded d.
//
// Every FP64 operation here is a separately rounded IEEE operation: contraction into fused
// multiply-adds is switched off for this file, so the chosen codes do not depend on it.
#include "common.h"
#include "launch.h"
#include "fp4w4a16.h"

#pragma clang fp contract(off)

namespace fp4 {

// Nearest finite E4M3 code of v >= 0, ties to the even code, saturating at 0x7E (448).
__device__ __forceinline__ int e4m3_rne(double v) {
  if (!(v > 0.0)) return 0;
  if (v >= 448.0) return 126;
  if (v < 0.015625) {  // below 2^-6 the grid is k * 2^-9; code k (k = 8 is 2^-6, the first normal)
    return (int)rint(v * 512.0);
  }
  int e;
  const double f = frexp(v, &e);                  // v = f 2^e, f in [0.5, 1)
  const int code = (e + 6) * 8 + (int)rint(16.0 * f - 8.0);  // exponent field e + 6, mantissa m
  return code > 126 ? 126 : code;
}

// Value of a finite non-negative E4M3 / UE4M3 code (0..126), exact.
__device__ __forceinline__ double e4m3_value(int c) {
  const int e = c >> 3, m = c & 7;
  return e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
}

// ---------------------------------------------------------------- NVFP4
__global__ void nvfp4_zero_kernel(float* g) { g[0] = 0.f; }

__global__ void nvfp4_amax_kernel(const float* __restrict__ w, int64_t count, float* g) {
  float a = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x)
    a = fmaxf(a, fabsf(w[i]));
  for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  if ((threadIdx.x & 63) == 0) atomicMax(reinterpret_cast<unsigned int*>(g), __float_as_uint(a));
}

// the global scale from amax: fl32(amax / 2688), or 0 when that is not positive
__device__ __forceinline__ float nvfp4_global(float amax) {
  return amax > 0.f ? (float)((double)amax / 2688.0) : 0.f;
}

// one thread per 16-weight block
__global__ void nvfp4_pack_kernel(const float* __restrict__ w, int64_t nblocks, const float* __restrict__ gbuf,
                                  uint8_t* __restrict__ wq, uint8_t* __restrict__ ws) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const float g = nvfp4_global(gbuf[0]);
  float v[16];
  const f32x4* src = reinterpret_cast<const f32x4*>(w + b * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 t = src[i];
    v[4 * i] = t[0]; v[4 * i + 1] = t[1]; v[4 * i + 2] = t[2]; v[4 * i + 3] = t[3];
  }
  uint8_t codes[16];
  uint8_t sc = 0;
  if (g > 0.f) {
    double a = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmax(a, fabs((double)v[i]));
    sc = (uint8_t)e4m3_rne(a / (6.0 * (double)g));
    const double d = e4m3_value(sc) * (double)g;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const double x = fabs((double)v[i]);
      int c = 0;
      if (d > 0.0) {
        // E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6: midpoints .25 .75 1.25 1.75 2.5 3.5 5
        const double mid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
#pragma unroll
        for (int j = 0; j < 7; ++j) c += (x > mid[j] * d) ? 1 : 0;
        if (c < 7 && (c & 1) && x == mid[c] * d) ++c;   // exact tie -> even code
      }
      codes[i] = (uint8_t)(c | ((v[i] < 0.f && c != 0) ? 8 : 0));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) codes[i] = 0;
  }
  u32x2 packed = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) packed[i >> 2] |= (uint32_t)(codes[2 * i] | (codes[2 * i + 1] << 4)) << (8 * (i & 3));
  *reinterpret_cast<u32x2*>(wq + b * 8) = packed;
  ws[b] = sc;
}

__global__ void nvfp4_finish_kernel(float* g) {
  const float gg = nvfp4_global(g[0]);
  g[0] = gg > 0.f ? gg : 1.0f;
}

// ---------------------------------------------------------------- ROCmFP4
// Codebook10 magnitude code of a / s: count midpoints * s below a, exact ties to the even code.
__device__ __forceinline__ int cb10_nearest(double a, double s) {
  if (s == 0.0) return 0;
  const double mid[7] = {0.5, 1.5, 2.5, 3.5, 5.0, 7.0, 9.0};
  int c = 0;
#pragma unroll
  for (int j = 0; j < 7; ++j) c += (a > mid[j] * s) ? 1 : 0;
  if (c < 7 && (c & 1) && a == mid[c] * s) ++c;
  return c;
}

__device__ __forceinline__ double cb10_level(int c) {
  return c < 5 ? (double)c : (c == 5 ? 6.0 : (c == 6 ? 8.0 : 10.0));
}

template <int G>
__device__ __forceinline__ double group_error(const float* wv, const float* iv, double s) {
  double e = 0.0;
  for (int i = 0; i < G; ++i) {
    const double a = fabs((double)wv[i]);
    const double dlt = a - cb10_level(cb10_nearest(a, s)) * s;
    double t = dlt * dlt;
    if (iv) t = (double)iv[i] * t;
    e = e + t;
  }
  return e;
}

// a better than b in the order (error, |code - start|, code)
__device__ __forceinline__ bool better(double ea, int ca, double eb, int cb, int start) {
  if (ea != eb) return ea < eb;
  const int da = abs(ca - start), db = abs(cb - start);
  if (da != db) return da < db;
  return ca < cb;
}

template <int G>
__device__ int search_group(const float* wv, const float* iv, int lane) {
  double amax = 0.0;
  for (int i = 0; i < G; ++i) amax = fmax(amax, fabs((double)wv[i]));
  const int start = e4m3_rne(fmin(amax / 10.0, 448.0));
  int bc = lane;
  double be = group_error<G>(wv, iv, e4m3_value(lane));
  if (lane + 64 < 127) {
    const int c2 = lane + 64;
    const double e2 = group_error<G>(wv, iv, e4m3_value(c2));
    if (better(e2, c2, be, bc, start)) { be = e2; bc = c2; }
  }
  for (int off = 32; off > 0; off >>= 1) {
    const double oe = __shfl_xor(be, off);
    const int oc = __shfl_xor(bc, off);
    if (better(oe, oc, be, bc, start)) { be = oe; bc = oc; }
  }
  return bc;
}

// Safe pruning (ROCmFP4 design page, section 03: pruning may only skip work that cannot change the selected
// scale). Two lower bounds of E(c), each a sum of some of E(c)'s own terms, computed with E's operations in
// E's order (so each is <= the computed E(c)), and each only growing as the scale moves away from the start:
//  * smaller scales: every weight with |w| > 10 s takes level 10, term v (|w| - 10 s)^2 -- more such weights,
//    each with a larger term, as s falls;
//  * larger scales: every weight with |w| <= s / 2 takes level 0, term v w^2 -- more such weights as s grows.
// Candidates are visited outward from the start code (distance d = 1, 2, ...; the lower code first). A
// candidate visited later can only replace the best one with a strictly smaller error (it is not nearer to
// the start, and at equal distance not lower), so once a direction's bound reaches the best error no code in
// that direction can win and the direction is dropped. The winner is the exhaustive search's. Pruning is off
// (every candidate scored) for groups with a non-finite weight or an importance that is negative or NaN.
template <int G>
__device__ __forceinline__ double bound_down(const float* wv, const float* iv, double s) {
  double e = 0.0;
  for (int i = 0; i < G; ++i) {
    const double a = fabs((double)wv[i]);
    if (a > 10.0 * s) {
      const double dlt = a - 10.0 * s;
      double t = dlt * dlt;
      if (iv) t = (double)iv[i] * t;
      e = e + t;
    }
  }
  return e;
}

template <int G>
__device__ __forceinline__ double bound_up(const float* wv, const float* iv, double s) {
  double e = 0.0;
  for (int i = 0; i < G; ++i) {
    const double a = fabs((double)wv[i]);
    if (a <= 0.5 * s) {
      const double dlt = a - 0.0 * s;
      double t = dlt * dlt;
      if (iv) t = (double)iv[i] * t;
      e = e + t;
    }
  }
  return e;
}

template <int G>
__device__ int search_group_pruned(const float* wv, const float* iv) {
  double amax = 0.0;
  bool prune = true;
  for (int i = 0; i < G; ++i) {
    amax = fmax(amax, fabs((double)wv[i]));
    if (!(fabs((double)wv[i]) <= 1.0e308)) prune = false;
    if (iv && !(iv[i] >= 0.f)) prune = false;
  }
  const int start = e4m3_rne(fmin(amax / 10.0, 448.0));
  int bc = start;
  double be = group_error<G>(wv, iv, e4m3_value(start));
  bool down = true, up = true;
  for (int d = 1; d <= 126 && (down || up); ++d) {
    if (down) {
      const int c = start - d;
      if (c < 0) {
        down = false;
      } else {
        const double sc = e4m3_value(c);
        if (prune && bound_down<G>(wv, iv, sc) >= be) {
          down = false;
        } else {
          const double e = group_error<G>(wv, iv, sc);
          if (better(e, c, be, bc, start)) { be = e; bc = c; }
        }
      }
    }
    if (up) {
      const int c = start + d;
      if (c > 126) {
        up = false;
      } else {
        const double sc = e4m3_value(c);
        if (prune && bound_up<G>(wv, iv, sc) >= be) {
          up = false;
        } else {
          const double e = group_error<G>(wv, iv, sc);
          if (better(e, c, be, bc, start)) { be = e; bc = c; }
        }
      }
    }
  }
  return bc;
}

// the block's packed bytes from its scale codes
template <int F>
__device__ __forceinline__ void rocm_write_block(uint8_t* ob, const float* wv, const int (&sc)[2], int j) {
  constexpr int NS = (F == DUAL) ? 2 : 1;
  const double s_lo = e4m3_value(sc[0]), s_hi = e4m3_value(sc[1]);
  const int c_lo = cb10_nearest(fabs((double)wv[j]), s_lo);
  const int c_hi = cb10_nearest(fabs((double)wv[j + 16]), s_hi);
  const int n_lo = c_lo | ((wv[j] < 0.f && c_lo) ? 8 : 0);
  const int n_hi = c_hi | ((wv[j + 16] < 0.f && c_hi) ? 8 : 0);
  ob[NS + j] = (uint8_t)(n_lo | (n_hi << 4));
}

// one thread per 32-weight block, pruned search
template <int F>
__global__ __launch_bounds__(256) void rocm_pack_pruned_kernel(const float* __restrict__ w, const float* __restrict__ imp,
                                                               int64_t nblocks, uint8_t* __restrict__ out) {
  const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= nblocks) return;
  float wv[32], iv[32];
  const f32x4* src = reinterpret_cast<const f32x4*>(w + blk * 32);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const f32x4 t = src[i];
    wv[4 * i] = t[0]; wv[4 * i + 1] = t[1]; wv[4 * i + 2] = t[2]; wv[4 * i + 3] = t[3];
  }
  if (imp) {
    const f32x4* isrc = reinterpret_cast<const f32x4*>(imp + blk * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x4 t = isrc[i];
      iv[4 * i] = t[0]; iv[4 * i + 1] = t[1]; iv[4 * i + 2] = t[2]; iv[4 * i + 3] = t[3];
    }
  }
  constexpr int BB = (F == DUAL) ? 18 : 17;
  int sc[2];
  if constexpr (F == DUAL) {
    sc[0] = search_group_pruned<16>(wv, imp ? iv : nullptr);
    sc[1] = search_group_pruned<16>(wv + 16, imp ? iv + 16 : nullptr);
  } else {
    sc[0] = search_group_pruned<32>(wv, imp ? iv : nullptr);
    sc[1] = sc[0];
  }
  uint8_t* ob = out + blk * BB;
  ob[0] = (uint8_t)sc[0];
  if (F == DUAL) ob[1] = (uint8_t)sc[1];
  for (int j = 0; j < 16; ++j) rocm_write_block<F>(ob, wv, sc, j);
}

// one wave (64 threads) per 32-weight block, every candidate scored (two per lane)
template <int F>
__global__ __launch_bounds__(256) void rocm_pack_kernel(const float* __restrict__ w, const float* __restrict__ imp,
                                                        int64_t nblocks, uint8_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  if (blk >= nblocks) return;
  float wv[32], iv[32];
  const f32x4* src = reinterpret_cast<const f32x4*>(w + blk * 32);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const f32x4 t = src[i];
    wv[4 * i] = t[0]; wv[4 * i + 1] = t[1]; wv[4 * i + 2] = t[2]; wv[4 * i + 3] = t[3];
  }
  if (imp) {
    const f32x4* isrc = reinterpret_cast<const f32x4*>(imp + blk * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x4 t = isrc[i];
      iv[4 * i] = t[0]; iv[4 * i + 1] = t[1]; iv[4 * i + 2] = t[2]; iv[4 * i + 3] = t[3];
    }
  }
  constexpr int BB = (F == DUAL) ? 18 : 17, NS = (F == DUAL) ? 2 : 1;
  int sc[2];
  if constexpr (F == DUAL) {
    sc[0] = search_group<16>(wv, imp ? iv : nullptr, lane);
    sc[1] = search_group<16>(wv + 16, imp ? iv + 16 : nullptr, lane);
  } else {
    sc[0] = search_group<32>(wv, imp ? iv : nullptr, lane);
    sc[1] = sc[0];
  }
  uint8_t* ob = out + blk * BB;
  if (lane < 16) rocm_write_block<F>(ob, wv, sc, lane);
  if (lane == 0) {
    ob[0] = (uint8_t)sc[0];
    if (NS == 2) ob[1] = (uint8_t)sc[1];
  }
}

__global__ void q4_0_pack_kernel(const float* __restrict__ w, int64_t nblocks, uint8_t* __restrict__ out) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const float* wb = w + b * 32;
  float m = 0.f, am = 0.f;
  for (int i = 0; i < 32; ++i) {       // first weight of the largest magnitude, sign kept
    const float a = fabsf(wb[i]);
    if (a > am) {
      am = a;
      m = wb[i];
    }
  }
  const float d = m * -0.125f + 0.0f;  // m / -8, exact; an all-zero block gives +0
  const _Float16 d16 = (_Float16)d;    // round to nearest even
  const uint16_t hb = __builtin_bit_cast(uint16_t, d16);
  uint8_t* ob = out + b * 18;
  ob[0] = (uint8_t)(hb & 0xFF);
  ob[1] = (uint8_t)(hb >> 8);
  uint8_t q[32];
  for (int i = 0; i < 32; ++i) {
    int c = 8;
    if (d != 0.f) {
      const double t = floor((double)wb[i] / (double)d + 8.5);
      c = t < 0.0 ? 0 : t > 15.0 ? 15 : (int)t;
    }
    q[i] = (uint8_t)c;
  }
  for (int j = 0; j < 16; ++j) ob[2 + j] = (uint8_t)(q[j] | (q[j + 16] << 4));
}

}  // namespace fp4

using namespace fp4;

extern "C" int fp4_quantize_nvfp4(int64_t N, int64_t K, const float* w, void* wq, void* ws, float* g_out,
                                  void* stream) {
  if (!w || !wq || !ws || !g_out) return -1;
  int rc = fp4_check_nk(NVFP4, N, K);
  if (rc) return rc;
  if (!fp4_aligned(w, 16) || !fp4_aligned(wq, 8) || !fp4_aligned(g_out, 4)) return -3;
  hipStream_t st = (hipStream_t)stream;
  const int64_t count = N * K, nblocks = count / 16;
  rc = fp4_launch(nvfp4_zero_kernel, dim3(1), dim3(1), 0, st, g_out);
  if (rc) return rc;
  int grid = (int)((count + 255) / 256);
  if (grid > 4096) grid = 4096;
  rc = fp4_launch(nvfp4_amax_kernel, dim3(grid), dim3(256), 0, st, w, count, g_out);
  if (rc) return rc;
  rc = fp4_launch(nvfp4_pack_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, st, w, nblocks,
                  (const float*)g_out, (uint8_t*)wq, (uint8_t*)ws);
  if (rc) return rc;
  return fp4_launch(nvfp4_finish_kernel, dim3(1), dim3(1), 0, st, g_out);
}

extern "C" int fp4_quantize_rocmfp4(int fmt, int64_t N, int64_t K, const float* w, const float* importance,
                                    void* blocks, void* stream) {
  if ((fmt != DUAL && fmt != FAST) || !w || !blocks) return -1;
  int rc = fp4_check_nk(fmt, N, K);
  if (rc) return rc;
  if (!fp4_aligned(w, 16) || (importance && !fp4_aligned(importance, 16))) return -3;
  hipStream_t st = (hipStream_t)stream;
  const int64_t nblocks = N * K / 32;
  const int64_t grid = (nblocks * 64 + 255) / 256;
  if (grid > 0x7fffffffLL) return -4;
  uint8_t* ob = (uint8_t*)blocks;
  if (fp4_tuning().quant_exhaustive == 1) {  // tuning override: every candidate of every group scored
    if (fmt == DUAL) return fp4_launch(rocm_pack_kernel<DUAL>, dim3((unsigned)grid), dim3(256), 0, st, w, importance, nblocks, ob);
    return fp4_launch(rocm_pack_kernel<FAST>, dim3((unsigned)grid), dim3(256), 0, st, w, importance, nblocks, ob);
  }
  const dim3 pg((unsigned)((nblocks + 255) / 256));
  if (fmt == DUAL) return fp4_launch(rocm_pack_pruned_kernel<DUAL>, pg, dim3(256), 0, st, w, importance, nblocks, ob);
  return fp4_launch(rocm_pack_pruned_kernel<FAST>, pg, dim3(256), 0, st, w, importance, nblocks, ob);
}

extern "C" int fp4_quantize_q4_0(int64_t N, int64_t K, const float* w, void* blocks, void* stream) {
  if (!w || !blocks) return -1;
  int rc = fp4_check_nk(Q4_0, N, K);
  if (rc) return rc;
  if (!fp4_aligned(w, 16)) return -3;
  const int64_t nblocks = N * K / 32;
  const int64_t grid = (nblocks + 255) / 256;
  if (grid > 0x7fffffffLL) return -4;
  return fp4_launch(q4_0_pack_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, w, nblocks,
                    (uint8_t*)blocks);
}
