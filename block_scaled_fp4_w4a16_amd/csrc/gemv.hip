// Decode-shaped W4A16 product (1 <= M <= 16).
//
// One workgroup owns T consecutive 16-row tiles of W and the whole K range; its W waves
// split the 128-wide K chunks (wave w takes chunks w, w + W, ...). Per chunk a lane loads
// 16 bytes of nibbles per tile (row n = lane % 16, lane group g = lane / 16) and the row's
// scale bytes, decodes to exact bf16 levels and issues one MFMA per scale group:
//   A = x fragment (row m = lane % 16, zero for m >= M), B = unscaled levels, C = 0,
// then folds the group scale into FP32: acc += scale * C. The waves' partial sums are
// reduced through LDS in a fixed order, multiplied by the global scale and stored.
#include "common.h"
#include "launch.h"
#include "fp4w4a16.h"
#include <stdlib.h>

namespace fp4 {


template <int F>
struct WeightRegs {
  u32x4 q;
  uint32_t s[F == FAST ? 1 : 2];
};

template <int F>
__device__ __forceinline__ void load_unit(WeightRegs<F>& r, const uint8_t* __restrict__ qp,
                                          const uint8_t* __restrict__ sp, int64_t unit, int lane, int n) {
  r.q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qp + unit * UNIT_Q + lane * 16));
  if constexpr (F == FAST) {
    r.s[0] = *reinterpret_cast<const uint32_t*>(sp + unit * unit_s(F) + n * 4);
  } else {
    const u32x2 v = *reinterpret_cast<const u32x2*>(sp + unit * unit_s(F) + n * 8);
    r.s[0] = v[0];
    r.s[1] = v[1];
  }
}

// acc[r] += scale * (x_frag . levels) for one scale group; RU = rows of C in use.
template <int RU>
__device__ __forceinline__ void fold(f32x4& acc, const f32x4& p, float sc) {
#pragma unroll
  for (int r = 0; r < RU; ++r) acc[r] = __builtin_fmaf(sc, p[r], acc[r]);
}

template <int F, int RU>
__device__ __forceinline__ void unit_mac(f32x4& acc, const WeightRegs<F>& w, const void* xa) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  if constexpr (F == NVFP4) {
    const bf16x4* xf = reinterpret_cast<const bf16x4*>(xa);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t word = w.q[d];
      // MFMA 2d uses bytes 0,1 of the dword; MFMA 2d+1 uses bytes 2,3
      const bf16x4 b0 = cat(e2m1x2_to_bf16<0>(word), e2m1x2_to_bf16<1>(word));
      const bf16x4 b1 = cat(e2m1x2_to_bf16<2>(word), e2m1x2_to_bf16<3>(word));
      const f32x4 p0 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xf[2 * d], b0, zero, 0, 0, 0);
      const f32x4 p1 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xf[2 * d + 1], b1, zero, 0, 0, 0);
      // the two scale bytes of groups 2d and 2d+1, converted together
      const f32x2 sc = (d & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(w.s[d >> 1], true)
                               : __builtin_amdgcn_cvt_pk_f32_fp8(w.s[d >> 1], false);
      const float sc0 = sc[0], sc1 = sc[1];
      fold<RU>(acc, p0, sc0);
      fold<RU>(acc, p1, sc1);
    }
  } else if constexpr (F == DUAL) {
    const bf16x4* xf = reinterpret_cast<const bf16x4*>(xa);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t lo, hi;
      cb10_to_e4m3(w.q[d], lo, hi);
      const bf16x4 b0 = cat(e4m3x2_to_bf16<false>(lo), e4m3x2_to_bf16<true>(lo));
      const bf16x4 b1 = cat(e4m3x2_to_bf16<false>(hi), e4m3x2_to_bf16<true>(hi));
      const f32x4 p0 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xf[2 * d], b0, zero, 0, 0, 0);
      const f32x4 p1 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xf[2 * d + 1], b1, zero, 0, 0, 0);
      // the two scale bytes of groups 2d and 2d+1, converted together
      const f32x2 sc = (d & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(w.s[d >> 1], true)
                               : __builtin_amdgcn_cvt_pk_f32_fp8(w.s[d >> 1], false);
      const float sc0 = sc[0], sc1 = sc[1];
      fold<RU>(acc, p0, sc0);
      fold<RU>(acc, p1, sc1);
    }
  } else {
    const bf16x8* xf = reinterpret_cast<const bf16x8*>(xa);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t lo, hi;
      cb10_to_e4m3(w.q[d], lo, hi);
      const bf16x8 b = cat(e4m3x2_to_bf16<false>(lo), e4m3x2_to_bf16<true>(lo),
                           e4m3x2_to_bf16<false>(hi), e4m3x2_to_bf16<true>(hi));
      const f32x4 p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[d], b, zero, 0, 0, 0);
      float sc;
      switch (d) {
        case 0: sc = e4m3_to_f32<0>(w.s[0]); break;
        case 1: sc = e4m3_to_f32<1>(w.s[0]); break;
        case 2: sc = e4m3_to_f32<2>(w.s[0]); break;
        default: sc = e4m3_to_f32<3>(w.s[0]); break;
      }
      fold<RU>(acc, p, sc);
    }
  }
}

// x staging. Each wave copies the x columns of the chunks it is about to process into its own LDS
// region, in per-lane fragment order: for chunk slot u, lane group g and x row m, the 32 bf16 that lane
// (m, g) feeds to the MFMAs of that chunk sit as 64 contiguous bytes. The copy is one coalesced
// 16-byte global load per piece (a chunk row of x is 16 pieces), issued before the wave's weight
// loads so that it does not queue behind them; no workgroup barrier is involved.
template <int F, int U>
__device__ __forceinline__ void stage_x_wave(uint8_t* xs, const uint16_t* __restrict__ x, int M, int K, int c0, int W,
                                             int nchunk, int lane) {
  const int pieces = U * M * 16;
  for (int p0 = 0; p0 < pieces; p0 += 64 * 4) {
    u32x4 v[4];
    int dst[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {       // up to four loads in flight per lane before the writes
      const int p = p0 + 64 * i + lane;
      dst[i] = -1;
      v[i] = u32x4{0u, 0u, 0u, 0u};
      if (p < pieces) {
        const int u = p / (M * 16), rem = p - u * (M * 16), m = rem >> 4, qq = rem & 15;
        const int c = c0 + u * W;
        const int k = c * CHUNK_K + 8 * qq;
        if (c < nchunk && k < K) v[i] = *reinterpret_cast<const u32x4*>(x + (int64_t)m * K + k);
        dst[i] = (u * 4 * M + m) * 64 + ((F == FAST) ? ((qq & 3) * M * 64 + 16 * (qq >> 2))
                                                        : (2 * (qq & 1) * M * 64 + 8 * (qq >> 1)));
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (dst[i] < 0) continue;
      if constexpr (F == FAST) {        // k = 32 j + 8 g + t: fragment j = qq / 4 of lane group qq % 4
        *reinterpret_cast<u32x4*>(xs + dst[i]) = v[i];
      } else {                          // k = 16 j + 4 g + t: halves go to lane groups 2 (qq & 1) and +1
        *reinterpret_cast<u32x2*>(xs + dst[i]) = u32x2{v[i][0], v[i][1]};
        *reinterpret_cast<u32x2*>(xs + dst[i] + M * 64) = u32x2{v[i][2], v[i][3]};
      }
    }
  }
}

template <int F, int T, int U>
__device__ __forceinline__ void load_batch(WeightRegs<F> (&wr)[U][T], const uint8_t* __restrict__ qp,
                                           const uint8_t* __restrict__ sp, int c0, int W, int nchunk, int tile0,
                                           int ntiles, int lane, int n) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = c0 + u * W;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if (c < nchunk && tile0 + t < ntiles) {
        load_unit<F>(wr[u][t], qp, sp, (int64_t)(tile0 + t) * nchunk + c, lane, n);
      } else {
        wr[u][t].q = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < (F == FAST ? 1 : 2); ++i) wr[u][t].s[i] = 0u;
      }
    }
  }
}

// Dynamic LDS: [W waves][U chunks][4 lane groups][M rows][64 B] of staged x, then the
// cross-wave reduction buffer [W][T][64 lanes][4] floats.
template <int F, int T, int RU, int U>
__global__ __launch_bounds__(1024) void gemv_kernel(const uint8_t* __restrict__ qp, const uint8_t* __restrict__ sp,
                                                    const uint16_t* __restrict__ x, float* __restrict__ y,
                                                    int M, int N, int K, int ntiles, int nchunk, float gscale) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, W = blockDim.x >> 6;
  const int n = lane & 15, g = lane >> 4, m = lane & 15;
  const int tile0 = blockIdx.x * T;
  const bool xrow = m < M;
  const size_t xw_bytes = (size_t)U * 4 * M * 64;
  uint8_t* xs = smem + wave * xw_bytes;
  float* red = reinterpret_cast<float*>(smem + W * xw_bytes);

  f32x4 acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  WeightRegs<F> wr[U][T];
  bool have = false;
  for (int c0 = wave; c0 < nchunk; c0 += W * U) {
    stage_x_wave<F, U>(xs, x, M, K, c0, W, nchunk, lane);     // x first: it must not wait behind weights
    if (!have) load_batch<F, T, U>(wr, qp, sp, c0, W, nchunk, tile0, ntiles, lane, n);
    // the next batch's weights go out before this batch is computed
    WeightRegs<F> nx[U][T];
    const int c1 = c0 + W * U;
    have = c1 < nchunk;
    if (have) load_batch<F, T, U>(nx, qp, sp, c1, W, nchunk, tile0, ntiles, lane, n);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + u * W < nchunk) {
        // this lane's 32 x values of chunk slot u, read from the wave's staging area just before use
        uint32_t xa[16];
        if (xrow) {
          const u32x4* src = reinterpret_cast<const u32x4*>(xs + ((u * 4 + g) * M + m) * 64);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const u32x4 w4 = src[v];
            xa[4 * v] = w4[0]; xa[4 * v + 1] = w4[1]; xa[4 * v + 2] = w4[2]; xa[4 * v + 3] = w4[3];
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) xa[i] = 0u;
        }
#pragma unroll
        for (int t = 0; t < T; ++t) unit_mac<F, RU>(acc[t], wr[u][t], xa);
      }
    }
    if (have) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < T; ++t) wr[u][t] = nx[u][t];
    }
  }

  // cross-wave reduction in a fixed order, then y = g * sum
  float* mine = red + ((size_t)wave * T * 64 + lane) * 4;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    *reinterpret_cast<f32x4*>(mine + (size_t)t * 256) = acc[t];
  }
  __syncthreads();
  const int total = T * 64 * 4;
  for (int e = threadIdx.x; e < total; e += blockDim.x) {
    const int t = e / 256, l = (e >> 2) & 63, r = e & 3;
    const int mrow = 4 * (l >> 4) + r;
    const int col = (tile0 + t) * TILE_N + (l & 15);
    if (mrow < M && col < N) {
      float sum = 0.f;
      for (int w = 0; w < W; ++w) sum += red[(size_t)w * total + e];
      y[(int64_t)mrow * N + col] = sum * gscale;
    }
  }
}

constexpr int GEMV_LDS_MAX = 160 * 1024;

template <int F, int T, int RU, int U>
static void launch_gemv(int nwg, int W, hipStream_t st, const uint8_t* q, const uint8_t* s, const uint16_t* x,
                        float* y, int M, int N, int K, int ntiles, int nchunk, float g) {
  const size_t lds = (size_t)W * U * 4 * M * 64 + (size_t)W * T * 64 * 4 * sizeof(float);
  // allow more than 64 KiB of dynamic LDS for this instantiation (once; thread-safe static init)
  static const bool attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_kernel<F, T, RU, U>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, GEMV_LDS_MAX) == hipSuccess;
  (void)attr;
  hipLaunchKernelGGL((gemv_kernel<F, T, RU, U>), dim3(nwg), dim3(64 * W), lds, st, q, s, x, y, M, N, K, ntiles,
                     nchunk, g);
}

template <int F>
static void dispatch_gemv(int M, hipStream_t st, const uint8_t* q, const uint8_t* s, const uint16_t* x, float* y,
                          int N, int K, float g) {
  const int ntiles = (N + TILE_N - 1) / TILE_N;
  const int nchunk = (K + CHUNK_K - 1) / CHUNK_K;
  const int T = (M > 4) ? 2 : 1;
  const int nwg = (ntiles + T - 1) / T;
  int W = (4096 + nwg - 1) / nwg;  // aim for ~16 waves per CU across 256 CUs
  if (const char* e = getenv("FP4_GEMV_WAVES")) W = atoi(e);  // tuning override
  const int wmax = (M > 4) ? 8 : 16;  // keep the staged x (W * U * M * 256 B) inside the LDS
  if (W > wmax) W = wmax;
  if (W > nchunk) W = nchunk;
  if (W < 1) W = 1;
  if (M == 1)      launch_gemv<F, 1, 1, 4>(nwg, W, st, q, s, x, y, M, N, K, ntiles, nchunk, g);
  else if (M == 2) launch_gemv<F, 1, 2, 4>(nwg, W, st, q, s, x, y, M, N, K, ntiles, nchunk, g);
  else if (M <= 4) launch_gemv<F, 1, 4, 4>(nwg, W, st, q, s, x, y, M, N, K, ntiles, nchunk, g);
  else             launch_gemv<F, 2, 4, 2>(nwg, W, st, q, s, x, y, M, N, K, ntiles, nchunk, g);
}

}  // namespace fp4

using namespace fp4;

extern "C" int w4a16_gemv(int fmt, int64_t M, int64_t N, int64_t K, const void* q, const void* s,
                          float global_scale, const void* x_bf16, float* y, void* stream) {
  if (!fp4_valid_format(fmt)) return -1;
  if (M < 0) return -2;
  if (M > 16) return -4;
  int rc = fp4_check_nk(fmt, N, K);
  if (rc) return rc;
  if (M == 0) return 0;
  if (!q || !s || !x_bf16 || !y) return -1;
  if (!fp4_aligned(q, 16) || !fp4_aligned(s, 16) || !fp4_aligned(x_bf16, 16) || !fp4_aligned(y, 4)) return -3;
  hipStream_t st = (hipStream_t)stream;
  const uint8_t* qq = (const uint8_t*)q;
  const uint8_t* ss = (const uint8_t*)s;
  const uint16_t* xx = (const uint16_t*)x_bf16;
  switch (fmt) {
    case NVFP4: dispatch_gemv<NVFP4>((int)M, st, qq, ss, xx, y, (int)N, (int)K, global_scale); break;
    case DUAL:  dispatch_gemv<DUAL>((int)M, st, qq, ss, xx, y, (int)N, (int)K, global_scale); break;
    default:    dispatch_gemv<FAST>((int)M, st, qq, ss, xx, y, (int)N, (int)K, global_scale); break;
  }
  return fp4_launch_status();
}
