// Prefill-shaped W4A16 product (any M >= 1; intended for M >= 64).
//
// A workgroup computes a BM x BN tile of y. Per 128-wide K chunk it
//   1. stages the x tile [BM][128] (bf16) into LDS, in the chunk's permuted k' order, and
//   2. loads the packed weight units of its BN rows, dequantizes every weight once to
//      exact bf16 level*scale (g deferred) and writes the tile [BN][128] into LDS, in the
//      same k' order (the contraction only needs A and B to agree on the k order),
// then its four waves run bf16 MFMA 16x16x32 over the chunk with FP32 accumulators.
// The epilogue multiplies by g and stores fp32 y. Global loads of chunk c+1 are issued
// before the MFMAs of chunk c so that memory latency hides under the matrix work.
#include "common.h"
#include "launch.h"
#include "fp4w4a16.h"

namespace fp4 {

constexpr int GM_BM = 128, GM_BN = 128, GM_THREADS = 256;
constexpr int LDS_ROW = CHUNK_K * 2 + 16;        // bytes per LDS row (128 bf16 + pad)
constexpr int X_PIECES = GM_BM * 16 / GM_THREADS;  // 16-byte x pieces per thread per chunk (8)
constexpr int W_PIECES = (GM_BN / TILE_N) * 64 / GM_THREADS;  // lane pieces per thread (2)

// bf16 of two f32 values (exact here: level*scale has at most 7 significant bits)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  uint32_t u;
  __builtin_memcpy(&u, &v, 4);
  return u;
}

// 32 weights of one lane piece -> 16 dwords of bf16 pairs in lane-position order i = 0..31.
template <int F>
__device__ __forceinline__ void dequant_piece(const u32x4& q, const u32x2& s, uint32_t (&out)[16]) {
  if constexpr (F == NVFP4) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      // positions 8d..8d+7; group of position i is i / 4 -> groups 2d (bytes 0,1) and 2d+1 (bytes 2,3)
      const uint32_t sw = s[d >> 1];
      const float s0 = (d & 1) ? e4m3_to_f32<2>(sw) : e4m3_to_f32<0>(sw);
      const float s1 = (d & 1) ? e4m3_to_f32<3>(sw) : e4m3_to_f32<1>(sw);
      const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[d], 1.0f, 0);
      const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[d], 1.0f, 1);
      const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[d], 1.0f, 2);
      const f32x2 e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[d], 1.0f, 3);
      out[4 * d + 0] = pack_bf16x2(a[0] * s0, a[1] * s0);
      out[4 * d + 1] = pack_bf16x2(b[0] * s0, b[1] * s0);
      out[4 * d + 2] = pack_bf16x2(c[0] * s1, c[1] * s1);
      out[4 * d + 3] = pack_bf16x2(e[0] * s1, e[1] * s1);
    }
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t lo, hi;
      cb10_to_e4m3(q[d], lo, hi);
      float s0, s1;
      if constexpr (F == DUAL) {  // positions 8d..8d+3 -> group 2d, 8d+4..8d+7 -> group 2d+1
        const uint32_t sw = s[d >> 1];
        s0 = (d & 1) ? e4m3_to_f32<2>(sw) : e4m3_to_f32<0>(sw);
        s1 = (d & 1) ? e4m3_to_f32<3>(sw) : e4m3_to_f32<1>(sw);
      } else {                    // positions 8d..8d+7 -> block d
        const uint32_t sw = s[0];
        s0 = (d == 0) ? e4m3_to_f32<0>(sw) : (d == 1) ? e4m3_to_f32<1>(sw) : (d == 2) ? e4m3_to_f32<2>(sw)
                                                                                    : e4m3_to_f32<3>(sw);
        s1 = s0;
      }
      const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 1.0f, false);
      const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 1.0f, true);
      const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 1.0f, false);
      const f32x2 e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 1.0f, true);
      out[4 * d + 0] = pack_bf16x2(a[0] * s0, a[1] * s0);
      out[4 * d + 1] = pack_bf16x2(b[0] * s0, b[1] * s0);
      out[4 * d + 2] = pack_bf16x2(c[0] * s1, c[1] * s1);
      out[4 * d + 3] = pack_bf16x2(e[0] * s1, e[1] * s1);
    }
  }
}

template <int F>
__global__ __launch_bounds__(GM_THREADS) void gemm_kernel(const uint8_t* __restrict__ qp,
                                                          const uint8_t* __restrict__ sp,
                                                          const uint16_t* __restrict__ x, float* __restrict__ y,
                                                          int M, int N, int K, int ntiles, int nchunk,
                                                          int tiles_m, float gscale) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[GM_BM * LDS_ROW];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[GM_BN * LDS_ROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bm = blockIdx.x % tiles_m, bn = blockIdx.x / tiles_m;
  const int m0 = bm * GM_BM, n0 = bn * GM_BN;
  const int tile_base = n0 / TILE_N;

  // ---- per-thread global load assignments ----
  // x: piece p = tid + 256 * u  ->  row p / 16, 16-byte column p % 16 of the chunk
  // w: piece p = tid + 256 * u  ->  tile p / 64 of the block, lane piece p % 64
  u32x4 xr[X_PIECES];
  u32x4 wq[W_PIECES];
  u32x2 ws[W_PIECES];

  auto load_chunk = [&](int c) {
#pragma unroll
    for (int u = 0; u < X_PIECES; ++u) {
      const int p = tid + GM_THREADS * u;
      const int row = m0 + (p >> 4);
      const int k = c * CHUNK_K + 8 * (p & 15);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < M && k < K) v = *reinterpret_cast<const u32x4*>(x + (int64_t)row * K + k);
      xr[u] = v;
    }
#pragma unroll
    for (int u = 0; u < W_PIECES; ++u) {
      const int p = tid + GM_THREADS * u;
      const int tile = tile_base + (p >> 6), l = p & 63;
      u32x4 v = {0u, 0u, 0u, 0u};
      u32x2 sv = {0u, 0u};
      if (tile < ntiles) {
        const int64_t unit = (int64_t)tile * nchunk + c;
        v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qp + unit * UNIT_Q + l * 16));
        const uint8_t* srow = sp + unit * unit_s(F) + (l & 15) * scales_per_row_chunk(F);
        if constexpr (F == FAST) {
          sv[0] = *reinterpret_cast<const uint32_t*>(srow);
        } else {
          sv = *reinterpret_cast<const u32x2*>(srow);
        }
      }
      wq[u] = v;
      ws[u] = sv;
    }
  };

  auto store_chunk = [&]() {
#pragma unroll
    for (int u = 0; u < X_PIECES; ++u) {
      const int p = tid + GM_THREADS * u;
      const int r = p >> 4, q = p & 15;
      uint8_t* rowp = lds_a + r * LDS_ROW;
      if constexpr (F == FAST) {
        // k = 8q + t -> k' = 32 (q % 4) + 8 (q / 4) + t
        *reinterpret_cast<u32x4*>(rowp + 2 * (32 * (q & 3) + 8 * (q >> 2))) = xr[u];
      } else {
        // k = 8q + u -> k' = 64 (q % 2) + 4 (q / 2) + u (u < 4), + 32 more for u >= 4
        const int kp = 64 * (q & 1) + 4 * (q >> 1);
        *reinterpret_cast<u32x2*>(rowp + 2 * kp) = u32x2{xr[u][0], xr[u][1]};
        *reinterpret_cast<u32x2*>(rowp + 2 * (kp + 32)) = u32x2{xr[u][2], xr[u][3]};
      }
    }
#pragma unroll
    for (int u = 0; u < W_PIECES; ++u) {
      const int p = tid + GM_THREADS * u;
      const int t = p >> 6, l = p & 63;
      const int row = TILE_N * t + (l & 15), g = l >> 4;
      uint32_t out[16];
      dequant_piece<F>(wq[u], ws[u], out);
      uint8_t* dst = lds_b + row * LDS_ROW + 2 * 32 * g;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        *reinterpret_cast<u32x4*>(dst + 16 * v) = u32x4{out[4 * v], out[4 * v + 1], out[4 * v + 2], out[4 * v + 3]};
    }
  };

  const int wm = wave & 1, wn = wave >> 1;  // 2 x 2 waves, 64 x 64 each
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_chunk(0);
  for (int c = 0; c < nchunk; ++c) {
    __syncthreads();  // previous chunk's MFMAs are done with the LDS tiles
    store_chunk();
    __syncthreads();
    if (c + 1 < nchunk) load_chunk(c + 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kb = 2 * (32 * ks + 8 * (lane >> 4));
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(lds_a + (64 * wm + 16 * i + (lane & 15)) * LDS_ROW + kb);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(lds_b + (64 * wn + 16 * j + (lane & 15)) * LDS_ROW + kb);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }

  // epilogue: C[16 i + 4 (lane/16) + r][16 j + lane % 16]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + 64 * wm + 16 * i + 4 * (lane >> 4) + r;
        const int col = n0 + 64 * wn + 16 * j + (lane & 15);
        if (row < M && col < N) y[(int64_t)row * N + col] = acc[i][j][r] * gscale;
      }
}

template <int F>
static void launch_gemm(hipStream_t st, const uint8_t* q, const uint8_t* s, const uint16_t* x, float* y, int M,
                        int N, int K, float g) {
  const int ntiles = (N + TILE_N - 1) / TILE_N;
  const int nchunk = (K + CHUNK_K - 1) / CHUNK_K;
  const int tiles_m = (M + GM_BM - 1) / GM_BM;
  const int tiles_n = (N + GM_BN - 1) / GM_BN;
  hipLaunchKernelGGL(gemm_kernel<F>, dim3(tiles_m * tiles_n), dim3(GM_THREADS), 0, st, q, s, x, y, M, N, K, ntiles,
                     nchunk, tiles_m, g);
}

}  // namespace fp4

using namespace fp4;

extern "C" int w4a16_gemm(int fmt, int64_t M, int64_t N, int64_t K, const void* q, const void* s,
                          float global_scale, const void* x_bf16, float* y, void* stream) {
  if (!fp4_valid_format(fmt)) return -1;
  if (M < 0) return -2;
  int rc = fp4_check_nk(fmt, N, K);
  if (rc) return rc;
  if (M == 0) return 0;
  if (M > (1LL << 30)) return -4;
  if (!q || !s || !x_bf16 || !y) return -1;
  if (!fp4_aligned(q, 16) || !fp4_aligned(s, 16) || !fp4_aligned(x_bf16, 16) || !fp4_aligned(y, 4)) return -3;
  const int64_t grid = ((M + GM_BM - 1) / GM_BM) * ((N + GM_BN - 1) / GM_BN);
  if (grid > 0x7fffffffLL) return -4;
  hipStream_t st = (hipStream_t)stream;
  const uint8_t* qq = (const uint8_t*)q;
  const uint8_t* ss = (const uint8_t*)s;
  const uint16_t* xx = (const uint16_t*)x_bf16;
  switch (fmt) {
    case NVFP4: launch_gemm<NVFP4>(st, qq, ss, xx, y, (int)M, (int)N, (int)K, global_scale); break;
    case DUAL:  launch_gemm<DUAL>(st, qq, ss, xx, y, (int)M, (int)N, (int)K, global_scale); break;
    default:    launch_gemm<FAST>(st, qq, ss, xx, y, (int)M, (int)N, (int)K, global_scale); break;
  }
  return fp4_launch_status();
}

extern "C" int w4a16_matmul(int fmt, int64_t M, int64_t N, int64_t K, const void* q, const void* s,
                            float global_scale, const void* x_bf16, float* y, void* stream) {
  if (M >= 0 && M <= 16) return w4a16_gemv(fmt, M, N, K, q, s, global_scale, x_bf16, y, stream);
  return w4a16_gemm(fmt, M, N, K, q, s, global_scale, x_bf16, y, stream);
}
