// Decode-shaped W4A16 product (1 <= M <= 16), and the mid-M product (M <= 64) further down.
//
// One workgroup owns T consecutive 16-row tiles of W and the whole K range; its W waves
// split the 128-wide K chunks (wave w takes chunks w, w + W, ...). Per chunk a lane loads
// 16 bytes of nibbles per tile (row n = lane % 16, lane group g = lane / 16) and the row's
// scale bytes, decodes to exact bf16 levels and issues one MFMA per scale group:
//   A = x fragment (row m = lane % 16, zero for m >= M), B = unscaled levels, C = 0,
// then folds the group scale into FP32: acc += scale * C. The waves' partial sums are
// reduced through LDS in a fixed order, multiplied by the global scale and stored. Long K at M = 1
// on large grids uses a variant that keeps a ring of chunks in flight per wave (gemv_ring_kernel).
#include "common.h"
#include "launch.h"
#include "fp4w4a16.h"
#include <stdlib.h>
#include <atomic>

namespace fp4 {


template <int F>
struct WeightRegs {
  u32x4 q;
  uint32_t s[F == FAST ? 1 : 2];
};

// Buffer descriptors: the workgroup's tiles of both planes, and x. A load at an offset a descriptor
// does not reach returns zeros, so no load needs a branch or a select; OOB is such an offset (every
// descriptor here covers less than 2^31 bytes).
constexpr uint32_t OOB = 0x80000000u;

// dynamic LDS a workgroup may ask for (all of a CU's LDS)
constexpr int GEMV_LDS_MAX = 160 * 1024;

struct Srcs {
  __amdgpu_buffer_rsrc_t q, s, x;
};

template <int F>
__device__ __forceinline__ void load_unit(WeightRegs<F>& r, const Srcs& src, uint32_t qoff, uint32_t soff) {
  r.q = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(src.q, qoff, 0, 2 /* nt */));
  if constexpr (F == FAST) {
    r.s[0] = __builtin_amdgcn_raw_buffer_load_b32(src.s, soff, 0, 0);
  } else {
    const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(src.s, soff, 0, 0));
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
  } else if constexpr (F == FAST) {
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
  } else {
    // Q4_0, level q - 8: B holds the bf16 numbers 128 + q, built by placing each nibble in the low
    // mantissa bits of bf16 128 (exact), and the MFMA starts from C = -136 * (x . 1) of the block
    // (one more MFMA against a constant -136), so that it returns sum (q - 8) x in FP32.
    const bf16x8* xf = reinterpret_cast<const bf16x8*>(xa);
    const u32x4 m136 = {0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u};  // bf16 -136
    const bf16x8 neg136 = __builtin_bit_cast(bf16x8, m136);
    // bf16 128 in both halves, kept in a VGPR so that mask-and-insert is one v_and_or_b32 (a VOP3
    // instruction can take one scalar operand, here the mask, but no literal)
    uint32_t magic = 0x43004300u;
    asm volatile("" : "+v"(magic));
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const f32x4 c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[d], neg136, zero, 0, 0, 0);
      const uint32_t wq = w.q[d];
      // positions 8d..8d+3 are the low nibbles of bytes 0..3, 8d+4..8d+7 the high nibbles
      const uint32_t p01 = __builtin_amdgcn_perm(0u, wq, 0x0C010C00u);  // bytes 0, 1 -> halves 0, 1
      const uint32_t p23 = __builtin_amdgcn_perm(0u, wq, 0x0C030C02u);  // bytes 2, 3 -> halves 0, 1
      const u32x4 bw = {(p01 & 0x000F000Fu) | magic, (p23 & 0x000F000Fu) | magic,
                        ((p01 >> 4) & 0x000F000Fu) | magic, ((p23 >> 4) & 0x000F000Fu) | magic};
      const f32x4 p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[d], __builtin_bit_cast(bf16x8, bw), c0, 0, 0, 0);
      // the block's FP16 scale: half-word d % 2 of scale dword d / 2
      const uint16_t hb = (uint16_t)(w.s[d >> 1] >> (16 * (d & 1)));
      fold<RU>(acc, p, (float)__builtin_bit_cast(_Float16, hb));
    }
  }
}

// Bytes from one lane group's staged x rows to the next (M rows of 64 B). With M even, M * 64 is a multiple
// of 128 B and the four groups of a chunk would start on the same LDS banks: a commit that writes one piece
// to each of them (32-weight blocks) would hit one bank set four times, so 16 B follow each group. With M
// odd the groups already alternate between two bank halves, and a pad there measured slightly slower.
__host__ __device__ constexpr int x_gs(int M) { return M * 64 + ((M & 1) ? 0 : 16); }

// x staging. Each wave copies the x columns of the chunks it is about to process into its own LDS
// region, in per-lane fragment order: for chunk slot u, lane group g and x row m, the 32 bf16 that lane
// (m, g) feeds to the MFMAs of that chunk sit as 64 contiguous bytes at (4 u + g) x_gs(M) + 64 m. The copy is split in two so that
// the weight loads can be issued in between: `issue` starts coalesced 16-byte global loads (a chunk
// row of x is 16 pieces) into registers, `commit` writes them to LDS. Loads complete in order, so
// committing waits only for x, never for the weight loads issued after it; no workgroup barrier is
// involved. MX bounds M, so NX = U * MX / 4 loads per lane cover every piece.
template <int U, int MX>
struct XStage {
  static constexpr int NX = (U * MX * 16 + 63) / 64;
  u32x4 v[NX];
};

// byte offset of x piece p (16 bytes: 8 consecutive k of one row) of the batch starting at chunk c0.
// WRAP (M known at compile time): lanes past the last piece take piece p % pieces, so that they load and
// stage the same bytes as another lane and the staging store needs no branch (a branch there lets the
// compiler sink the x load below the weight loads, and staging x would then wait for all of them).
template <int U, bool WRAP = false>
__device__ __forceinline__ uint32_t x_piece_off(int p, int M, int K, int c0, int W, int nchunk) {
  const int pieces = U * M * 16;
  if constexpr (WRAP) p = p % pieces;
  // (with one chunk slot every valid piece is in slot 0: no division)
  const int u = U == 1 ? 0 : p / (M * 16), rem = p - u * (M * 16), m = rem >> 4, qq = rem & 15;
  const int c = c0 + u * W;
  const int k = c * CHUNK_K + 8 * qq;
  return (p < pieces && c < nchunk && k < K) ? (uint32_t)(m * K + k) * 2u : OOB;
}

template <int F, int U, int MX, bool WRAP = false>
__device__ __forceinline__ void stage_x_issue(XStage<U, MX>& st, const Srcs& src, int M, int K, int c0, int W,
                                              int nchunk, int lane) {
#pragma unroll
  for (int i = 0; i < XStage<U, MX>::NX; ++i) {
    const uint32_t off = x_piece_off<U, WRAP>(64 * i + lane, M, K, c0, W, nchunk);
    st.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(src.x, off, 0, 0));
  }
}

template <int F, int U, int MX, bool WRAP = false>
__device__ __forceinline__ void stage_x_commit(uint8_t* xs, const XStage<U, MX>& st, int M, int lane) {
  const int pieces = U * M * 16;
#pragma unroll
  for (int i = 0; i < XStage<U, MX>::NX; ++i) {
    const int p = WRAP ? (64 * i + lane) % pieces : 64 * i + lane;
    if (WRAP || p < pieces) {
      const int u = U == 1 ? 0 : p / (M * 16), rem = p - u * (M * 16), m = rem >> 4, qq = rem & 15;
      const int gs = x_gs(M);
      const int dst = u * 4 * gs + m * 64 + (block32(F) ? ((qq & 3) * gs + 16 * (qq >> 2))
                                                        : (2 * (qq & 1) * gs + 8 * (qq >> 1)));
      if constexpr (block32(F)) {        // k = 32 j + 8 g + t: fragment j = qq / 4 of lane group qq % 4
        *reinterpret_cast<u32x4*>(xs + dst) = st.v[i];
      } else {                          // k = 16 j + 4 g + t: halves go to lane groups 2 (qq & 1) and +1
        *reinterpret_cast<u32x2*>(xs + dst) = u32x2{st.v[i][0], st.v[i][1]};
        *reinterpret_cast<u32x2*>(xs + dst + gs) = u32x2{st.v[i][2], st.v[i][3]};
      }
    }
  }
}

// Loads and commits a batch's x in one go, four loads per lane in flight at a time (used when x has
// too many rows to be held in registers across the weight loads).
template <int F, int U>
__device__ __forceinline__ void stage_x_now(uint8_t* xs, const Srcs& src, int M, int K, int c0, int W, int nchunk,
                                            int lane) {
  const int pieces = U * M * 16;
  for (int p0 = 0; p0 < pieces; p0 += 64 * 4) {
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = u32x4{0u, 0u, 0u, 0u};
      if (p0 + 64 * i < pieces) {      // wave-uniform: no load instruction for a wholly empty group
        const uint32_t off = x_piece_off<U>(p0 + 64 * i + lane, M, K, c0, W, nchunk);
        v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(src.x, off, 0, 0));
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = p0 + 64 * i + lane;
      if (p >= pieces) continue;
      const int u = p / (M * 16), rem = p - u * (M * 16), m = rem >> 4, qq = rem & 15;
      const int gs = x_gs(M);
      const int dst = u * 4 * gs + m * 64 + (block32(F) ? ((qq & 3) * gs + 16 * (qq >> 2))
                                                        : (2 * (qq & 1) * gs + 8 * (qq >> 1)));
      if constexpr (block32(F)) {
        *reinterpret_cast<u32x4*>(xs + dst) = v[i];
      } else {
        *reinterpret_cast<u32x2*>(xs + dst) = u32x2{v[i][0], v[i][1]};
        *reinterpret_cast<u32x2*>(xs + dst + gs) = u32x2{v[i][2], v[i][3]};
      }
    }
  }
}

// Weight units of one batch: chunk c0 + u W of each of the T tiles. Units past the last chunk, or
// of a tile past the last one (outside the descriptor), read as zeros.
template <int F, int T, int U>
__device__ __forceinline__ void load_batch(WeightRegs<F> (&wr)[U][T], const Srcs& src, int c0, int W, int nchunk,
                                           int lane, int n) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = c0 + u * W;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const uint32_t unit = (uint32_t)(t * nchunk + c);
      const bool ok = c < nchunk;
      load_unit<F>(wr[u][t], src, ok ? unit * UNIT_Q + lane * 16 : OOB,
                   ok ? unit * unit_s(F) + n * (unit_s(F) / TILE_N) : OOB);
      __builtin_amdgcn_sched_barrier(0);  // units in order: each unit's nibbles and scales together
    }
  }
}

// One matrix of a launch. A launch covers one or more matrices that share the format and M; the
// grid is the concatenation of their workgroup ranges, matrix i owning workgroups [wg0, next wg0).
struct GemvItem {
  const uint8_t* q;
  const uint8_t* s;
  const uint16_t* x;
  float* y;
  int N, K, nchunk, wg0;
  float g;
  int pad;
};

// start[i] is item i's first workgroup (INT_MAX for unused entries). Launches of up to 4 matrices also
// pass starts 1..3 as preloaded scalars; larger ones read them here, together ahead of the items, with
// wide scalar loads.
template <int MAXI>
struct GemvBatch {
  int count;
  int start[MAXI];
  GemvItem it[MAXI];
};

// How a launch's waves cover K. BATCH_LOOP: batches of U chunk slots, the next prefetched during the
// current one. The others take all of a wave's chunks in one batch (wave w: chunks w, w + W, ...,
// w + (U - 1) W) and differ in which slots may lie past the last chunk (such a slot reads zeros):
// ONE_CHECKED any (each slot is tested), ONE_LAST only the last one ((U - 1) W <= nchunk for every
// matrix), ONE_FULL none (nchunk = U W for every matrix).
enum OneBatch { BATCH_LOOP = 0, ONE_CHECKED = 1, ONE_LAST = 2, ONE_FULL = 3 };

// Dynamic LDS: [W waves][U chunks][4 lane groups][M rows][64 B] of staged x, then the
// cross-wave reduction buffer: [W][T][64 lanes][4] floats, or with M <= 4 fixed at compile time only the
// stored C rows, [W][T][M][16] floats.
// MC > 0 fixes M = MC at compile time (the x address arithmetic then reduces to shifts and masks);
// MC = 0 takes M from mw (at most MX). mw = M | W << 8, W = waves per workgroup. ONE (a OneBatch
// value) other than BATCH_LOOP: every wave's chunks fit in one batch (nchunk <= U * W for every matrix of
// the launch), so there is no next batch to prefetch. wg0 is the matrix's first workgroup.
template <int F, int T, int RU, int U, int MX, int MC, int ONE>
__device__ __forceinline__ void gemv_body(const uint8_t* __restrict__ qp, const uint8_t* __restrict__ sp,
                                          const uint16_t* __restrict__ x, float* __restrict__ y, int N, int K,
                                          float gscale, int wg0, int mw) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int M = MC > 0 ? MC : (mw & 0xff);
  const int W = mw >> 8;
  const int nchunk = (K + CHUNK_K - 1) / CHUNK_K;
  const int ntiles = (N + TILE_N - 1) / TILE_N;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar branches
  const int n = lane & 15, g = lane >> 4, m = lane & 15;
  const int tile0 = ((int)blockIdx.x - wg0) * T;
  const int tiles_here = min(T, ntiles - tile0);
  Srcs src;
  src.q = make_rsrc(qp + (int64_t)tile0 * nchunk * UNIT_Q, (uint32_t)(tiles_here * nchunk * UNIT_Q));
  src.s = make_rsrc(sp + (int64_t)tile0 * nchunk * unit_s(F), (uint32_t)(tiles_here * nchunk * unit_s(F)));
  src.x = make_rsrc(x, (uint32_t)(M * K) * 2u);
  const size_t xw_bytes = (size_t)U * 4 * x_gs(M);
  uint8_t* xs = smem + wave * xw_bytes;
  float* red = reinterpret_cast<float*>(smem + W * xw_bytes);

  f32x4 acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Rows m >= M of the MFMA A operand read x row M - 1: their products land in C rows that are never
  // stored, and reading a valid row keeps every lane on one path with no zero fill.
  const int xm = m < M ? m : M - 1;
  WeightRegs<F> wr[U][T];
  // With few x rows (XPF) a batch's x is loaded ahead of its weights and held in registers until
  // they are issued, and the next batch's x is prefetched together with its weights. With many rows
  // that would cost too many registers: x is then loaded and committed at the top of each batch.
  constexpr bool XPF = XStage<U, MX>::NX <= (ONE != BATCH_LOOP ? 6 : 2);
  XStage<U, XPF ? MX : 1> xst;
  if constexpr (XPF) {
    if (wave < nchunk) {
      // x first, then every weight load, in that order (the scheduler may not interleave them with
      // the staging below: staging waits for x only because loads complete in order)
      stage_x_issue<F, U, MX, (MC > 0)>(xst, src, M, K, wave, W, nchunk, lane);
      __builtin_amdgcn_sched_barrier(0);
      load_batch<F, T, U>(wr, src, wave, W, nchunk, lane, n);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  bool have = XPF;  // wr already holds this batch's weights
  for (int c0 = wave; c0 < nchunk; c0 += ONE != BATCH_LOOP ? nchunk : W * U) {
    if constexpr (XPF) {
      stage_x_commit<F, U, MX, (MC > 0)>(xs, xst, M, lane);
    } else {
      stage_x_now<F, U>(xs, src, M, K, c0, W, nchunk, lane);
      if (!have) load_batch<F, T, U>(wr, src, c0, W, nchunk, lane, n);
    }
    // the next batch (x first, then weights) goes out before this batch is computed
    WeightRegs<F> nx[U][T];
    const int c1 = ONE != BATCH_LOOP ? nchunk : c0 + W * U;
    have = ONE == BATCH_LOOP && c1 < nchunk;
    if (have) {
      if constexpr (XPF) stage_x_issue<F, U, MX, (MC > 0)>(xst, src, M, K, c1, W, nchunk, lane);
      load_batch<F, T, U>(nx, src, c1, W, nchunk, lane, n);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // Slots the launch guarantees to hold a chunk are computed without a test: straight-line code
      // lets the compiler interleave one unit's decode with the previous unit's MFMAs.
      const bool sure = ONE == ONE_FULL || (ONE == ONE_LAST && u < U - 1);
      if (sure || c0 + u * W < nchunk) {
        // this lane's 32 x values of chunk slot u, read from the wave's staging area just before use
        uint32_t xa[16];
        const u32x4* src = reinterpret_cast<const u32x4*>(xs + (u * 4 + g) * x_gs(M) + xm * 64);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const u32x4 w4 = src[v];
          xa[4 * v] = w4[0]; xa[4 * v + 1] = w4[1]; xa[4 * v + 2] = w4[2]; xa[4 * v + 3] = w4[3];
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
  if constexpr (MC >= 1 && MC <= 4) {
    // at most 4 x rows: the stored C rows 0 .. MC - 1 are elements 0 .. MC - 1 of lanes 0-15, so only
    // they go through LDS: red[wave][t][r][16]
    if (lane < 16) {
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int r = 0; r < MC; ++r) red[((wave * T + t) * MC + r) * 16 + lane] = acc[t][r];
    }
    __syncthreads();
    constexpr int per_wave = T * MC * 16;
    if ((int)threadIdx.x < per_wave) {
      const int e = threadIdx.x, t = e / (MC * 16), r = (e >> 4) % MC, col = (tile0 + t) * TILE_N + (e & 15);
      if (col < N) {
        float sum = 0.f;
        for (int w = 0; w < W; ++w) sum += red[w * per_wave + e];
        y[(int64_t)r * N + col] = sum * gscale;
      }
    }
    return;
  }
  float* mine = red + ((size_t)wave * T * 64 + lane) * 4;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    *reinterpret_cast<f32x4*>(mine + (size_t)t * 256) = acc[t];
  }
  __syncthreads();
  const int total = T * 64 * 4;
  for (int e = threadIdx.x; e < total; e += W * 64) {
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

// Long-K single-row product (M = 1, one tile per workgroup, more than 4 chunks per wave): each wave
// keeps D chunks in flight in a ring of D weight-register slots, refilling a slot as soon as its chunk
// has been multiplied, so a wave holds D units of registers (not two batches of them) and more waves fit
// on a CU. The workgroup's whole x (nchunk * 256 B) is staged in LDS once, in fragment order, behind a
// single barrier; the waves' first weight loads are issued before it.
template <int F, int D>
__device__ __forceinline__ void gemv_ring_body(const uint8_t* __restrict__ qp, const uint8_t* __restrict__ sp,
                                               const uint16_t* __restrict__ x, float* __restrict__ y, int N, int K,
                                               float gscale, int mw) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int XMAX = 4;  // x pieces per thread: 16 * nchunk <= XMAX * 64 * W (the host keeps nchunk <= 256, W = 16)
  const int W = mw >> 8;
  const int nchunk = (K + CHUNK_K - 1) / CHUNK_K;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int tile = (int)blockIdx.x;
  Srcs src;
  src.q = make_rsrc(qp + (int64_t)tile * nchunk * UNIT_Q, (uint32_t)(nchunk * UNIT_Q));
  src.s = make_rsrc(sp + (int64_t)tile * nchunk * unit_s(F), (uint32_t)(nchunk * unit_s(F)));
  src.x = make_rsrc(x, (uint32_t)K * 2u);
  uint8_t* xs = smem;                                               // [nchunk][4 lane groups][64 B]
  float* red = reinterpret_cast<float*>(smem + (size_t)nchunk * 256);  // [W][64 lanes][4]
  const int pieces = nchunk * 16;
  const int nthr = W * 64;

  // x pieces of the workgroup (16 B = 8 consecutive k each), first
  u32x4 xv[XMAX];
#pragma unroll
  for (int i = 0; i < XMAX; ++i) {
    const int p = (int)threadIdx.x + i * nthr;
    const uint32_t off = (p < pieces && 8 * p < K) ? (uint32_t)p * 16u : OOB;
    xv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(src.x, off, 0, 0));
  }
  __builtin_amdgcn_sched_barrier(0);
  // this wave's chunks: wave + j W, j = 0 .. nper - 1; the first D go out now
  const int nper = wave < nchunk ? (nchunk - wave + W - 1) / W : 0;
  WeightRegs<F> wr[D];
#pragma unroll
  for (int s = 0; s < D; ++s) {
    const int c = wave + s * W;
    const bool ok = c < nchunk;
    load_unit<F>(wr[s], src, ok ? (uint32_t)c * UNIT_Q + lane * 16 : OOB,
                 ok ? (uint32_t)c * unit_s(F) + n * (unit_s(F) / TILE_N) : OOB);
    __builtin_amdgcn_sched_barrier(0);
  }
  // x into LDS in fragment order (piece p: chunk p / 16, piece qq = p % 16 of it)
#pragma unroll
  for (int i = 0; i < XMAX; ++i) {
    const int p = (int)threadIdx.x + i * nthr;
    if (p < pieces) {
      const int c = p >> 4, qq = p & 15;
      const int dst = c * 256 + (block32(F) ? ((qq & 3) * 64 + 16 * (qq >> 2)) : (2 * (qq & 1) * 64 + 8 * (qq >> 1)));
      if constexpr (block32(F)) {
        *reinterpret_cast<u32x4*>(xs + dst) = xv[i];
      } else {
        *reinterpret_cast<u32x2*>(xs + dst) = u32x2{xv[i][0], xv[i][1]};
        *reinterpret_cast<u32x2*>(xs + dst + 64) = u32x2{xv[i][2], xv[i][3]};
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's x stores are done
  asm volatile("s_barrier" ::: "memory");

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int base = 0; base < nper; base += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      const int j = base + s;
      const int c = wave + j * W;
      if (j < nper) {
        uint32_t xa[16];
        const u32x4* xsrc = reinterpret_cast<const u32x4*>(xs + c * 256 + g * 64);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const u32x4 w4 = xsrc[v];
          xa[4 * v] = w4[0]; xa[4 * v + 1] = w4[1]; xa[4 * v + 2] = w4[2]; xa[4 * v + 3] = w4[3];
        }
        unit_mac<F, 1>(acc, wr[s], xa);
      }
      // refill the slot, on every path (past this wave's last chunk the load reads nothing): every
      // path then has the same loads in flight, so the waits stay counted instead of draining
      const bool more = j + D < nper;
      const uint32_t cn = (uint32_t)(c + D * W);
      load_unit<F>(wr[s], src, more ? cn * UNIT_Q + lane * 16 : OOB,
                   more ? cn * unit_s(F) + n * (unit_s(F) / TILE_N) : OOB);
    }
  }

  // cross-wave reduction in a fixed order, then y = g * sum (only C row 0, lanes 0-15, is stored)
  if (lane < 16) red[wave * 16 + lane] = acc[0];
  __syncthreads();
  if ((int)threadIdx.x < 16) {
    const int col = tile * TILE_N + (int)threadIdx.x;
    if (col < N) {
      float sum = 0.f;
      for (int w = 0; w < W; ++w) sum += red[w * 16 + (int)threadIdx.x];
      y[col] = sum * gscale;
    }
  }
}

template <int F, int D>
__global__ __launch_bounds__(1024) void gemv_ring_kernel(const uint8_t* q, const uint8_t* s, const uint16_t* x, float* y,
                                                         int N, int K, float g, int mw) {
  gemv_ring_body<F, D>(q, s, x, y, N, K, g, mw);
}

// The ring kernel runs with 16 waves, so one thread stages at most 4 of the 16 * nchunk x pieces: up to
// RING_MAX_CHUNKS = 256 chunks (K <= 32768), 64 KiB of staged x.
constexpr int RING_WAVES = 16;
constexpr int RING_MAX_CHUNKS = 256;

template <int F, int D>
struct RingLaunch {
  static const void* fn() { return reinterpret_cast<const void*>(&gemv_ring_kernel<F, D>); }
  static size_t lds(int W, int nchunk) { return (size_t)nchunk * 256 + (size_t)W * 64 * 4 * sizeof(float); }
  static int launch(const GemvItem& it, int W, hipStream_t st) {
    static Fp4LdsLimit lds_limit;
    lds_limit.ensure(fn(), GEMV_LDS_MAX);
    const int nchunk = (it.K + CHUNK_K - 1) / CHUNK_K, ntiles = (it.N + TILE_N - 1) / TILE_N;
    return fp4_launch(gemv_ring_kernel<F, D>, dim3(ntiles), dim3(64 * W), lds(W, nchunk), st, it.q, it.s, it.x, it.y,
                      it.N, it.K, it.g, 1 | (W << 8));
  }
};

// Entry points. Both take their leading arguments in scalar registers that the library is built to
// preload at wave start, so a wave does not first wait on the kernel-argument memory; W comes in mw, so
// no dispatch-packet field is read either.
// One matrix: everything the body needs is preloaded.
template <int F, int T, int RU, int U, int MX, int MC, int ONE>
__global__ __launch_bounds__(1024) void gemv_kernel(const uint8_t* q, const uint8_t* s, const uint16_t* x, float* y,
                                                    int N, int K, float g, int mw) {
  gemv_body<F, T, RU, U, MX, MC, ONE>(q, s, x, y, N, K, g, 0, mw);
}

// Several matrices: with at most 4 the starts of matrices 1..3 are preloaded (INT_MAX where unused), so
// the workgroup's matrix is known at once and its fields take one read of the argument memory; with
// more the starts are searched in the GemvBatch.
template <int F, int T, int RU, int U, int MX, int MAXI, int MC, int ONE>
__global__ __launch_bounds__(1024) void gemv_group_kernel(int st1, int st2, int st3, int mw, const GemvBatch<MAXI> batch) {
  const int b = (int)blockIdx.x;
  int item = 0;
  if constexpr (MAXI <= 4) {
    item = (b >= st1 ? 1 : 0) + (b >= st2 ? 1 : 0) + (b >= st3 ? 1 : 0);
  } else {
#pragma unroll
    for (int i = 1; i < MAXI; ++i) item += b >= batch.start[i] ? 1 : 0;  // starts ascend
  }
  const GemvItem& it = batch.it[item];
  gemv_body<F, T, RU, U, MX, MC, ONE>(it.q, it.s, it.x, it.y, it.N, it.K, it.g, it.wg0, mw);
}

// ---------------------------------------------------------------------------------------------------
// Mid-M product (5 <= M <= 64 where the one-batch GEMV does not fit). Same layout, workgroup shape and K
// split as the GEMV (one 16-row tile per workgroup, waves take chunks wave, wave + W, ...), with each
// wave's chunks in a chain (the next chunk's x and weights in flight while the current one is computed).
// With more than one block of 16 x rows (MB > 1) every unit's weights are decoded once into bf16 MFMA
// operands that already carry the group scale (level * scale, exact in bf16) and are reused by the MB
// blocks, one 16x16x32 MFMA per 32 positions and block accumulating straight into FP32. With one block
// the scales are folded per group into FP32 after the MFMAs instead, as in the GEMV (fewer VALU
// instructions per unit: 2-4% faster for Dual and FAST at M = 9, the same for NVFP4). The waves' sums
// are reduced through LDS in a fixed order.
//
// B operand j (j = 0..3) of a unit is dword j of the lane's 16 bytes: positions 8 j .. 8 j + 7. For
// 16-weight groups those are positions 4 t of group 2 j (first four) and of group 2 j + 1 (last four),
// matching x fragments 2 j and 2 j + 1 of the staged row; for FAST they are block j.
template <int F>
__device__ __forceinline__ void decode_scaled(const WeightRegs<F>& w, bf16x8 (&b)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t d = w.q[j];
    if constexpr (F == FAST) {
      const float sc = (j == 0) ? e4m3_to_f32<0>(w.s[0]) : (j == 1) ? e4m3_to_f32<1>(w.s[0])
                     : (j == 2) ? e4m3_to_f32<2>(w.s[0]) : e4m3_to_f32<3>(w.s[0]);
      const uint32_t lo = cb10_quad<false>(d), hi = cb10_quad<true>(d);
      b[j] = to_bf16x8(__builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 1.0f, false),
                       __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 1.0f, true),
                       __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 1.0f, false),
                       __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 1.0f, true), sc);
    } else {
      // scales of groups 2 j and 2 j + 1: half-word j % 2 of scale dword j / 2
      const f32x2 sc = (j & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(w.s[j >> 1], true)
                               : __builtin_amdgcn_cvt_pk_f32_fp8(w.s[j >> 1], false);
      if constexpr (F == DUAL) {
        const uint32_t lo = cb10_quad<false>(d), hi = cb10_quad<true>(d);
        b[j] = to_bf16x8(__builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 1.0f, false),
                         __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 1.0f, true),
                         __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 1.0f, false),
                         __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 1.0f, true), sc[0], sc[1]);
      } else {
        b[j] = to_bf16x8(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0),
                         __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1),
                         __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2),
                         __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3), sc[0], sc[1]);
      }
    }
  }
}

// Dynamic LDS: [W waves][4 lane groups][x_gs(M) B] of staged x (one chunk per wave; the pad that x_gs adds
// for even M took FAST 9728 x 2560 at M = 16 from 7.80 to 6.86 us); after the K loop
// the same space holds the cross-wave reduction buffer [W][T][MB][64 lanes][4] floats. wg0 is the
// matrix's first workgroup (grouped launches).
template <int F, int MB, int T, int MXB = 16 * MB>
__device__ __forceinline__ void midm_body(const uint8_t* __restrict__ qp, const uint8_t* __restrict__ sp,
                                          const uint16_t* __restrict__ x, float* __restrict__ y, int N, int K,
                                          float gscale, int mw, int wg0) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int MXR = MXB;  // bound on M: the x loads per chunk cover MXR rows (1 <= M <= MXR)
  const int M = mw & 0xff, W = mw >> 8;
  const int ntiles = (N + TILE_N - 1) / TILE_N, nchunk = (K + CHUNK_K - 1) / CHUNK_K;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4, m16 = lane & 15;
  const int tile0 = ((int)blockIdx.x - wg0) * T;
  const int tiles_here = min(T, ntiles - tile0);
  Srcs src;
  src.q = make_rsrc(qp + (int64_t)tile0 * nchunk * UNIT_Q, (uint32_t)(tiles_here * nchunk * UNIT_Q));
  src.s = make_rsrc(sp + (int64_t)tile0 * nchunk * unit_s(F), (uint32_t)(tiles_here * nchunk * unit_s(F)));
  src.x = make_rsrc(x, (uint32_t)(M * K) * 2u);
  const size_t xw_bytes = (size_t)4 * x_gs(M);
  uint8_t* xs = smem + wave * xw_bytes;
  const uint32_t soff_lane = n * (unit_s(F) / TILE_N);

  f32x4 acc[T][MB];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[t][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // x of the wave's next chunk is loaded into registers (all of it at once) together with the next
  // weights while the current chunk is computed, then committed to LDS at the top of the next chunk.
  // The T tiles of the workgroup share that x.
  XStage<1, MXR> xst;
  WeightRegs<F> wr[T];
  if (wave < nchunk) {
    stage_x_issue<F, 1, MXR>(xst, src, M, K, wave, W, nchunk, lane);
#pragma unroll
    for (int t = 0; t < T; ++t)
      load_unit<F>(wr[t], src, (uint32_t)(t * nchunk + wave) * UNIT_Q + lane * 16,
                   (uint32_t)(t * nchunk + wave) * unit_s(F) + soff_lane);
  }
  for (int c = wave; c < nchunk; c += W) {
    stage_x_commit<F, 1, MXR>(xs, xst, M, lane);
    WeightRegs<F> nx[T];               // next units of this wave, in flight during these
    const int c1 = c + W;
    if (c1 < nchunk) {
      stage_x_issue<F, 1, MXR>(xst, src, M, K, c1, W, nchunk, lane);
#pragma unroll
      for (int t = 0; t < T; ++t)
        load_unit<F>(nx[t], src, (uint32_t)(t * nchunk + c1) * UNIT_Q + lane * 16,
                     (uint32_t)(t * nchunk + c1) * unit_s(F) + soff_lane);
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if constexpr (MB == 1) {           // one block of x rows: unscaled levels, scales folded per group
        const uint8_t* xr = xs + g * x_gs(M) + min(m16, M - 1) * 64;
        uint32_t xa[16];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const u32x4 w4 = *reinterpret_cast<const u32x4*>(xr + 16 * v);
          xa[4 * v] = w4[0]; xa[4 * v + 1] = w4[1]; xa[4 * v + 2] = w4[2]; xa[4 * v + 3] = w4[3];
        }
        unit_mac<F, 4>(acc[t][0], wr[t], xa);
      } else {
        bf16x8 b[4];
        decode_scaled<F>(wr[t], b);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int row = min(mb * 16 + m16, M - 1);  // rows past M repeat a valid row; never stored
          const uint8_t* xr = xs + g * x_gs(M) + row * 64;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(xr + 16 * j);
            acc[t][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[j], acc[t][mb], 0, 0, 0);
          }
        }
      }
    }
    if (c1 < nchunk) {
#pragma unroll
      for (int t = 0; t < T; ++t) wr[t] = nx[t];
    }
  }

  __syncthreads();                     // every wave is done with its staged x: reuse the space
  float* red = reinterpret_cast<float*>(smem);
  const int total = T * MB * 256;
  float* mine = red + (size_t)wave * total + lane * 4;
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) *reinterpret_cast<f32x4*>(mine + (size_t)(t * MB + mb) * 256) = acc[t][mb];
  __syncthreads();
  for (int e = threadIdx.x; e < total; e += W * 64) {
    const int t = e / (MB * 256), mb = (e / 256) % MB, l = (e >> 2) & 63, r = e & 3;
    const int mrow = mb * 16 + 4 * (l >> 4) + r;
    const int col = (tile0 + t) * TILE_N + (l & 15);
    if (mrow < M && col < N) {
      float sum = 0.f;
      for (int w = 0; w < W; ++w) sum += red[(size_t)w * total + e];
      y[(int64_t)mrow * N + col] = sum * gscale;
    }
  }
}

template <int F, int MB, int T, int WMAX = 8, int MXB = 16 * MB>
__global__ __launch_bounds__(64 * WMAX) void midm_kernel(const uint8_t* __restrict__ qp, const uint8_t* __restrict__ sp,
                                                   const uint16_t* __restrict__ x, float* __restrict__ y, int N,
                                                   int K, float gscale, int mw) {
  midm_body<F, MB, T, MXB>(qp, sp, x, y, N, K, gscale, mw, 0);
}

// Several matrices with one block of x rows (5 <= M <= 16) in one launch; the workgroup finds its matrix
// as the grouped GEMV does.
template <int F, int MAXI, int WMAX, int MXB>
__global__ __launch_bounds__(64 * WMAX) void midm_group_kernel(int st1, int st2, int st3, int mw,
                                                               const GemvBatch<MAXI> batch) {
  const int b = (int)blockIdx.x;
  int item = 0;
  if constexpr (MAXI <= 4) {
    item = (b >= st1 ? 1 : 0) + (b >= st2 ? 1 : 0) + (b >= st3 ? 1 : 0);
  } else {
#pragma unroll
    for (int i = 1; i < MAXI; ++i) item += b >= batch.start[i] ? 1 : 0;  // starts ascend
  }
  const GemvItem& it = batch.it[item];
  midm_body<F, 1, 1, MXB>(it.q, it.s, it.x, it.y, it.N, it.K, it.g, mw, it.wg0);
}

// Workgroups of W waves of kernel `k` that one compute unit holds at once, with `lds` bytes of dynamic
// LDS each (from the occupancy calculator; remembered per wave count and LDS size class).
static int resident_per_cu(const void* k, int W, size_t lds) {
  int b = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, k, 64 * W, lds) != hipSuccess || b < 1) b = 1;
  return b;
}

template <int F, int T, int RU, int U, int MX, int MAXI, int MC, int ONE = BATCH_LOOP>
struct GemvLaunch {
  static const void* fn() {
    if constexpr (MAXI == 1) return reinterpret_cast<const void*>(&gemv_kernel<F, T, RU, U, MX, MC, ONE>);
    else return reinterpret_cast<const void*>(&gemv_group_kernel<F, T, RU, U, MX, MAXI, MC, ONE>);
  }
  static size_t lds(int W, int M) { return (size_t)W * U * 4 * x_gs(M) + (size_t)W * T * 64 * 4 * sizeof(float); }
  // workgroups resident per CU for W = 1, 2, 4, 8, 16 at this M (computed once per M class)
  static int resident(int W, int M) {
    static std::atomic<int> cache[64][5][17];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int wi = 0;
    while ((1 << wi) < W) ++wi;
    const int mi = M > 16 ? 16 : M;
    int r = cache[dev][wi][mi].load(std::memory_order_relaxed);
    if (r <= 0) {
      attr();
      r = resident_per_cu(fn(), W, lds(W, M));
      cache[dev][wi][mi].store(r, std::memory_order_relaxed);
    }
    return r;
  }
  // allow more than 64 KiB of dynamic LDS for this instantiation (once per device)
  static void attr() {
    static Fp4LdsLimit lds_limit;
    lds_limit.ensure(fn(), GEMV_LDS_MAX);
  }
  static int launch(const GemvBatch<MAXI>& b, int nwg, int W, int M, hipStream_t st) {
    attr();
    if constexpr (MAXI == 1) {
      const GemvItem& i0 = b.it[0];
      return fp4_launch(gemv_kernel<F, T, RU, U, MX, MC, ONE>, dim3(nwg), dim3(64 * W), lds(W, M), st, i0.q, i0.s, i0.x,
                        i0.y, i0.N, i0.K, i0.g, M | (W << 8));
    } else {
      const int inf = 0x7fffffff;
      return fp4_launch(gemv_group_kernel<F, T, RU, U, MX, MAXI, MC, ONE>, dim3(nwg), dim3(64 * W), lds(W, M), st,
                        MAXI > 1 ? b.start[1 % MAXI] : inf, MAXI > 2 ? b.start[2 % MAXI] : inf,
                        MAXI > 3 ? b.start[3 % MAXI] : inf, M | (W << 8), b);
    }
  }
};

// Picks the wave count of a launch: the most (up to 16, and up to wmax) that give every wave at least
// two K chunks and, for M > 1, keep the whole grid resident at once (one round of workgroups).
template <class L>
static int pick_waves(int nwg, int min_chunks, int M, int wmax) {
  const int cus = fp4_device_cus();
  int W = 16;
  // M = 1 (single-batch kernels, high occupancy): the most waves that keep two chunks per wave, even when
  // the grid then takes a second round (a wave working through more chunks costs more than the round).
  const bool fit = M > 1;
  while (W > 1 && (W > wmax || min_chunks < 2 * W || (fit && (int64_t)nwg > (int64_t)L::resident(W, M) * cus)))
    W >>= 1;
  const int tw = fp4_tuning().gemv_waves;  // tuning override
  if (tw > 0 && tw <= 16) W = tw;
  return W;
}

// One tile per workgroup: fills in the workgroup ranges; returns the workgroup count.
template <int MAXI>
static int fill_ranges(GemvBatch<MAXI>& b, int T, int& min_chunks, int& max_chunks) {
  int nwg = 0;
  min_chunks = 1 << 30;
  max_chunks = 0;
  for (int i = 0; i < b.count; ++i) {
    GemvItem& it = b.it[i];
    it.nchunk = (it.K + CHUNK_K - 1) / CHUNK_K;
    it.wg0 = nwg;
    b.start[i] = nwg;
    nwg += ((it.N + TILE_N - 1) / TILE_N + T - 1) / T;
    min_chunks = min_chunks < it.nchunk ? min_chunks : it.nchunk;
    max_chunks = max_chunks > it.nchunk ? max_chunks : it.nchunk;
  }
  for (int i = b.count; i < MAXI; ++i) b.start[i] = 0x7fffffff;
  return nwg;
}

// Launches L when its grid fits the chip in one round, else returns -1.
template <class L, int MAXI>
static int one_batch_fit(const GemvBatch<MAXI>& b, int nwg, int W, int M, hipStream_t st) {
  if ((int64_t)nwg > (int64_t)L::resident(W, M) * fp4_device_cus()) return -1;
  return L::launch(b, nwg, W, M, st);
}

// 2 <= M <= 8: every chunk of a wave in one batch, as at M = 1 (x first, then all of the wave's weight
// units, so a wave waits about one memory latency rather than one per batch). Wave count as at M = 1; up
// to 6 slots per wave with M <= 4, up to 3 with more rows of x, where the grid must also fit the chip in
// one round (the staged x of U chunks per wave then limits the workgroups per CU). Returns -1 where it does
// not apply (then nothing is launched).
template <int F, int MAXI>
static int try_one_batch(GemvBatch<MAXI>& b, int M, hipStream_t st) {
  if (M < 2 || M > 8 || fp4_tuning().one_batch == 0) return -1;
  int min_chunks, max_chunks;
  const int nwg = fill_ranges(b, 1, min_chunks, max_chunks);
  int W = pick_waves<GemvLaunch<F, 1, 4, 4, 4, MAXI, 4, ONE_CHECKED>>(nwg, min_chunks, 1, 16);
  if (W == 16 && (max_chunks + 7) / 8 <= 4) W = 8;
  const int U = (max_chunks + W - 1) / W;
  if (M <= 4 && U > 6) return -1;
  if (M == 2) return U <= 3 ? GemvLaunch<F, 1, 2, 3, 2, MAXI, 2, ONE_CHECKED>::launch(b, nwg, W, M, st)
                   : U == 4 ? GemvLaunch<F, 1, 2, 4, 2, MAXI, 2, ONE_CHECKED>::launch(b, nwg, W, M, st)
                            : GemvLaunch<F, 1, 2, 6, 2, MAXI, 2, ONE_CHECKED>::launch(b, nwg, W, M, st);
  if (M == 3) return U <= 3 ? GemvLaunch<F, 1, 4, 3, 3, MAXI, 3, ONE_CHECKED>::launch(b, nwg, W, M, st)
                   : U == 4 ? GemvLaunch<F, 1, 4, 4, 3, MAXI, 3, ONE_CHECKED>::launch(b, nwg, W, M, st)
                            : GemvLaunch<F, 1, 4, 6, 3, MAXI, 3, ONE_CHECKED>::launch(b, nwg, W, M, st);
  if (M == 4) return U <= 3 ? GemvLaunch<F, 1, 4, 3, 4, MAXI, 4, ONE_CHECKED>::launch(b, nwg, W, M, st)
                   : U == 4 ? GemvLaunch<F, 1, 4, 4, 4, MAXI, 4, ONE_CHECKED>::launch(b, nwg, W, M, st)
                            : GemvLaunch<F, 1, 4, 6, 4, MAXI, 4, ONE_CHECKED>::launch(b, nwg, W, M, st);
  if (U > 3) return -1;
  // M fixed at compile time here too (x loads and addressing for exactly M rows: 5-8% faster than a
  // runtime M bounded by 8)
  if (M == 5) return one_batch_fit<GemvLaunch<F, 1, 4, 3, 5, MAXI, 5, ONE_CHECKED>>(b, nwg, W, M, st);
  if (M == 6) return one_batch_fit<GemvLaunch<F, 1, 4, 3, 6, MAXI, 6, ONE_CHECKED>>(b, nwg, W, M, st);
  if (M == 7) return one_batch_fit<GemvLaunch<F, 1, 4, 3, 7, MAXI, 7, ONE_CHECKED>>(b, nwg, W, M, st);
  return one_batch_fit<GemvLaunch<F, 1, 4, 3, 8, MAXI, 8, ONE_CHECKED>>(b, nwg, W, M, st);
}

// The grouped mid-M kernel (one block of x rows) for a launch of one or more matrices, 5 <= M <= 16: wave
// count as for one matrix (the most, up to 16, that give every wave two chunks of the shortest K and keep
// the grid resident in one round).
template <int F, int MAXI, int WMAX, int MXB>
struct MidmGroupLaunch {
  static const void* fn() { return reinterpret_cast<const void*>(&midm_group_kernel<F, MAXI, WMAX, MXB>); }
  static size_t lds(int W, int M) {
    const size_t stage = (size_t)W * 4 * x_gs(M), red = (size_t)W * 64 * 4 * sizeof(float);
    return stage > red ? stage : red;
  }
  static int resident(int W, int M) {    // workgroups per CU (per device, wave count and M)
    static std::atomic<int> cache[64][5][17];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int wi = 0;
    while ((1 << wi) < W) ++wi;
    int r = cache[dev][wi][M].load(std::memory_order_relaxed);
    if (r <= 0) {
      static Fp4LdsLimit lds_limit;
      lds_limit.ensure(fn(), GEMV_LDS_MAX);
      r = resident_per_cu(fn(), W, lds(W, M));
      cache[dev][wi][M].store(r, std::memory_order_relaxed);
    }
    return r;
  }
  static int launch(const GemvBatch<MAXI>& b, int nwg, int W, int M, hipStream_t st) {
    static Fp4LdsLimit lds_limit;
    lds_limit.ensure(fn(), GEMV_LDS_MAX);
    const int inf = 0x7fffffff;
    return fp4_launch(midm_group_kernel<F, MAXI, WMAX, MXB>, dim3(nwg), dim3(64 * W), lds(W, M), st,
                      MAXI > 1 ? b.start[1 % MAXI] : inf, MAXI > 2 ? b.start[2 % MAXI] : inf,
                      MAXI > 3 ? b.start[3 % MAXI] : inf, M | (W << 8), b);
  }
};

template <int F, int MAXI, int MXB>
static int dispatch_midm_group_mx(GemvBatch<MAXI>& b, int M, hipStream_t st) {
  int min_chunks, max_chunks;
  const int nwg = fill_ranges(b, 1, min_chunks, max_chunks);
  const int cus = fp4_device_cus();
  int W = 16;
  while (W > 1 && (min_chunks < 2 * W ||
                   (int64_t)nwg > (int64_t)cus * (W > 8 ? MidmGroupLaunch<F, MAXI, 16, MXB>::resident(W, M)
                                                        : MidmGroupLaunch<F, MAXI, 8, MXB>::resident(W, M))))
    W >>= 1;
  const int tw = fp4_tuning().midm_waves;  // tuning override
  if (tw > 0 && tw <= 16) W = tw;
  if (W > 8) return MidmGroupLaunch<F, MAXI, 16, MXB>::launch(b, nwg, W, M, st);
  return MidmGroupLaunch<F, MAXI, 8, MXB>::launch(b, nwg, W, M, st);
}

// x loads covering 12 rows for M <= 12, else 16
template <int F, int MAXI>
static int dispatch_midm_group(GemvBatch<MAXI>& b, int M, hipStream_t st) {
  if (M <= 12) return dispatch_midm_group_mx<F, MAXI, 12>(b, M, st);
  return dispatch_midm_group_mx<F, MAXI, 16>(b, M, st);
}

// M = 1, one batch of U slots per wave (U here is the kernel's slot count, at least the slots the launch
// needs). One matrix: straight-line slots (ONE_FULL where U W = nchunk, else ONE_LAST where (U - 1) W <=
// nchunk, which U = ceil(nchunk / W) always allows; the U tuning override can break it and then takes the
// checked form). Several matrices: ONE_FULL when every one has U W chunks, else every slot is tested.
template <int F, int U, int MAXI>
static int launch_one_m1(const GemvBatch<MAXI>& b, int nwg, int W, int min_chunks, int max_chunks, hipStream_t st) {
  if constexpr (U <= 4) {
    if (min_chunks == max_chunks && U * W == max_chunks)
      return GemvLaunch<F, 1, 1, U, 1, MAXI, 1, ONE_FULL>::launch(b, nwg, W, 1, st);
  }
  if constexpr (MAXI == 1) {
    if ((U - 1) * W <= min_chunks) return GemvLaunch<F, 1, 1, U, 1, MAXI, 1, ONE_LAST>::launch(b, nwg, W, 1, st);
  }
  return GemvLaunch<F, 1, 1, U, 1, MAXI, 1, ONE_CHECKED>::launch(b, nwg, W, 1, st);
}

// Fills in the workgroup ranges, picks the variant and wave count, and launches. Every item has N, K >= 1.
template <int F, int MAXI>
static int dispatch_gemv(GemvBatch<MAXI>& b, int M, hipStream_t st) {
  const int one = try_one_batch<F, MAXI>(b, M, st);
  if (one != -1) return one;
  // From 5 rows of x on: the mid-M kernel's one-block form, per item
  if (M > 4) return dispatch_midm_group<F, MAXI>(b, M, st);
  int min_chunks, max_chunks;
  const int nwg = fill_ranges(b, 1, min_chunks, max_chunks);
  const int wmax = 16;
  if (M == 1) {
    // One batch of U chunk slots per wave when W * U covers the longest K (no prefetch registers);
    // U is the fewest slots that do at the picked wave count.
    using L4 = GemvLaunch<F, 1, 1, 4, 1, MAXI, 1>;
    using O4 = GemvLaunch<F, 1, 1, 4, 1, MAXI, 1, ONE_CHECKED>;
    int W = pick_waves<O4>(nwg, min_chunks, M, wmax);
    // 8 waves of up to 4 chunks beat 16 waves of 2 (K = 4096: 3-10% faster, fewer waves to reduce)
    const Fp4Tuning& tu = fp4_tuning();
    if (W == 16 && (max_chunks + 7) / 8 <= 4 && tu.gemv_waves < 0) W = 8;
    int U = (max_chunks + W - 1) / W;
    if (tu.gemv_u >= 2 && tu.gemv_u <= 4 && tu.gemv_u * W >= max_chunks) U = tu.gemv_u;  // tuning override
    using L2 = GemvLaunch<F, 1, 1, 2, 1, MAXI, 1>;
    const bool batch_loop = tu.gemv_one == 0;  // tuning override: batch loop with prefetch
    // Long K on a grid of at least two workgroups per CU: the ring kernel (3 chunks in flight per wave,
    // so two 16-wave workgroups fit on a CU where the batch loop fits one).
    const bool ring_fits = MAXI == 1 && max_chunks <= RING_MAX_CHUNKS;
    const bool ring = ring_fits && (tu.gemv_ring >= 0 ? tu.gemv_ring == 1 : (U > 4 && nwg >= 2 * fp4_device_cus()));
    if (ring) return RingLaunch<F, 3>::launch(b.it[0], RING_WAVES, st);
    if (batch_loop && U <= 2) return L2::launch(b, nwg, W, M, st);
    if (batch_loop && U <= 4) return L4::launch(b, nwg, W, M, st);
    // up to 6 slots in one batch (the 2560 x 9728 matrix: 5.90 -> 5.18 us against the batch loop)
    if (U <= 2) return launch_one_m1<F, 2, MAXI>(b, nwg, W, min_chunks, max_chunks, st);
    if (U == 3) return launch_one_m1<F, 3, MAXI>(b, nwg, W, min_chunks, max_chunks, st);
    if (U == 4) return launch_one_m1<F, 4, MAXI>(b, nwg, W, min_chunks, max_chunks, st);
    if (U == 5) return launch_one_m1<F, 5, MAXI>(b, nwg, W, min_chunks, max_chunks, st);
    if (U == 6) return launch_one_m1<F, 6, MAXI>(b, nwg, W, min_chunks, max_chunks, st);
    return L4::launch(b, nwg, pick_waves<L4>(nwg, min_chunks, M, wmax), M, st);
  }
  if (M == 2) {
    using L4 = GemvLaunch<F, 1, 2, 4, 2, MAXI, 2>;
    return L4::launch(b, nwg, pick_waves<L4>(nwg, min_chunks, M, wmax), M, st);
  } else if (M == 3) {
    using L4 = GemvLaunch<F, 1, 4, 4, 3, MAXI, 3>;
    return L4::launch(b, nwg, pick_waves<L4>(nwg, min_chunks, M, wmax), M, st);
  } else if (M == 4) {
    using L4 = GemvLaunch<F, 1, 4, 4, 4, MAXI, 4>;
    return L4::launch(b, nwg, pick_waves<L4>(nwg, min_chunks, M, wmax), M, st);
  }
  return -6;  // not reached: M <= 4 is handled above
}

template <int MAXI>
static int dispatch_fmt(int fmt, GemvBatch<MAXI>& b, int M, hipStream_t st) {
  switch (fmt) {
    case NVFP4: return dispatch_gemv<NVFP4>(b, M, st);
    case DUAL:  return dispatch_gemv<DUAL>(b, M, st);
    case FAST:  return dispatch_gemv<FAST>(b, M, st);
    default:    return dispatch_gemv<Q4_0>(b, M, st);
  }
}

}  // namespace fp4

using namespace fp4;

// Checks one matrix of a GEMV call; 0 or a negative status.
static int check_item(int fmt, int64_t M, int64_t N, int64_t K, const void* q, const void* s, const void* x,
                      const float* y) {
  int rc = fp4_check_nk(fmt, N, K);
  if (rc) return rc;
  if (K > (1 << 24)) return -4;  // 32-bit buffer offsets within a tile row of the planes and within x
  (void)M;
  if (!q || !s || !x || !y) return -1;
  if (!fp4_aligned(q, 16) || !fp4_aligned(s, 16) || !fp4_aligned(x, 16) || !fp4_aligned(y, 4)) return -3;
  return 0;
}

template <int F, int MB, int T, int WMAX = 8, int MXB = 16 * MB>
static int launch_midm(int W, hipStream_t st, const uint8_t* q, const uint8_t* s, const uint16_t* x, float* y,
                       int M, int N, int K, float g) {
  const int ntiles = (N + TILE_N - 1) / TILE_N;
  const size_t stage = (size_t)W * 4 * x_gs(M), red = (size_t)W * T * MB * 64 * 4 * sizeof(float);
  const size_t lds = stage > red ? stage : red;
  static Fp4LdsLimit lds_limit;
  lds_limit.ensure(reinterpret_cast<const void*>(&midm_kernel<F, MB, T, WMAX, MXB>), GEMV_LDS_MAX);
  return fp4_launch(midm_kernel<F, MB, T, WMAX, MXB>, dim3((ntiles + T - 1) / T), dim3(64 * W), lds, st, q, s, x,
                    y, N, K, g, M | (W << 8));
}

template <int F, int MXB>
static int launch_midm_mb1(int T, int W, hipStream_t st, const uint8_t* q, const uint8_t* s, const uint16_t* x,
                           float* y, int M, int N, int K, float g) {
  if (T == 2) return launch_midm<F, 1, 2, 8, MXB>(W, st, q, s, x, y, M, N, K, g);
  if (W > 8) return launch_midm<F, 1, 1, 16, MXB>(W, st, q, s, x, y, M, N, K, g);
  return launch_midm<F, 1, 1, 8, MXB>(W, st, q, s, x, y, M, N, K, g);
}

template <int F, int MB>
static int dispatch_midm_mb(int M, hipStream_t st, const uint8_t* q, const uint8_t* s, const uint16_t* x, float* y,
                             int N, int K, float g) {
  const int nchunk = (K + CHUNK_K - 1) / CHUNK_K, ntiles = (N + TILE_N - 1) / TILE_N;
  // Two tiles per workgroup share the staged x (half the x traffic) when that still leaves two
  // workgroups per CU; not with four 16-row blocks of x, where the registers would not suffice.
  const int T = (MB <= 3 && ntiles >= 2 * 2 * 256) ? 2 : 1;
  const int nwg = (ntiles + T - 1) / T;
  // Waves per workgroup: the most that give every wave at least two chunks and keep the grid resident at
  // once (16 waves per CU with two 16-row blocks of x and one tile, 8 otherwise, at this kernel's register
  // use). Up to 16 with one block of x and one tile (the kernel then fits 128 VGPRs; the staged x of 16 waves
  // is at most 66 KiB), else up to 8 (the staged x of 8 waves at M = 64 fills 129 KiB of LDS).
  const int resident = (MB <= 2 && T == 1 ? 16 : 8) * 256;
  const int wmax = (MB == 1 && T == 1) ? 16 : 8;
  int W = wmax;
  while (W > 1 && (nchunk < 2 * W || nwg * W > resident)) W >>= 1;
  const int tw = fp4_tuning().midm_waves;  // tuning override
  if (tw > 0 && tw <= wmax) W = tw;
  if constexpr (MB == 1) {
    // with one block of x rows, the x loads cover 8, 12 or 16 rows (M = 9: 6.44 -> 6.13 us on the
    // 9728 x 2560 NVFP4 matrix against a 16-row bound)
    if (M <= 8) return launch_midm_mb1<F, 8>(T, W, st, q, s, x, y, M, N, K, g);
    if (M <= 12) return launch_midm_mb1<F, 12>(T, W, st, q, s, x, y, M, N, K, g);
    return launch_midm_mb1<F, 16>(T, W, st, q, s, x, y, M, N, K, g);
  } else {
    if constexpr (MB <= 3) {
      if (T == 2) return launch_midm<F, MB, 2>(W, st, q, s, x, y, M, N, K, g);
    }
    return launch_midm<F, MB, 1>(W, st, q, s, x, y, M, N, K, g);
  }
}

template <int F>
static int dispatch_midm(int M, hipStream_t st, const uint8_t* q, const uint8_t* s, const uint16_t* x, float* y,
                         int N, int K, float g) {
  const int mb = (M + 15) / 16;
  if (mb == 1) return dispatch_midm_mb<F, 1>(M, st, q, s, x, y, N, K, g);
  if (mb == 2) return dispatch_midm_mb<F, 2>(M, st, q, s, x, y, N, K, g);
  if (mb == 3) return dispatch_midm_mb<F, 3>(M, st, q, s, x, y, N, K, g);
  return dispatch_midm_mb<F, 4>(M, st, q, s, x, y, N, K, g);
}


extern "C" int w4a16_gemv(int fmt, int64_t M, int64_t N, int64_t K, const void* q, const void* s,
                          float global_scale, const void* x_bf16, float* y, void* stream) {
  if (!fp4_valid_format(fmt)) return -1;
  if (M < 0) return -2;
  if (M > 16) return -4;
  int rc = fp4_check_nk(fmt, N, K);
  if (rc) return rc;
  if (K > (1 << 24)) return -4;
  if (M == 0) return 0;
  rc = check_item(fmt, M, N, K, q, s, x_bf16, y);
  if (rc) return rc;
  GemvBatch<1> b;
  b.count = 1;
  b.it[0] = GemvItem{(const uint8_t*)q, (const uint8_t*)s, (const uint16_t*)x_bf16, y, (int)N, (int)K, 0, 0,
                     global_scale, 0};
  if (M >= 5) {
    // From 5 rows of x on: the one-batch GEMV where its grid fits the chip in one round, else the mid-M
    // kernel (chunks in a chain per wave; with M <= 16 one block of x rows and the scales folded per group,
    // which also covers Q4_0), both faster than the GEMV's batch loop
    int one = -1;
    switch (fmt) {
      case NVFP4: one = try_one_batch<NVFP4, 1>(b, (int)M, (hipStream_t)stream); break;
      case DUAL:  one = try_one_batch<DUAL, 1>(b, (int)M, (hipStream_t)stream); break;
      case FAST:  one = try_one_batch<FAST, 1>(b, (int)M, (hipStream_t)stream); break;
      default:    one = try_one_batch<Q4_0, 1>(b, (int)M, (hipStream_t)stream); break;
    }
    if (one != -1) return one;
    hipStream_t st = (hipStream_t)stream;
    const uint8_t* qq = (const uint8_t*)q;
    const uint8_t* ss = (const uint8_t*)s;
    const uint16_t* xx = (const uint16_t*)x_bf16;
    switch (fmt) {
      case NVFP4: return dispatch_midm<NVFP4>((int)M, st, qq, ss, xx, y, (int)N, (int)K, global_scale);
      case DUAL:  return dispatch_midm<DUAL>((int)M, st, qq, ss, xx, y, (int)N, (int)K, global_scale);
      case FAST:  return dispatch_midm<FAST>((int)M, st, qq, ss, xx, y, (int)N, (int)K, global_scale);
      default:    return dispatch_midm_mb<Q4_0, 1>((int)M, st, qq, ss, xx, y, (int)N, (int)K, global_scale);
    }
  }
  return dispatch_fmt(fmt, b, (int)M, (hipStream_t)stream);
}

template <int MAXI>
static void fill_batch(GemvBatch<MAXI>& b, int count, const fp4_gemv_item* items) {
  b.count = count;
  for (int i = 0; i < count; ++i) {
    const fp4_gemv_item& it = items[i];
    b.it[i] = GemvItem{(const uint8_t*)it.q, (const uint8_t*)it.s, (const uint16_t*)it.x_bf16, it.y, (int)it.N,
                       (int)it.K, 0, 0, it.global_scale, 0};
  }
  for (int i = count; i < MAXI; ++i) b.it[i] = GemvItem{};
}

extern "C" int w4a16_gemv_batched(int fmt, int64_t M, int count, const fp4_gemv_item* items, void* stream) {
  if (!fp4_valid_format(fmt)) return -1;
  if (M < 0) return -2;
  if (M > 16) return -4;
  if (count < 0) return -1;
  if (count > FP4_GEMV_MAX_ITEMS) return -4;
  if (count > 0 && !items) return -1;
  if (M == 0 || count == 0) return 0;
  for (int i = 0; i < count; ++i) {
    const fp4_gemv_item& it = items[i];
    const int rc = check_item(fmt, M, it.N, it.K, it.q, it.s, it.x_bf16, it.y);
    if (rc) return rc;
  }
  // one matrix takes the one-matrix kernel (all of its arguments preloaded); up to 4 pass a 4-entry table
  // (a smaller kernel-argument block, starts preloaded), else 32
  if (count == 1) {
    GemvBatch<1> b;
    fill_batch(b, count, items);
    return dispatch_fmt(fmt, b, (int)M, (hipStream_t)stream);
  }
  if (count <= 4) {
    GemvBatch<4> b;
    fill_batch(b, count, items);
    return dispatch_fmt(fmt, b, (int)M, (hipStream_t)stream);
  }
  GemvBatch<FP4_GEMV_MAX_ITEMS> b;
  fill_batch(b, count, items);
  return dispatch_fmt(fmt, b, (int)M, (hipStream_t)stream);
}

// Mid-M entry point (17 <= M <= 64 through w4a16_matmul; any 1 <= M <= 64 accepted).
extern "C" int w4a16_midm(int fmt, int64_t M, int64_t N, int64_t K, const void* q, const void* s,
                          float global_scale, const void* x_bf16, float* y, void* stream) {
  if (!fp4_valid_format(fmt)) return -1;
  if (M < 0) return -2;
  if (M > 64) return -4;
  if (fmt == Q4_0) return -4;  // its FP16-scaled weights are not exact in bf16; Q4_0 runs through the GEMV
  int rc = fp4_check_nk(fmt, N, K);
  if (rc) return rc;
  if (K > (1 << 24)) return -4;
  if (M == 0) return 0;
  rc = check_item(fmt, M, N, K, q, s, x_bf16, y);
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  const uint8_t* qq = (const uint8_t*)q;
  const uint8_t* ss = (const uint8_t*)s;
  const uint16_t* xx = (const uint16_t*)x_bf16;
  switch (fmt) {
    case NVFP4: return dispatch_midm<NVFP4>((int)M, st, qq, ss, xx, y, (int)N, (int)K, global_scale);
    case DUAL:  return dispatch_midm<DUAL>((int)M, st, qq, ss, xx, y, (int)N, (int)K, global_scale);
    default:    return dispatch_midm<FAST>((int)M, st, qq, ss, xx, y, (int)N, (int)K, global_scale);
  }
}
