// Prefill-shaped W4A16 product (any M >= 1; intended for M >= 64).
//
// A workgroup of 4 waves computes a 256 x 256 tile of y; wave w owns all 256 rows of the tile and weight rows
// 64 w .. 64 w + 63, so every weight is dequantized exactly once per workgroup. The K loop runs over pipeline
// stages of 64 positions: stage h is half hh = h % 2 of 128-wide chunk c = h / 2, i.e. lane pieces g = 2 hh
// and 2 hh + 1 of every packed unit.
//  * All global reads are buffer loads that write LDS directly (no registers), into a 3-deep ring, two
//    stages ahead of use: the 256 x 64 x-values of the stage (natural k order over the stage's k subset,
//    16-byte segments XOR-swizzled by row so the MFMA operand reads have no bank conflicts), each wave's
//    packed weight bytes and scale bytes.
//  * Each wave reads its packed weights back and dequantizes them straight into bf16 MFMA B operands as
//    exact level * scale; x fragments are the A operands. bf16 MFMA 32x32x16, FP32 accumulators. The
//    k-steps are software-pipelined: the next k-step's A reads and B dequantization are issued before the
//    current k-step's MFMAs so that one wave per SIMD keeps the matrix core busy.
//  * The epilogue multiplies by g and stores fp32 y.
// Rows beyond M / N and columns beyond K come back as zeros from the buffer loads (raw buffers return zero
// past num_records), so the loop has no bounds branches.
#include "common.h"
#include "launch.h"
#include "fp4w4a16.h"
#include <atomic>
#include <stdlib.h>

namespace fp4 {

constexpr int GM_BM = 256, GM_BN = 256, GM_WAVES = 4, GM_THREADS = 64 * GM_WAVES;
constexpr int GM_STAGE_K = 64;                        // positions per pipeline stage
constexpr int GM_ROW_BYTES = GM_STAGE_K * 2;          // 128 bytes of x per row and stage
constexpr int GM_X_BYTES = GM_BM * GM_ROW_BYTES;      // 32 KiB of x per stage
constexpr int GM_W_BYTES = GM_WAVES * 4 * 512;        // per wave: 4 tiles x 2 lane pieces of 256 B
constexpr int GM_S_BYTES = GM_WAVES * 4 * 128;        // per wave: 4 tiles x scale bytes (<= 128 each)
constexpr int GM_STAGE_BYTES = GM_X_BYTES + GM_W_BYTES + GM_S_BYTES;  // 42 KiB
constexpr int GM_RING = 3;
constexpr int GM_LDS = GM_RING * GM_STAGE_BYTES;      // 126 KiB
// A tile has 32 MI rows of x: MI = 8 (256 rows) or 6 (192 rows, the shorter tiles that even out the last
// round of a grid). A thread then has MI 16-byte x slots per stage (each 8 rows below the previous).
// Vector-memory instructions per thread per stage: x slots, 2 weight loads, scale loads (512 or 256 bytes).
// NB = 32-column blocks of weight rows per wave: 2 (256-column tiles) or 1 (128-column tiles for small grids).
// Scale-byte loads per stage: 4-byte loads of the 2 NB tiles' scale rows, 64 lanes each (at least one).
__host__ __device__ constexpr int gm_scale_parts(int f, int nb) {
  return 2 * nb * (unit_s(f) / 4) / 64 > 1 ? 2 * nb * (unit_s(f) / 4) / 64 : 1;
}
__host__ __device__ constexpr int gm_loads_per_stage(int f, int mi, int nb = 2) { return mi + nb + gm_scale_parts(f, nb); }
// Stage layout per tile shape: x, then each wave's weight pieces, then each wave's scale bytes. 256-column
// tiles (NB = 2) keep the layout above whatever MI (32 KiB of x, 2 KiB of weights and 512 B of scales per
// wave: 42 KiB); 128-column tiles (NB = 1) take only what they use (32 MI rows of x, 1 KiB and 256 B per
// wave), so a ring of 128-row tiles fits in 63 KiB and two workgroups can share a CU.
__host__ __device__ constexpr int gm_x_bytes(int mi, int nb) { return nb == 2 ? GM_X_BYTES : mi * 32 * GM_ROW_BYTES; }
__host__ __device__ constexpr int gm_w_wave(int nb) { return 1024 * nb; }
__host__ __device__ constexpr int gm_s_wave(int nb) { return 256 * nb; }
__host__ __device__ constexpr int gm_stage_bytes(int mi, int nb) {
  return gm_x_bytes(mi, nb) + GM_WAVES * (gm_w_wave(nb) + gm_s_wave(nb));
}
__host__ __device__ constexpr int gm_lds(int mi, int nb) { return GM_RING * gm_stage_bytes(mi, nb); }
static_assert(gm_stage_bytes(8, 2) == GM_STAGE_BYTES && gm_stage_bytes(6, 2) == GM_STAGE_BYTES, "prefill layout");
constexpr int GM_SHORT_ROWS = 192;   // rows of an MI = 6 tile
constexpr int GM_SHORT_BANDS = 8;    // MI = 6 tiles cover rows 0 .. 8 * 192 - 1 of their columns
constexpr int64_t GM_SPLIT_MAX_OUT = 5 << 19;  // most outputs (M N) for which a small grid splits K in two

typedef float f32x16 __attribute__((ext_vector_type(16)));

// This lane's weight bytes for one stage, read back from LDS: for each of the wave's two 32-row column
// tiles, dwords 2 kh and 2 kh + 1 of the row's two lane pieces, and the row's scale bytes of the chunk that
// its k half (kh) uses: bytes 4 kh .. 4 kh + 3 of 8 (16-weight groups), or 2 kh, 2 kh + 1 of 4 (FAST), so
// that the byte a k-step needs is a constant index.
struct WRegs {
  u32x2 w[2][2];
  uint32_t sc[2];
};

// Buffer descriptors (raw, stride 0): loads past num_records return zeros.
struct GemmSrc {
  __amdgpu_buffer_rsrc_t x, q, s;
};

// Stage k subset and its natural order (segment sigma = 16-byte group of 8 positions, 8 per stage):
//   16-weight groups: sigma = j -> k = 16 sigma + 8 hh + u          (u = 0..7; group j of the chunk)
//   FAST:             sigma = 2 j + b -> k = 32 j + 16 hh + 8 b + u (block j of the chunk)
template <int F>
__device__ __forceinline__ int stage_k(int c, int hh, int sigma) {
  return c * CHUNK_K + (F == FAST ? 32 * (sigma >> 1) + 16 * hh + 8 * (sigma & 1) : 16 * sigma + 8 * hh);
}

// Segment swizzle of x row `row` in a stage: any 8 consecutive rows (aligned) use 8 different 16-byte
// segments, and within any 16 aligned rows the even rows and the odd rows each use 8 different ones, so
// the MFMA operand reads (8 or 16 lanes per LDS access, consecutive rows) have no bank conflicts.
__device__ __forceinline__ int x_swizzle(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// x of stage h: global -> its LDS ring slot `base`, one 16-byte direct load per slot. Slot S of the stage
// holds row S / 8, physical segment S % 8 = sigma ^ x_swizzle(row).
template <int F, int MI, bool RAGGED, int NB = 2>
__device__ __forceinline__ void issue_x(const GemmSrc& src, uint8_t* base, int h, int K, int wave, int lane) {
  const int c = h >> 1, hh = h & 1;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int first = (wave * MI + i) * 64;                  // first slot of this instruction (uniform)
    const int slot = first + lane;
    const int row = slot >> 3, sigma = (slot & 7) ^ x_swizzle(row);
    const int k = stage_k<F>(c, hh, sigma);
    const uint32_t off = (!RAGGED || k < K) ? (uint32_t)(row * K + k) * 2u : 0xFFFFFFF0u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.x, (__attribute__((address_space(3))) void*)(base + first * 16),
                                             16, off, 0, 0, 0);
  }
}

// Weights of stage h: the two lane pieces 2 hh, 2 hh + 1 of a unit are 512 contiguous bytes, so the wave's four
// tiles take 2 KiB (two 16-byte direct loads per lane), plus the scale bytes of the same four tiles.
template <int F, int MI, int NB = 2>
__device__ __forceinline__ void issue_w(const GemmSrc& src, uint8_t* stage, int h, int nchunk, int wave, int lane) {
  const int c = h >> 1, hh = h & 1;
  constexpr int XB = gm_x_bytes(MI, NB), WB = GM_WAVES * gm_w_wave(NB);
#pragma unroll
  for (int part = 0; part < NB; ++part) {
    const int tt = 2 * part + (lane >> 5);
    const uint32_t off = (uint32_t)(tt * nchunk + c) * UNIT_Q + 512 * hh + (lane & 31) * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        src.q, (__attribute__((address_space(3))) void*)(stage + XB + wave * gm_w_wave(NB) + part * 1024), 16, off,
        0, 0, 0);
  }
  constexpr int us = unit_s(F);                   // 128 (16-weight groups) or 64 (FAST) bytes per unit
  constexpr int lanes_per_tile = us / 4;          // 4-byte loads
  constexpr int parts = gm_scale_parts(F, NB);    // 2 or 1
#pragma unroll
  for (int part = 0; part < parts; ++part) {
    const int idx = part * 64 + lane;
    const int tt = idx / lanes_per_tile;
    const uint32_t off = (uint32_t)(tt * nchunk + c) * us + (idx % lanes_per_tile) * 4;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        src.s, (__attribute__((address_space(3))) void*)(stage + XB + WB + wave * gm_s_wave(NB) + part * 256), 4, off,
        0, 0, 0);
  }
}

// Per-lane parts of the direct-load offsets, computed once per tile. Rows and tiles stay in the
// per-lane (range-checked) offset: x slot i of a lane is 8 rows below slot 0 (its segment differs in the
// swizzle's parity bit for odd i, hence two x offsets), the second weight and scale parts two tiles
// further, each one add per load. Only the stage term (chunk, half-chunk), which stays inside a row of x
// and a tile's row of units, goes into the scalar offset.
struct LoadOffs {
  uint32_t x[2], w, s;
};

template <int F>
__host__ __device__ constexpr int seg_k(int sigma) {   // stage_k without the chunk and half-chunk terms
  return (F == FAST) ? 32 * (sigma >> 1) + 8 * (sigma & 1) : 16 * sigma;
}

template <int F, int MI>
__device__ __forceinline__ void load_offsets(LoadOffs& o, int K, int nchunk, int wave, int lane) {
  const int row = wave * 8 * MI + (lane >> 3);          // slot 0 of the lane: row of x in the tile
  const int sigma = (lane & 7) ^ x_swizzle(row);
  o.x[0] = (uint32_t)(row * K + seg_k<F>(sigma)) * 2u;
  o.x[1] = (uint32_t)(row * K + seg_k<F>(sigma ^ 1)) * 2u;
  o.w = (uint32_t)((lane >> 5) * nchunk) * UNIT_Q + (lane & 31) * 16;
  constexpr int us = unit_s(F), lanes_per_tile = us / 4;
  o.s = (uint32_t)((lane / lanes_per_tile) * nchunk) * us + (lane % lanes_per_tile) * 4;
}

// Part P (0, 1, 2) of stage h's direct loads (K a multiple of 128): x slots 3P .. 3P + 2 (the last part
// has two), then in part 1 the weight pieces and in part 2 the scale bytes. Spreading a stage's loads over
// three k-steps keeps each burst of vector-memory issue short.
template <int F, int MI, int P, int NB = 2>
__device__ __forceinline__ void issue_stage_part(const GemmSrc& src, const LoadOffs& o, uint8_t* stage, int h, int K,
                                                 int nchunk, int wave) {
  const int c = h >> 1, hh = h & 1;
  constexpr int XB = gm_x_bytes(MI, NB), WB = GM_WAVES * gm_w_wave(NB);
  const int xs = 2 * (c * CHUNK_K + hh * (F == FAST ? 16 : 8));
  const uint32_t xrow8 = (uint32_t)K * 16u;                 // 8 rows of bf16
#pragma unroll
  for (int i = 3 * P; i < 3 * P + 3 && i < MI; ++i) {
    const int first = (wave * MI + i) * 64;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.x, (__attribute__((address_space(3))) void*)(stage + first * 16), 16,
                                             o.x[i & 1] + i * xrow8, xs, 0, 0);
  }
  if constexpr (P == 1) {
    const int ws = c * UNIT_Q + 512 * hh;
#pragma unroll
    for (int part = 0; part < NB; ++part)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          src.q, (__attribute__((address_space(3))) void*)(stage + XB + wave * gm_w_wave(NB) + part * 1024), 16,
          o.w + (uint32_t)(part * 2 * nchunk * UNIT_Q), ws, 0, 0);
  }
  if constexpr (P == 2) {
    constexpr int us = unit_s(F), parts = gm_scale_parts(F, NB);
    const int ss = c * us;
#pragma unroll
    for (int part = 0; part < parts; ++part)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          src.s, (__attribute__((address_space(3))) void*)(stage + XB + WB + wave * gm_s_wave(NB) + part * 256), 4,
          o.s + (uint32_t)(part * 2 * nchunk * us), ss, 0, 0);
  }
}

// Load I (0 .. MI + 3) of stage h's direct loads (K a multiple of 128): x slots 0 .. MI - 1, the two weight
// pieces, then the scale loads (two for 16-weight groups, one for FAST). Issued one or two at a time between
// MFMAs so that no burst of vector-memory instructions holds up the wave.
template <int F, int MI, int I, int NB = 2>
__device__ __forceinline__ void issue_stage_one(const GemmSrc& src, const LoadOffs& o, uint8_t* stage, int h, int K,
                                                int nchunk, int wave) {
  const int c = h >> 1, hh = h & 1;
  constexpr int XB = gm_x_bytes(MI, NB), WB = GM_WAVES * gm_w_wave(NB);
  if constexpr (I < MI) {
    const int xs = 2 * (c * CHUNK_K + hh * (F == FAST ? 16 : 8));
    const uint32_t xrow8 = (uint32_t)K * 16u;               // 8 rows of bf16
    const int first = (wave * MI + I) * 64;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.x, (__attribute__((address_space(3))) void*)(stage + first * 16), 16,
                                             o.x[I & 1] + I * xrow8, xs, 0, 0);
  } else if constexpr (I < MI + NB) {
    constexpr int part = I - MI;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        src.q, (__attribute__((address_space(3))) void*)(stage + XB + wave * gm_w_wave(NB) + part * 1024), 16,
        o.w + (uint32_t)(part * 2 * nchunk * UNIT_Q), c * UNIT_Q + 512 * hh, 0, 0);
  } else {
    constexpr int us = unit_s(F), parts = gm_scale_parts(F, NB);
    constexpr int part = I - MI - NB;
    if constexpr (part < parts)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          src.s, (__attribute__((address_space(3))) void*)(stage + XB + WB + wave * gm_s_wave(NB) + part * 256), 4,
          o.s + (uint32_t)(part * 2 * nchunk * us), c * us, 0, 0);
  }
}

// All of stage h's loads into its ring slot `stage`: the three parts, or the per-slot path when K is ragged.
template <int F, int MI, bool RAGGED, int NB = 2>
__device__ __forceinline__ void issue_stage(const GemmSrc& src, const LoadOffs& o, uint8_t* stage, int h, int K,
                                            int nchunk, int wave, int lane) {
  if constexpr (RAGGED) {
    issue_x<F, MI, RAGGED, NB>(src, stage, h, K, wave, lane);
    issue_w<F, MI, NB>(src, stage, h, nchunk, wave, lane);
  } else {
    issue_stage_part<F, MI, 0, NB>(src, o, stage, h, K, nchunk, wave);
    issue_stage_part<F, MI, 1, NB>(src, o, stage, h, K, nchunk, wave);
    issue_stage_part<F, MI, 2, NB>(src, o, stage, h, K, nchunk, wave);
  }
}

template <int MI, int NB = 2>
__device__ __forceinline__ void read_w(WRegs& r, const uint8_t* stage, int F_spr, int F_us, int wave, int lane) {
  constexpr int XB = gm_x_bytes(MI, NB), WB = GM_WAVES * gm_w_wave(NB);
  const int kh = lane >> 5;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int rl = 32 * j + (lane & 31);
    const int t = rl >> 4, n = rl & 15;
    const uint8_t* wb = stage + XB + wave * gm_w_wave(NB) + t * 512 + n * 16 + 8 * kh;
    r.w[j][0] = *reinterpret_cast<const u32x2*>(wb);
    r.w[j][1] = *reinterpret_cast<const u32x2*>(wb + 256);
    const uint8_t* sb = stage + XB + WB + wave * gm_s_wave(NB) + t * F_us + n * F_spr;
    if (F_spr == 4) r.sc[j] = *reinterpret_cast<const uint16_t*>(sb + 2 * kh);
    else r.sc[j] = *reinterpret_cast<const uint32_t*>(sb + 4 * kh);
  }
}

// Workgroup barrier without a memory fence; the "memory" clobber keeps the compiler from moving LDS
// accesses across it. The waits that make the LDS data complete are explicit (wait_vmcnt).
__device__ __forceinline__ void workgroup_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt with only a vector-memory bound (gfx9 encoding: vmcnt in bits 3:0 and 15:14)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Dequantization of one B operand (k-step S, column tile j) in four slices, so that the work can be
// spread between the MFMAs of the previous k-step: scale and byte lookup, pair converts to FP32, then
// the two halves of "times scale, round to bf16" (exact). The operand is 8 consecutive positions of the
// stage's k subset for weight row 32 j + lane % 32, taken from this lane's two dwords of lane pieces
// 2 hh and 2 hh + 1 (w0, w1):
//   FAST:  dword S / 2 of piece S % 2, positions in lane-piece order;
//   Dual:  the low (S even) or high nibbles of dword S / 2 of each piece: 4 positions from each;
//   NVFP4: 16-bit half S % 2 of dword S / 2 of each piece (4 nibbles each), joined into one dword.
struct BDec {
  uint32_t q0, q1;
  f32x2 p[4];
  float sc;
};

template <int F, int S, int SL>
__device__ __forceinline__ void b_slice(BDec& d, u32x4& out, const WRegs& r, int j) {
  if constexpr (SL == 0) {
    d.sc = __builtin_amdgcn_cvt_f32_fp8(r.sc[j], F == FAST ? (S >> 1) : S);   // scale byte of this k-step
    const u32x2 w0 = r.w[j][0], w1 = r.w[j][1];
    if constexpr (F == FAST) {
      const uint32_t w = (S & 1) ? w1[S >> 1] : w0[S >> 1];
      d.q0 = cb10_quad<false>(w);
      d.q1 = cb10_quad<true>(w);
    } else if constexpr (F == DUAL) {
      d.q0 = cb10_quad<(S & 1) != 0>(w0[S >> 1]);
      d.q1 = cb10_quad<(S & 1) != 0>(w1[S >> 1]);
    } else {
      d.q0 = __builtin_amdgcn_perm(w1[S >> 1], w0[S >> 1], (S & 1) ? 0x07060302u : 0x05040100u);
    }
  } else if constexpr (SL == 1) {
    if constexpr (F == NVFP4) {
      d.p[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d.q0, 1.0f, 0);
      d.p[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d.q0, 1.0f, 1);
      d.p[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d.q0, 1.0f, 2);
      d.p[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d.q0, 1.0f, 3);
    } else {
      d.p[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d.q0, 1.0f, false);
      d.p[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d.q0, 1.0f, true);
      d.p[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d.q1, 1.0f, false);
      d.p[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d.q1, 1.0f, true);
    }
  } else if constexpr (SL == 2) {
    out[0] = pack_bf16x2(d.p[0][0] * d.sc, d.p[0][1] * d.sc);
    out[1] = pack_bf16x2(d.p[1][0] * d.sc, d.p[1][1] * d.sc);
  } else {
    out[2] = pack_bf16x2(d.p[2][0] * d.sc, d.p[2][1] * d.sc);
    out[3] = pack_bf16x2(d.p[3][0] * d.sc, d.p[3][1] * d.sc);
  }
}

// The same dequantization in eight smaller pieces (one per MFMA of a group of four), so that each runs
// in the shadow of a single MFMA: scale and low lookup, high lookup, two pair converts each, then the
// four "times scale, pack" steps.
template <int F, int S, int SUB>
__device__ __forceinline__ void b_sub(BDec& d, u32x4& out, const WRegs& r, int j) {
  const u32x2 w0 = r.w[j][0], w1 = r.w[j][1];
  if constexpr (SUB == 0) {
    d.sc = __builtin_amdgcn_cvt_f32_fp8(r.sc[j], F == FAST ? (S >> 1) : S);
    if constexpr (F == FAST) d.q0 = cb10_quad<false>((S & 1) ? w1[S >> 1] : w0[S >> 1]);
    else if constexpr (F == DUAL) d.q0 = cb10_quad<(S & 1) != 0>(w0[S >> 1]);
    else d.q0 = __builtin_amdgcn_perm(w1[S >> 1], w0[S >> 1], (S & 1) ? 0x07060302u : 0x05040100u);
  } else if constexpr (SUB == 1) {
    if constexpr (F == FAST) d.q1 = cb10_quad<true>((S & 1) ? w1[S >> 1] : w0[S >> 1]);
    else if constexpr (F == DUAL) d.q1 = cb10_quad<(S & 1) != 0>(w1[S >> 1]);
  } else if constexpr (SUB == 2) {
    if constexpr (F == NVFP4) {
      d.p[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d.q0, 1.0f, 0);
      d.p[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d.q0, 1.0f, 1);
    } else {
      d.p[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d.q0, 1.0f, false);
      d.p[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d.q0, 1.0f, true);
    }
  } else if constexpr (SUB == 3) {
    if constexpr (F == NVFP4) {
      d.p[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d.q0, 1.0f, 2);
      d.p[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d.q0, 1.0f, 3);
    } else {
      d.p[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d.q1, 1.0f, false);
      d.p[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d.q1, 1.0f, true);
    }
  } else {
    constexpr int e = SUB - 4;
    out[e] = pack_bf16x2(d.p[e][0] * d.sc, d.p[e][1] * d.sc);
  }
}

// Per-lane LDS offsets of x fragment 0 for each ring slot and k-step S: row r = lane % 32, segment
// sigma = 4 kh + S, swizzled. Fragment i (rows 32 i + r) has r's swizzle (the swizzle reads bits 0-3 of
// the row), so it sits a constant 32 rows further: reads need no per-fragment address arithmetic.
struct XBase {
  uint32_t v[GM_RING][4];
};

template <int MI, int NB>
__device__ __forceinline__ void x_bases(XBase& xb, int lane) {
  const int r = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int slot = 0; slot < GM_RING; ++slot)
#pragma unroll
    for (int S = 0; S < 4; ++S)
      xb.v[slot][S] = (uint32_t)(slot * gm_stage_bytes(MI, NB) + r * GM_ROW_BYTES + 16 * ((4 * kh + S) ^ x_swizzle(r)));
}

// x fragment i (rows 32 i .. 32 i + 31) at per-lane offset `base` of fragment 0.
__device__ __forceinline__ bf16x8 a_frag(const uint8_t* ring, uint32_t base, int i) {
  return *reinterpret_cast<const bf16x8*>(ring + base + 32 * GM_ROW_BYTES * i);
}

// Operands of one k-step, double-buffered across k-steps.
template <int MI>
struct KOps {
  bf16x8 a[MI];
  u32x4 b[2];
};

// The next k-step's operands, prepared in eight slices (x fragment G when the tile has it, and quarter G % 4
// of B operand G / 4).
template <int F, int MI, int S, int G, int NB = 2>
__device__ __forceinline__ void prep_slice(KOps<MI>& nx, BDec (&d)[2], const WRegs& r, const uint8_t* ring,
                                           uint32_t xbase) {
  if constexpr (G < MI) nx.a[G] = a_frag(ring, xbase, G);
  if constexpr ((G >> 2) < NB) b_slice<F, S, G & 3>(d[G >> 2], nx.b[G >> 2], r, G >> 2);
}

// The B dequantization pieces (b_sub) that run after MFMA slot SLOT (0 .. 2 MI - 1) of a k-step. With 16
// MFMAs (MI = 8) slot s takes piece s % 8 of operand s / 8; with 12 (MI = 6) each operand's six slots take
// pieces 0, 1, 2, 3, then 4 and 5, then 6 and 7; with 8 (MI = 4) slot s takes pieces 2 (s % 4) and
// 2 (s % 4) + 1 of operand s / 4.
template <int F, int MI, int S, int SLOT>
__device__ __forceinline__ void b_slot(BDec (&d)[2], u32x4 (&b)[2], const WRegs& r) {
  if constexpr (MI == 8) {
    constexpr int t = SLOT >> 3, q = SLOT & 7;
    b_sub<F, S, q>(d[t], b[t], r, t);
  } else if constexpr (MI == 4) {
    constexpr int t = SLOT >> 2, q = 2 * (SLOT & 3);
    b_sub<F, S, q>(d[t], b[t], r, t);
    b_sub<F, S, q + 1>(d[t], b[t], r, t);
  } else {
    constexpr int t = SLOT / 6, q = SLOT % 6;
    if constexpr (q < 4) {
      b_sub<F, S, q>(d[t], b[t], r, t);
    } else {
      b_sub<F, S, 4 + 2 * (q - 4)>(d[t], b[t], r, t);
      b_sub<F, S, 5 + 2 * (q - 4)>(d[t], b[t], r, t);
    }
  }
}

template <int MI, int G, int J>
__device__ __forceinline__ void mfma_one(f32x16 (&acc)[MI][2], const KOps<MI>& k) {
  acc[G][J] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k.a[G], __builtin_bit_cast(bf16x8, k.b[J]), acc[G][J], 0, 0, 0);
}

template <int MI, int G, int NB = 2>
__device__ __forceinline__ void mfma_group(f32x16 (&acc)[MI][2], const KOps<MI>& k) {
  const bf16x8 b0 = __builtin_bit_cast(bf16x8, k.b[0]);
  acc[G][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k.a[G], b0, acc[G][0], 0, 0, 0);
  if constexpr (NB == 2) {
    const bf16x8 b1 = __builtin_bit_cast(bf16x8, k.b[1]);
    acc[G][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k.a[G], b1, acc[G][1], 0, 0, 0);
  }
}

// Direct loads to issue during a k-step: part P of stage h (nothing when h is past the last stage).
struct StageLoads {
  const GemmSrc* src;
  const LoadOffs* o;
  uint8_t* dst;  // ring slot of stage h
  int h, K, nchunk, wave, lane;
};

// The loads of issue point Q (0 .. 3 MI / 2 - 1): load I goes out at point I * points / loads, so the
// stage's loads spread evenly (one per point with MI = 8, where the points and the loads are both 12; the
// first point takes two with MI = 6).
template <int F, int MI, int Q, int NB = 2, int I = 0>
__device__ __forceinline__ void issue_point(const StageLoads& L) {
  constexpr int NL = gm_loads_per_stage(F, MI, NB), NP = 3 * MI / 2;
  if constexpr (I < NL) {
    if constexpr (I * NP / NL == Q) issue_stage_one<F, MI, I, NB>(*L.src, *L.o, L.dst, L.h, L.K, L.nchunk, L.wave);
    issue_point<F, MI, Q, NB, I + 1>(L);
  }
}

// Loads issued after MFMA group G of k-step S: with K ragged, all of the stage at once (k-step 0, group 1);
// otherwise issue point S MI / 2 + G / 2 after each odd group of k-steps 0-2.
template <int F, int MI, bool RAGGED, int S, int G, int NB = 2>
__device__ __forceinline__ void issue_part(const StageLoads& L) {
  if constexpr (RAGGED) {
    if constexpr (S == 0 && G == 1)
      issue_stage<F, MI, true, NB>(*L.src, *L.o, L.dst, L.h, L.K, L.nchunk, L.wave, L.lane);
  } else {
    if constexpr (S < 3 && (G & 1)) issue_point<F, MI, S * (MI / 2) + (G >> 1), NB>(L);
  }
}

// One k-step of the wave's 32 MI x 64 tile: MI groups of 2 MFMAs (x fragment G against both column
// tiles), each MFMA followed by its share of the next k-step's operands (k-step S + 1 of this stage); after
// odd groups of k-steps 0-2 the wave issues loads of two stages ahead. Scheduling fences keep that order,
// so the LDS reads, VALU work and loads run while the matrix core is busy.
template <int F, int MI, bool RAGGED, int S, bool LOAD, int NB = 2>
__device__ __forceinline__ void kstep(f32x16 (&acc)[MI][2], const KOps<MI>& cur, KOps<MI>& nx, const WRegs& r,
                                      const uint8_t* ring, const uint32_t (&xc)[4], const StageLoads& L) {
  BDec d[2];
  // NB = 2: two MFMAs per x fragment G, each followed by a B-operand piece; NB = 1: one MFMA and one slot
#define FP4_GROUP(G)                                                      \
  if constexpr ((G) < MI) {                                               \
    mfma_one<MI, G, 0>(acc, cur);                                         \
    nx.a[G] = a_frag(ring, xc[S + 1], G);                                 \
    if constexpr (NB == 2) {                                              \
      b_slot<F, MI, S + 1, 2 * (G)>(d, nx.b, r);                          \
      __builtin_amdgcn_sched_barrier(0);                                  \
      mfma_one<MI, G, 1>(acc, cur);                                       \
      b_slot<F, MI, S + 1, 2 * (G) + 1>(d, nx.b, r);                      \
    } else {                                                              \
      b_slot<F, MI, S + 1, G>(d, nx.b, r);                                \
    }                                                                     \
    if constexpr (LOAD) issue_part<F, MI, RAGGED, S, G, NB>(L);           \
    __builtin_amdgcn_sched_barrier(0);                                    \
  }
  FP4_GROUP(0) FP4_GROUP(1) FP4_GROUP(2) FP4_GROUP(3) FP4_GROUP(4) FP4_GROUP(5) FP4_GROUP(6) FP4_GROUP(7)
#undef FP4_GROUP
}

// Operands of k-step 0 of a stage, all at once (the first stage only; later stages prepare them inside
// the previous stage's last k-step).
template <int F, int MI, int NB = 2>
__device__ __forceinline__ void prep_all0(KOps<MI>& k, const WRegs& r, const uint8_t* ring, uint32_t xb0) {
  BDec d[2];
  prep_slice<F, MI, 0, 0, NB>(k, d, r, ring, xb0); prep_slice<F, MI, 0, 1, NB>(k, d, r, ring, xb0);
  prep_slice<F, MI, 0, 2, NB>(k, d, r, ring, xb0); prep_slice<F, MI, 0, 3, NB>(k, d, r, ring, xb0);
  prep_slice<F, MI, 0, 4, NB>(k, d, r, ring, xb0); prep_slice<F, MI, 0, 5, NB>(k, d, r, ring, xb0);
  prep_slice<F, MI, 0, 6, NB>(k, d, r, ring, xb0); prep_slice<F, MI, 0, 7, NB>(k, d, r, ring, xb0);
}

// Stage h of the K loop (see the kernel). LOAD: the stage issues stage h + 2's loads; MORE: there is a
// stage h + 1, whose k-step 0 operands this stage prepares into ka. SLOT = h % 3 when known at compile
// time (the ring offsets are then constants), else -1. With SETS = 2 wave sets sharing the K range, h
// counts this set's own stages (ring slots), and the stage of K that it stands for is h0 + 2 h.
template <int F, int MI, bool RAGGED, bool LOAD, bool MORE, int SLOT = -1, int NB = 2, int SETS = 1>
__device__ __forceinline__ void stage_body(f32x16 (&acc)[MI][2], KOps<MI>& ka, KOps<MI>& kb, WRegs& r,
                                           const GemmSrc& src, const LoadOffs& lo, uint8_t* ring, const XBase& xb, int h, int K,
                                           int nchunk, int wave, int lane, int h0 = 0) {
  constexpr int LPS = gm_loads_per_stage(F, MI, NB);
  const int s0 = SLOT >= 0 ? SLOT : h % GM_RING;
  const int s1 = SLOT >= 0 ? (SLOT + 1) % GM_RING : (s0 == GM_RING - 1 ? 0 : s0 + 1);
  const int s2 = SLOT >= 0 ? (SLOT + 2) % GM_RING : (s1 == GM_RING - 1 ? 0 : s1 + 1);
  constexpr int SB = gm_stage_bytes(MI, NB);
  const StageLoads L{&src, &lo, ring + s2 * SB, h0 + SETS * (h + 2), K, nchunk, wave, lane};
  // this stage's and the next stage's per-lane fragment offsets (registers when the slot is known)
  uint32_t xc[4], xn[4];
#pragma unroll
  for (int S = 0; S < 4; ++S) {
    if constexpr (SLOT >= 0) {
      xc[S] = xb.v[SLOT][S];
      xn[S] = xb.v[(SLOT + 1) % GM_RING][S];
    } else {
      xc[S] = xb.v[0][S] + (uint32_t)(s0 * SB);
      xn[S] = xb.v[0][S] + (uint32_t)(s1 * SB);
    }
  }
  kstep<F, MI, RAGGED, 0, LOAD, NB>(acc, ka, kb, r, ring, xc, L);
  kstep<F, MI, RAGGED, 1, LOAD, NB>(acc, kb, ka, r, ring, xc, L);
  kstep<F, MI, RAGGED, 2, LOAD, NB>(acc, ka, kb, r, ring, xc, L);
  // k-step 3: MFMAs from kb; the operands of stage h + 1's k-step 0 go to ka
  mfma_group<MI, 0, NB>(acc, kb);
  __builtin_amdgcn_sched_barrier(0);
  const uint8_t* next = ring + s1 * SB;
  if constexpr (MORE) {
    // outstanding direct loads, oldest first: stage h + 1, then stage h + 2 if issued
    if constexpr (LOAD) wait_vmcnt<LPS>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads of stage h are done
    workgroup_barrier();
    read_w<MI, NB>(r, next, scales_per_row_chunk(F), unit_s(F), wave, lane);
  }
  __builtin_amdgcn_sched_barrier(0);
  BDec d[2];
  // MFMA groups 1 .. MI - 1 of k-step 3 carry the preparation of stage h + 1's k-step 0 (the shares of
  // groups 0 .. MI - 2 here, the last group's share after the loop body)
#define FP4_LAST(G)                                                                \
  if constexpr ((G) < MI) {                                                        \
    mfma_one<MI, G, 0>(acc, kb);                                                   \
    if constexpr (MORE) {                                                          \
      ka.a[(G) - 1] = a_frag(ring, xn[0], (G) - 1);                               \
      b_slot<F, MI, 0, NB * ((G) - 1)>(d, ka.b, r);                                \
    }                                                                              \
    __builtin_amdgcn_sched_barrier(0);                                             \
    if constexpr (NB == 2) {                                                       \
      mfma_one<MI, G, 1>(acc, kb);                                                 \
      if constexpr (MORE) b_slot<F, MI, 0, 2 * ((G) - 1) + 1>(d, ka.b, r);         \
      __builtin_amdgcn_sched_barrier(0);                                           \
    }                                                                              \
  }
  FP4_LAST(1) FP4_LAST(2) FP4_LAST(3) FP4_LAST(4) FP4_LAST(5) FP4_LAST(6) FP4_LAST(7)
#undef FP4_LAST
  if constexpr (MORE) {
    ka.a[MI - 1] = a_frag(ring, xn[0], MI - 1);
    b_slot<F, MI, 0, NB * (MI - 1)>(d, ka.b, r);
    if constexpr (NB == 2) b_slot<F, MI, 0, 2 * (MI - 1) + 1>(d, ka.b, r);
  }
}

// One tile of y: rows m0 .. m0 + 32 MI - 1, columns n0 .. n0 + 128 NB - 1 (see the kernel). SETS = 2: two
// sets of 4 waves (two waves per SIMD), each with a ring of its own, share the tile's K range: set s takes
// stages hb + s, hb + s + 2, ... (he - hb even), and set 1's sums are added to set 0's through LDS at the end
// (in that order, so the result does not depend on timing).
template <int F, int MI, bool RAGGED, int NB = 2, int SETS = 1>
__device__ __forceinline__ void gemm_tile(uint8_t* ring, const uint8_t* __restrict__ qp, const uint8_t* __restrict__ sp,
                                          const uint16_t* __restrict__ x, float* __restrict__ y, int M, int N, int K,
                                          int nchunk, int m0, int n0, float gscale, int hb, int he, bool add_out,
                                          bool keep = false) {
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave: keeps descriptors scalar
  const int wave = SETS == 1 ? wid : (wid & (GM_WAVES - 1));
  const int set = SETS == 1 ? 0 : (wid >> 2);
  const int wrow0 = n0 + 32 * NB * wave;       // this wave's 32 NB weight rows (2 NB tiles of 16)
  const int ntiles = (N + TILE_N - 1) / TILE_N;

  GemmSrc src;
  const int mrows = min(M - m0, 32 * MI);
  src.x = make_rsrc(x + (int64_t)m0 * K, (uint32_t)mrows * (uint32_t)K * 2u);
  const int tiles_here = max(0, min(ntiles - wrow0 / TILE_N, 2 * NB));
  src.q = make_rsrc(qp + (int64_t)(wrow0 / TILE_N) * nchunk * UNIT_Q, (uint32_t)(tiles_here * nchunk * UNIT_Q));
  src.s = make_rsrc(sp + (int64_t)(wrow0 / TILE_N) * nchunk * unit_s(F), (uint32_t)(tiles_here * nchunk * unit_s(F)));
  LoadOffs lo;
  load_offsets<F, MI>(lo, K, nchunk, wave, lane);

  f32x16 acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  // Pipeline over stages of 64 positions (4 k-steps each), 3 ring slots. Stage h + 1 is in LDS or on its
  // way while stage h is computed, and stage h + 2's loads are issued during k-steps 0-2 of stage h, into
  // the slot stage h - 1 freed at the last barrier. K-steps 0-2 prepare the next k-step's operands
  // between their MFMAs. In k-step 3 the wave waits for its share of stage h + 1, meets the other waves
  // at a barrier (every wave's share of stage h + 1 is then in LDS, and every wave is done reading stage
  // h), reads stage h + 1's packed weights and prepares its k-step 0 -- still between MFMAs.
  // Stages hb .. he - 1 (all of K, or one part of a split K); hb is a multiple of the ring period, so
  // stage h sits in ring slot h % 3 as when hb = 0.
  constexpr int LPS = gm_loads_per_stage(F, MI, NB);
  constexpr int SB = gm_stage_bytes(MI, NB);
  // With two sets, this set's stages are counted from 0 (stage v of the set is stage h0 + 2 v of K) and it
  // uses its own ring; with one, v is the stage of K itself (h0 = 0).
  const int h0 = SETS == 1 ? 0 : hb + set;
  const int vb = SETS == 1 ? hb : 0, ve = SETS == 1 ? he : (he - hb) / 2;
  if constexpr (SETS == 2) ring += set * gm_lds(MI, NB);
  issue_stage<F, MI, RAGGED, NB>(src, lo, ring + (vb % GM_RING) * SB, h0 + SETS * vb, K, nchunk, wave, lane);
  if (vb + 1 < ve)
    issue_stage<F, MI, RAGGED, NB>(src, lo, ring + ((vb + 1) % GM_RING) * SB, h0 + SETS * (vb + 1), K, nchunk, wave,
                                   lane);
  if (vb + 1 < ve) wait_vmcnt<LPS>();
  else wait_vmcnt<0>();
  workgroup_barrier();
  WRegs r;
  KOps<MI> ka, kb;
  read_w<MI, NB>(r, ring, scales_per_row_chunk(F), unit_s(F), wave, lane);
  XBase xb;
  x_bases<MI, NB>(xb, lane);
  prep_all0<F, MI, NB>(ka, r, ring, xb.v[0][0]);

  // Every stage but the last two issues the loads of stage h + 2; the last has no next stage. The stage
  // body is compiled for each case, so the loop has no per-group branches.
  int h = vb;
  // three stages per iteration (the ring period), so that every ring offset is a constant
  for (; h + 4 < ve; h += 3) {
    stage_body<F, MI, RAGGED, true, true, 0, NB, SETS>(acc, ka, kb, r, src, lo, ring, xb, h, K, nchunk, wave, lane, h0);
    stage_body<F, MI, RAGGED, true, true, 1, NB, SETS>(acc, ka, kb, r, src, lo, ring, xb, h + 1, K, nchunk, wave, lane,
                                                       h0);
    stage_body<F, MI, RAGGED, true, true, 2, NB, SETS>(acc, ka, kb, r, src, lo, ring, xb, h + 2, K, nchunk, wave, lane,
                                                       h0);
  }
  for (; h + 2 < ve; ++h)
    stage_body<F, MI, RAGGED, true, true, -1, NB, SETS>(acc, ka, kb, r, src, lo, ring, xb, h, K, nchunk, wave, lane, h0);
  if (h + 1 < ve)
    stage_body<F, MI, RAGGED, false, true, -1, NB, SETS>(acc, ka, kb, r, src, lo, ring, xb, h++, K, nchunk, wave, lane,
                                                         h0);
  stage_body<F, MI, RAGGED, false, false, -1, NB, SETS>(acc, ka, kb, r, src, lo, ring, xb, h, K, nchunk, wave, lane, h0);

  if constexpr (SETS == 2) {
    // set 1 hands its sums to set 0 through LDS (the rings are free once every wave has passed the barrier
    // after its last LDS read): [wave][i][j][e][lane] floats, 256 contiguous bytes per (i, j, e)
    ring -= set * gm_lds(MI, NB);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    workgroup_barrier();
    float* red = reinterpret_cast<float*>(ring) + (size_t)wave * (MI * NB * 16 * 64) + lane;
    if (set == 1) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) red[((i * NB + j) * 16 + e) * 64] = acc[i][j][e];
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    workgroup_barrier();
    if (set == 1) return;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] += red[((i * NB + j) * 16 + e) * 64];
  }

  // epilogue: acc[i][j][e] = C[32 i + 8 (e / 4) + 4 (lane / 32) + e % 4][32 j + lane % 32]; y is written
  // once and not read back here, so the stores are nontemporal (about 1% faster than plain ones). A
  // part of a split K adds its g-scaled sum into the zeroed y instead (FP32 atomics in L2): with two parts
  // every element is fl(0 + a + b) in either order, so the result does not depend on which part is first.
  if (add_out) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = m0 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          const int col = wrow0 + 32 * j + (lane & 31);
          if (row < M && col < N) unsafeAtomicAdd(y + (int64_t)row * N + col, acc[i][j][e] * gscale);
        }
    return;
  }
  if (keep) {  // a partial sum of a K part, read back soon by the combining kernel: plain stores
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = m0 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          const int col = wrow0 + 32 * j + (lane & 31);
          if (row < M && col < N) y[(int64_t)row * N + col] = acc[i][j][e] * gscale;
        }
    return;
  }
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int col = wrow0 + 32 * j + (lane & 31);
        if (row < M && col < N) __builtin_nontemporal_store(acc[i][j][e] * gscale, y + (int64_t)row * N + col);
      }
}

// Tiles. The first nbig workgroups take 256-row tiles, the rest (if any) 192-row tiles; the host picks the
// split so that a grid of between one and two rounds of 256-row tiles becomes two rounds whose second is
// made of the shorter tiles (the slowest CU then does 1.75 tiles of work, not 2).
//  * 192-row tiles: rows 0 .. 1535 (8 bands) of column tiles 0 .. ns - 1; workgroup nbig + i takes band
//    i % 8 and column tile i / 8.
//  * 256-row tiles: first column tiles ns .. tiles_n - 1 over all tiles_m bands (band = i % tiles_m), then
//    rows 1536 .. M - 1 (tiles_m - 6 bands) of column tiles 0 .. ns - 1.
// With ns = 0 every tile is 256 rows: workgroup i takes band i % tiles_m and column tile i / tiles_m.
// Block b runs on XCD b % 8, so with 8 bands the workgroups of one XCD share an x band in its L2.
template <int F, bool RAGGED>
__global__ __launch_bounds__(GM_THREADS) void gemm_kernel(const uint8_t* __restrict__ qp,
                                                          const uint8_t* __restrict__ sp,
                                                          const uint16_t* __restrict__ x, float* __restrict__ y,
                                                          int M, int N, int K, int nchunk, int tiles_m, int ns,
                                                          int nbig, float gscale) {
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
  const int b = (int)blockIdx.x;
  if (b < nbig) {
    const int tiles_n = (N + GM_BN - 1) / GM_BN;
    const int nwide = tiles_m * (tiles_n - ns);
    int m0, n0;
    if (b < nwide) {
      m0 = (b % tiles_m) * GM_BM;
      n0 = (ns + b / tiles_m) * GM_BN;
    } else {
      const int i = b - nwide, bands = tiles_m - GM_SHORT_BANDS * GM_SHORT_ROWS / GM_BM;
      m0 = GM_SHORT_BANDS * GM_SHORT_ROWS + (i % bands) * GM_BM;
      n0 = (i / bands) * GM_BN;
    }
    gemm_tile<F, 8, RAGGED>(ring, qp, sp, x, y, M, N, K, nchunk, m0, n0, gscale, 0, 2 * nchunk, false);
  } else {
    const int i = b - nbig;
    gemm_tile<F, 6, RAGGED>(ring, qp, sp, x, y, M, N, K, nchunk, (i % GM_SHORT_BANDS) * GM_SHORT_ROWS,
                            (i / GM_SHORT_BANDS) * GM_BN, gscale, 0, 2 * nchunk, false);
  }
}

// Small grids (a kernel of its own, so that the prefill kernel above keeps its code): tiles of 32 MI rows
// (MI = 4 or 6 when M fits one such band, else 8) and 128 NB columns (NB = 1: each wave owns 32 weight
// rows, so twice the tiles of the 256-column tiling), tile t taking band t % tiles_m and column tile
// t / tiles_m. ksplit > 0: workgroup t < ntiles takes stages 0 .. ksplit - 1 of tile t, workgroup ntiles + t
// the rest, and both add into the zeroed y. ksplit = -P (two-set tiles only): workgroup p ntiles + t takes
// chunks [p C / P, (p + 1) C / P) of tile t (C chunks) and writes its g-scaled sum to plane p of the
// workspace ws (P planes of M x N floats); gemm_combine_kernel then adds the planes into y.
template <int F, bool RAGGED, int MI, int NB, int SETS = 1>
__global__ __launch_bounds__(GM_THREADS * SETS) void gemm_small_kernel(const uint8_t* __restrict__ qp,
                                                                const uint8_t* __restrict__ sp,
                                                                const uint16_t* __restrict__ x,
                                                                float* __restrict__ y, int M, int N, int K,
                                                                int nchunk, int tiles_m, int ntiles, float gscale,
                                                                int ksplit, float* __restrict__ ws) {
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
  int t = (int)blockIdx.x;
  int hb = 0, he = 2 * nchunk;
  float* out = y;
  if (ksplit > 0) {
    const bool second = t >= ntiles;
    if (second) t -= ntiles;
    hb = second ? ksplit : 0;
    he = second ? he : ksplit;
  } else if (SETS == 2 && ksplit < 0) {
    const int parts = -ksplit, p = t / ntiles;
    t -= p * ntiles;
    hb = 2 * (int)((int64_t)p * nchunk / parts);
    he = 2 * (int)((int64_t)(p + 1) * nchunk / parts);
    out = ws + (int64_t)p * M * N;
  }
  gemm_tile<F, MI, RAGGED, NB, SETS>(ring, qp, sp, x, out, M, N, K, nchunk, (t % tiles_m) * 32 * MI,
                                     (t / tiles_m) * 128 * NB, gscale, hb, he, ksplit > 0, SETS == 2 && ksplit < 0);
}

// y = 0 before the parts of a split K add into it (a kernel, not a memset, so that the call can be
// captured in a graph). One 16-byte store per thread where y is 16-byte aligned and the element count a
// multiple of 4 (n4 = n / 4 stores); otherwise (n4 = 0) one element per thread.
__global__ void gemm_zero_kernel(float* __restrict__ y, int64_t n, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (n4 > 0) {
    if (i < n4) reinterpret_cast<f32x4*>(y)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  } else if (i < n) {
    y[i] = 0.f;
  }
}

// y = plane 0 + plane 1 + ... + plane P - 1 of the workspace (n floats each), added in that order, so the
// result does not depend on which K part finished first. Four elements per thread (16-byte loads and store)
// where n is a multiple of 4 and ws and y are 16-byte aligned (n4 = n / 4), else one.
__global__ void gemm_combine_kernel(const float* __restrict__ ws, float* __restrict__ y, int64_t n, int64_t n4,
                                    int parts) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (n4 > 0) {
    if (i >= n4) return;
    f32x4 a = reinterpret_cast<const f32x4*>(ws)[i];
    for (int p = 1; p < parts; ++p) {
      const f32x4 b = reinterpret_cast<const f32x4*>(ws + (int64_t)p * n)[i];
      a[0] += b[0];
      a[1] += b[1];
      a[2] += b[2];
      a[3] += b[3];
    }
    __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(y) + i);
  } else if (i < n) {
    float a = ws[i];
    for (int p = 1; p < parts; ++p) a += ws[(int64_t)p * n + i];
    y[i] = a;
  }
}

template <int F, bool RAGGED, int MI, int NB, int SETS = 1>
static int launch_gemm_small(hipStream_t st, int grid, const uint8_t* q, const uint8_t* s, const uint16_t* x, float* y,
                             int M, int N, int K, int nchunk, int tiles_m, int ntiles, float g, int ksplit,
                             float* ws = nullptr) {
  static Fp4LdsLimit lds_limit;
  constexpr int lds = SETS * gm_lds(MI, NB);
  lds_limit.ensure(reinterpret_cast<const void*>(&gemm_small_kernel<F, RAGGED, MI, NB, SETS>), lds);
  return fp4_launch(gemm_small_kernel<F, RAGGED, MI, NB, SETS>, dim3(grid), dim3(GM_THREADS * SETS), lds, st, q, s, x,
                    y, M, N, K, nchunk, tiles_m, ntiles, g, ksplit, ws);
}

template <int F, bool RAGGED, int NB>
static int launch_gemm_small_mi(int band_rows, bool sets2, hipStream_t st, int grid, const uint8_t* q, const uint8_t* s,
                                const uint16_t* x, float* y, int M, int N, int K, int nchunk, int tiles_m, int ntiles,
                                float g, int ksplit, float* ws = nullptr) {
  if constexpr (NB == 1) {
    if (sets2 && band_rows == 128)
      return launch_gemm_small<F, RAGGED, 4, 1, 2>(st, grid, q, s, x, y, M, N, K, nchunk, tiles_m, ntiles, g, ksplit,
                                                   ws);
  }
  if (band_rows == 128)
    return launch_gemm_small<F, RAGGED, 4, NB>(st, grid, q, s, x, y, M, N, K, nchunk, tiles_m, ntiles, g, ksplit);
  if (band_rows) return launch_gemm_small<F, RAGGED, 6, NB>(st, grid, q, s, x, y, M, N, K, nchunk, 1, ntiles, g, ksplit);
  return launch_gemm_small<F, RAGGED, 8, NB>(st, grid, q, s, x, y, M, N, K, nchunk, tiles_m, ntiles, g, ksplit);
}

// Launch shape of a GEMM call (the rules below), shared by the launch and by the workspace query.
struct GemmPlan {
  int nchunk, tiles_m, ns, nbig, band_rows, rows_m, ksplit, parts;
  int64_t Ut;
  bool narrow, sets2;
};

static GemmPlan plan_gemm(int M, int N, int K, size_t ws_bytes) {
  GemmPlan P{};
  const int nchunk = (K + CHUNK_K - 1) / CHUNK_K;
  const int tiles_m = (M + GM_BM - 1) / GM_BM;
  const int tiles_n = (N + GM_BN - 1) / GM_BN;
  // Between one and two rounds of 256-row tiles: 8 s columns' worth of rows 0 .. 1535 go to s = 8 ns
  // 192-row tiles (3/4 of the work each), chosen so that the grid is two rounds (s = 4 (2 cus - U), at
  // most every column tile), the second made of short tiles.
  const int cus = fp4_device_cus();
  const Fp4Tuning& tu = fp4_tuning();
  const int64_t U = (int64_t)tiles_m * tiles_n;
  int ns = 0;
  if (M % GM_BM == 0 && M >= GM_SHORT_BANDS * GM_SHORT_ROWS && U > cus && U < 2 * cus) {
    ns = (int)(4 * (2 * cus - U) / GM_SHORT_BANDS);
    if (ns > tiles_n) ns = tiles_n;
  }
  if (tu.gemm_short == 0) ns = 0;  // tuning override: 256-row tiles only
  const int nbig = (int)(U - (int64_t)(GM_SHORT_BANDS * GM_SHORT_ROWS / GM_BM) * ns);
  // Grids of 256-column tiles that fill at most half the CUs take 128-column tiles (twice the tiles, each
  // wave owning 32 weight rows) where twice the grid still fits one round.
  const bool narrow = ns == 0 && 2 * U <= cus && tu.gemm_narrow != 0;  // tuning override: 0 = 256 columns
  const int NBsel = narrow ? 1 : 2;
  const int64_t tiles_nb = (N + 128 * NBsel - 1) / (128 * NBsel);
  // Tile height: one band of 128 or 192 rows when M fits it. Above that, 128-column grids take 128-row tiles
  // over ceil(M / 128) bands where that grid still fits one workgroup per CU (twice the workgroups of 256-row
  // tiles): 14336 x 4096 at M = 256 38.1 us against 47.8 us, 9728 x 2560 at M = 256 22.9 against 32.4 us,
  // both with one wave set. With more bands than that, 256-row tiles win (M = 512: 62.3 against 66.9 us).
  // With two wave sets per 128-row tile (below), 128-row bands also beat one 192-row band for 128 < M <= 192
  // (14336 x 4096 at M = 160 30.4 against 36.8 us, 9728 x 2560 at M = 192 18.9 against 26.0 us).
  const bool sets_ok = tu.gemm_sets != 1;
  int band_rows = (M <= 128) ? 128 : (M <= GM_SHORT_ROWS && !(sets_ok && narrow)) ? GM_SHORT_ROWS : 0;
  int bands = 1;
  if (band_rows == 0 && narrow && (int64_t)((M + 127) / 128) * tiles_nb <= cus) {
    band_rows = 128;
    bands = (M + 127) / 128;
  }
  if (band_rows == 0 && M <= GM_SHORT_ROWS) band_rows = GM_SHORT_ROWS;
  if (tu.gemm_band_rows == 0) {  // tuning override: 256-row tiles
    band_rows = 0;
    bands = tiles_m;
  }
  const int rows_m = band_rows ? bands : tiles_m;  // bands of the grid
  const int64_t Ut = (int64_t)rows_m * tiles_nb;
  // Grids of at most half the CUs (in tiles of the shape chosen above) split K in two (at a multiple of
  // the 3-stage ring period, each part at least 6 stages) so that twice the workgroups run; y is zeroed
  // first and both parts add into it with FP32 atomics, whose cost grows with M N: on 14336 x 4096, M = 256
  // (3.7 M outputs) the split took 51.0 us against 47.9 us whole, at M = 160 (2.3 M) 36.3 against 40.3 us.
  // At M = 512 (112 tiles of 256 columns) the split had been 91 us against 79 us whole.
  int ksplit = 0;
  const int H = 2 * nchunk;
  if (ns == 0 && 2 * Ut <= cus && H >= 12 && (int64_t)M * N <= GM_SPLIT_MAX_OUT) ksplit = 3 * (H / 6);
  if (tu.gemm_split == 0) ksplit = 0;  // tuning override: whole K per workgroup
  // 128-row bands of 128-column tiles (a 63 KiB ring) run two sets of 4 waves per workgroup, each over every
  // other stage with a ring of its own (two waves per SIMD; each weight still decoded once per workgroup).
  // The sets need an even number of stages in each part of K. With them a stage costs about 0.7 us per
  // workgroup and the split's zero fill and atomics about 7.5 us per million outputs, so K splits only while
  // that is below a quarter of the stages' time (M N <= 23000 H): 14336 x 4096 at M = 128 26.4 us whole
  // against 28.9 us split, at M = 65 21.3 us split against 25.5 us whole.
  // (256-row tiles with two sets, each with a 2-slot ring to fit 148 KiB, were slower: 14336 x 4096 at
  // M = 512 64.1 against 58.7 us.)
  const bool sets2 = narrow && band_rows == 128 && sets_ok;  // tuning override FP4_GEMM_SETS=1: one set
  if (sets2 && ksplit) ksplit = (int64_t)M * N <= 23000LL * H ? 2 * (H / 4) : 0;
  if (sets2 && tu.gemm_split == 1 && ns == 0 && 2 * Ut <= cus && H >= 12) ksplit = 2 * (H / 4);  // tuning override
  // With a workspace, two-set grids that leave CUs idle split K into P parts instead (one round of Ut P
  // workgroups, at least one chunk each, at most 16 parts): each part writes its g-scaled sum to a plane of
  // the workspace and a second kernel adds the planes in a fixed order. P minimises a time model (ns):
  // 700 per stage of a set, H / (2 P) stages, plus 2000 for the second launch, the planes' traffic
  // ((P + 1) M N 4 bytes at 4 bytes per 1/1000 ns) and 400 per part. It replaces the two-part atomic split.
  // Measured (NVFP4, P swept): 2560 x 9728 at M = 128 20.3-20.9 us for P = 8-12 against 42.3 us before,
  // at M = 65 17.3-17.5 us for P = 8-10 against 29.4; 4096 x 4096 at M = 128 18.9 us at P = 4, 20.7 at 8.
  int parts = 1;
  if (sets2 && ns == 0 && tu.gemm_split != 0 && ws_bytes > 0) {
    int pmax = (int)(cus / Ut);
    if (pmax > nchunk) pmax = nchunk;
    if (pmax > 16) pmax = 16;
    double best = 700.0 * H / 2;
    for (int p = 2; p <= pmax; ++p) {
      if ((double)p * M * N * 4 > (double)ws_bytes) break;
      const double t = 700.0 * H / (2.0 * p) + 2000.0 + (p + 1) * (double)M * N / 1000.0 + 400.0 * p;
      if (t < best) {
        best = t;
        parts = p;
      }
    }
    const int tp = tu.gemm_parts;  // tuning override: that many parts where they fit
    if (tp >= 1 && tp <= pmax && (double)tp * M * N * 4 <= (double)ws_bytes) parts = tp;
    if (parts > 1) ksplit = 0;
  }
  P.nchunk = nchunk;
  P.tiles_m = tiles_m;
  P.ns = ns;
  P.nbig = nbig;
  P.band_rows = band_rows;
  P.rows_m = rows_m;
  P.ksplit = ksplit;
  P.parts = parts;
  P.Ut = Ut;
  P.narrow = narrow;
  P.sets2 = sets2;
  return P;
}

// Workspace bytes the K parts of a call would use (0: the call takes none).
static size_t gemm_workspace_bytes(int M, int N, int K) {
  const GemmPlan P = plan_gemm(M, N, K, ~(size_t)0);
  return P.parts > 1 ? (size_t)P.parts * (size_t)M * (size_t)N * sizeof(float) : 0;
}

template <int F, bool RAGGED>
static int launch_gemm_t(hipStream_t st, const uint8_t* q, const uint8_t* s, const uint16_t* x, float* y, int M,
                          int N, int K, float g, float* ws, size_t ws_bytes) {
  const GemmPlan P = plan_gemm(M, N, K, ws ? ws_bytes : 0);
  const int nchunk = P.nchunk, ksplit = P.ksplit;
  if (ksplit == 0 && P.parts == 1 && P.band_rows == 0 && !P.narrow) {
    static Fp4LdsLimit lds_limit;
    lds_limit.ensure(reinterpret_cast<const void*>(&gemm_kernel<F, RAGGED>), GM_LDS);
    return fp4_launch(gemm_kernel<F, RAGGED>, dim3(P.nbig + GM_SHORT_BANDS * P.ns), dim3(GM_THREADS), GM_LDS, st, q,
                      s, x, y, M, N, K, nchunk, P.tiles_m, P.ns, P.nbig, g);
  }
  if (ksplit) {
    const int64_t total = (int64_t)M * N;
    const int64_t n4 = (total % 4 == 0 && fp4_aligned(y, 16)) ? total / 4 : 0;
    const int64_t threads = n4 > 0 ? n4 : total;
    const int rc = fp4_launch(gemm_zero_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, y, total, n4);
    if (rc) return rc;
  }
  if (P.parts > 1) {  // K parts into the workspace planes, then their sum into y
    const int grid = P.parts * (int)P.Ut;
    int rc = launch_gemm_small_mi<F, RAGGED, 1>(P.band_rows, true, st, grid, q, s, x, y, M, N, K, nchunk, P.rows_m,
                                                (int)P.Ut, g, -P.parts, ws);
    if (rc) return rc;
    const int64_t total = (int64_t)M * N;
    const int64_t n4 = (total % 4 == 0 && fp4_aligned(y, 16) && fp4_aligned(ws, 16)) ? total / 4 : 0;
    const int64_t threads = n4 > 0 ? n4 : total;
    return fp4_launch(gemm_combine_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, ws, y, total, n4,
                      P.parts);
  }
  const int grid = ksplit ? 2 * (int)P.Ut : (int)P.Ut;
  if (P.narrow)
    return launch_gemm_small_mi<F, RAGGED, 1>(P.band_rows, P.sets2, st, grid, q, s, x, y, M, N, K, nchunk, P.rows_m,
                                              (int)P.Ut, g, ksplit);
  return launch_gemm_small_mi<F, RAGGED, 2>(P.band_rows, false, st, grid, q, s, x, y, M, N, K, nchunk, P.rows_m,
                                            (int)P.Ut, g, ksplit);
}

template <int F>
static int launch_gemm(hipStream_t st, const uint8_t* q, const uint8_t* s, const uint16_t* x, float* y, int M, int N,
                       int K, float g, float* ws, size_t ws_bytes) {
  if (K % CHUNK_K == 0) return launch_gemm_t<F, false>(st, q, s, x, y, M, N, K, g, ws, ws_bytes);
  return launch_gemm_t<F, true>(st, q, s, x, y, M, N, K, g, ws, ws_bytes);
}

}  // namespace fp4

using namespace fp4;

// Arguments of a GEMM call: 0 or a negative status.
static int check_gemm(int fmt, int64_t M, int64_t N, int64_t K) {
  if (!fp4_valid_format(fmt)) return -1;
  if (M < 0) return -2;
  if (fmt == Q4_0) return -4;  // its FP16-scaled weights are not exact in bf16; Q4_0 runs through the GEMV
  int rc = fp4_check_nk(fmt, N, K);
  if (rc) return rc;
  if (M > (1LL << 30)) return -4;
  if (K > (1LL << 22)) return -4;  // tile offsets are 32-bit buffer offsets: 256 rows x K x 2 bytes < 2^31
  const int64_t grid = ((M + GM_BM - 1) / GM_BM) * ((N + GM_BN - 1) / GM_BN);
  if (grid > 0x7fffffffLL) return -4;
  return 0;
}

extern "C" int64_t w4a16_gemm_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K) {
  const int rc = check_gemm(fmt, M, N, K);
  if (rc) return rc;
  if (M == 0) return 0;
  return (int64_t)gemm_workspace_bytes((int)M, (int)N, (int)K);
}

extern "C" int w4a16_gemm_ws(int fmt, int64_t M, int64_t N, int64_t K, const void* q, const void* s,
                             float global_scale, const void* x_bf16, float* y, void* workspace, size_t workspace_bytes,
                             void* stream) {
  const int rc = check_gemm(fmt, M, N, K);
  if (rc) return rc;
  if (M == 0) return 0;
  if (!q || !s || !x_bf16 || !y) return -1;
  if (!fp4_aligned(q, 16) || !fp4_aligned(s, 16) || !fp4_aligned(x_bf16, 16) || !fp4_aligned(y, 4)) return -3;
  if (workspace && !fp4_aligned(workspace, 16)) return -3;
  hipStream_t st = (hipStream_t)stream;
  const uint8_t* qq = (const uint8_t*)q;
  const uint8_t* ss = (const uint8_t*)s;
  const uint16_t* xx = (const uint16_t*)x_bf16;
  float* ws = (float*)workspace;
  const size_t wb = workspace ? workspace_bytes : 0;
  switch (fmt) {
    case NVFP4: return launch_gemm<NVFP4>(st, qq, ss, xx, y, (int)M, (int)N, (int)K, global_scale, ws, wb);
    case DUAL:  return launch_gemm<DUAL>(st, qq, ss, xx, y, (int)M, (int)N, (int)K, global_scale, ws, wb);
    default:    return launch_gemm<FAST>(st, qq, ss, xx, y, (int)M, (int)N, (int)K, global_scale, ws, wb);
  }
}

extern "C" int w4a16_gemm(int fmt, int64_t M, int64_t N, int64_t K, const void* q, const void* s,
                          float global_scale, const void* x_bf16, float* y, void* stream) {
  return w4a16_gemm_ws(fmt, M, N, K, q, s, global_scale, x_bf16, y, nullptr, 0, stream);
}

// 48 <= M <= 64 on matrices of at least 20 M weights: with K parts in a workspace the GEMM beats the mid-M
// kernel (NVFP4, one run each: 2560 x 9728 at M = 48 16.2 against 17.6 us, M = 64 17.2 against 22.2; 9728 x
// 2560 at M = 64 16.4 against 19.6; 14336 x 4096 at M = 64 21.6 against 35.6), while on 4096 x 4096 the mid-M
// kernel stays faster (M = 64 12.1 against 14.9 us).
static bool matmul_gemm_band(int fmt, int64_t M, int64_t N, int64_t K) {
  return M >= 48 && M <= 64 && fmt != Q4_0 && N * K >= (20LL << 20);
}

extern "C" int64_t w4a16_matmul_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K) {
  if (M > 64 || matmul_gemm_band(fmt, M, N, K)) return w4a16_gemm_workspace_bytes(fmt, M, N, K);
  if (!fp4_valid_format(fmt)) return -1;
  if (M < 0) return -2;
  return fp4_check_nk(fmt, N, K);
}

extern "C" int w4a16_matmul_ws(int fmt, int64_t M, int64_t N, int64_t K, const void* q, const void* s,
                               float global_scale, const void* x_bf16, float* y, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (M >= 0 && M <= 16) return w4a16_gemv(fmt, M, N, K, q, s, global_scale, x_bf16, y, stream);
  if (M <= 64) {
    if (workspace && matmul_gemm_band(fmt, M, N, K) && check_gemm(fmt, M, N, K) == 0) {
      const size_t need = gemm_workspace_bytes((int)M, (int)N, (int)K);
      if (need > 0 && workspace_bytes >= need)
        return w4a16_gemm_ws(fmt, M, N, K, q, s, global_scale, x_bf16, y, workspace, workspace_bytes, stream);
    }
    return w4a16_midm(fmt, M, N, K, q, s, global_scale, x_bf16, y, stream);
  }
  return w4a16_gemm_ws(fmt, M, N, K, q, s, global_scale, x_bf16, y, workspace, workspace_bytes, stream);
}

extern "C" int w4a16_matmul(int fmt, int64_t M, int64_t N, int64_t K, const void* q, const void* s,
                            float global_scale, const void* x_bf16, float* y, void* stream) {
  return w4a16_matmul_ws(fmt, M, N, K, q, s, global_scale, x_bf16, y, nullptr, 0, stream);
}

// The GEMM without a caller workspace and without allocating: its K-part planes live in `scratch`, a
// file-scope device array of FP4_GEMM_SCRATCH_BYTES on every GPU the library runs on. The K parts of one
// call fill at most one round of 128 x 128 tiles (parts x tiles <= CUs), so their planes hold at most
// 16384 floats per CU: 16 MiB covers every split on a 256-CU device. In host code `scratch` names a host
// stand-in, not device memory: the device address comes from hipGetSymbolAddress, taken once per device
// (on the first call there, with that device current) and kept per device.
static __device__ __align__(256) float scratch[FP4_GEMM_SCRATCH_BYTES / sizeof(float)];
static std::atomic<float*> scratch_addr[64];

static int scratch_of_current_device(float** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -6;
  float* p = scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return -6;
    p = static_cast<float*>(a);
    scratch_addr[dev].store(p, std::memory_order_release);  // a racing first call stores the same address
  }
  *out = p;
  return 0;
}

extern "C" int w4a16_gemm_noalloc(int fmt, int64_t M, int64_t N, int64_t K, const void* q, const void* s,
                                  float global_scale, const void* x_bf16, float* y, void* stream) {
  const int rc = check_gemm(fmt, M, N, K);
  if (rc) return rc;
  if (M == 0) return 0;
  if (!q || !s || !x_bf16 || !y) return -1;
  if (!fp4_aligned(q, 16) || !fp4_aligned(s, 16) || !fp4_aligned(x_bf16, 16) || !fp4_aligned(y, 4)) return -3;
  if (gemm_workspace_bytes((int)M, (int)N, (int)K) > FP4_GEMM_SCRATCH_BYTES) return -4;
  float* ws = nullptr;
  const int rs = scratch_of_current_device(&ws);
  if (rs) return rs;
  return w4a16_gemm_ws(fmt, M, N, K, q, s, global_scale, x_bf16, y, ws, FP4_GEMM_SCRATCH_BYTES, stream);
}
