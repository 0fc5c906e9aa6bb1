// Shared device definitions: kernel layout geometry and the nibble/scale decoders.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4 {

enum Fmt { NVFP4 = 1, DUAL = 2, FAST = 3, Q4_0 = 4 };

// Kernel layout. A "unit" is one 16-row tile x one 128-wide K chunk.
//   nibble plane: [tile][chunk][g = 0..3][n = 0..15][16 bytes]  -> 1024 B per unit
//   scale plane:  [tile][chunk][n = 0..15][spr bytes]           -> 16*spr B per unit
//                 (spr = 8 scale bytes for NVFP4 / Dual, 4 for FAST, 4 little-endian FP16 for Q4_0)
// Lane l = 16 g + n of a wave reads 16 bytes at offset 16 l of a unit: row n, the 32
// positions k' = 32 g + i (i = 0..31) of the chunk, permuted so that one MFMA covers
// exactly one scale group per row:
//   16-weight groups (NVFP4, Dual), MFMA 16x16x16: i = 4 j + t  <->  k = 16 j + 4 g + t
//   32-weight blocks (FAST, Q4_0),  MFMA 16x16x32: i = 8 j + t  <->  k = 32 j + 8 g + t
// Within the 16 bytes the nibble of position i sits where the decoder wants it:
//   NVFP4 (hardware E2M1 pair convert): byte i/2, low nibble when i is even;
//   Codebook10 (byte LUT + FP8 pair convert) and Q4_0 (byte permute into bf16 mantissas):
//   dword i/8, byte (i%8)%4, high nibble iff i%8 >= 4.
constexpr int TILE_N = 16;
constexpr int CHUNK_K = 128;
constexpr int UNIT_Q = 1024;

// 32-weight blocks (FAST, Q4_0) or 16-weight groups (NVFP4, Dual) share one scale
__host__ __device__ constexpr bool block32(int f) { return f == FAST || f == Q4_0; }
__host__ __device__ constexpr int group_size(int f) { return block32(f) ? 32 : 16; }
__host__ __device__ constexpr int scales_per_row_chunk(int f) { return CHUNK_K / group_size(f); }
// scale bytes per row and chunk: one byte per scale, two for Q4_0's FP16 scales
__host__ __device__ constexpr int scale_bytes_row_chunk(int f) { return scales_per_row_chunk(f) * (f == Q4_0 ? 2 : 1); }
__host__ __device__ constexpr int unit_s(int f) { return TILE_N * scale_bytes_row_chunk(f); }

// chunk-relative k of lane-group g, lane position i
__host__ __device__ constexpr int kmap(int f, int g, int i) {
  return block32(f) ? 32 * (i >> 3) + 8 * g + (i & 7) : 16 * (i >> 2) + 4 * g + (i & 3);
}
// (byte, high-nibble?) of lane position i inside the 16-byte lane piece
__host__ __device__ constexpr int nib_byte(int f, int i) { return f == NVFP4 ? (i >> 1) : 4 * (i >> 3) + (i & 3); }
__host__ __device__ constexpr int nib_high(int f, int i) { return f == NVFP4 ? (i & 1) : ((i & 7) >> 2); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Codebook10 magnitudes 0,1,2,3,4,6,8,10 as OCP E4M3 bytes, as two v_perm source words.
// v_perm_b32(S0, S1, sel): selector bytes 0..3 pick S1's bytes, 4..7 pick S0's bytes.
constexpr uint32_t CB10_E4M3_LO = 0x44403800u;  // codes 0..3 -> 0x00, 0x38, 0x40, 0x44
constexpr uint32_t CB10_E4M3_HI = 0x52504C48u;  // codes 4..7 -> 0x48, 0x4C, 0x50, 0x52

// Eight Codebook10 nibbles (one dword) -> two words of four E4M3 bytes each:
//   lo: the low nibbles of bytes 0..3, hi: the high nibbles of bytes 0..3.
__device__ __forceinline__ void cb10_to_e4m3(uint32_t w, uint32_t& lo, uint32_t& hi) {
  uint32_t mlo = w & 0x07070707u;
  uint32_t mhi = (w >> 4) & 0x07070707u;
  lo = __builtin_amdgcn_perm(CB10_E4M3_HI, CB10_E4M3_LO, mlo) | ((w << 4) & 0x80808080u);
  hi = __builtin_amdgcn_perm(CB10_E4M3_HI, CB10_E4M3_LO, mhi) | (w & 0x80808080u);
}

// Two E4M3 bytes (low or high half-word) -> exact bf16 pair. Scale 1.0 (the conversion
// uses only the scale's exponent, so a unit scale leaves the values untouched).
template <bool HIGH>
__device__ __forceinline__ bf16x2 e4m3x2_to_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HIGH);
}

// Byte SEL of w (two E2M1 nibbles, low nibble first) -> exact bf16 pair.
template <int SEL>
__device__ __forceinline__ bf16x2 e2m1x2_to_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
}

// E4M3 byte SEL of w -> f32 (OCP E4M3: bias 7, S.1111.111 NaN).
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8(w, SEL);
}

// Raw buffer descriptor (stride 0) over `bytes` bytes from `base`; loads past the end return zeros.
// The descriptor must live in scalar registers; its inputs are wave-uniform, so read them from lane 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ bf16x4 cat(bf16x2 a, bf16x2 b) { return bf16x4{a[0], a[1], b[0], b[1]}; }
__device__ __forceinline__ bf16x8 cat(bf16x2 a, bf16x2 b, bf16x2 c, bf16x2 d) {
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// bf16 pair of two f32 values that bf16 holds exactly (level * scale has at most 8 significant bits, so
// the low 16 bits of its f32 encoding are zero): the high halves of both, joined with one byte permute.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, a), 0x07060302u);
}

__device__ __forceinline__ bf16x8 to_bf16x8(const f32x2& a, const f32x2& b, const f32x2& c, const f32x2& e, float sc) {
  u32x4 v = {pack_bf16x2(a[0] * sc, a[1] * sc), pack_bf16x2(b[0] * sc, b[1] * sc), pack_bf16x2(c[0] * sc, c[1] * sc),
             pack_bf16x2(e[0] * sc, e[1] * sc)};
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// Four Codebook10 nibbles (the low nibbles of the four bytes of w when HIGH is false, the high nibbles
// otherwise) -> four E4M3 bytes.
template <bool HIGH>
__device__ __forceinline__ uint32_t cb10_quad(uint32_t w) {
  if constexpr (HIGH) {
    return __builtin_amdgcn_perm(CB10_E4M3_HI, CB10_E4M3_LO, (w >> 4) & 0x07070707u) | (w & 0x80808080u);
  } else {
    return __builtin_amdgcn_perm(CB10_E4M3_HI, CB10_E4M3_LO, w & 0x07070707u) | ((w << 4) & 0x80808080u);
  }
}

// Same with a separate scale for the first and the second four values.
__device__ __forceinline__ bf16x8 to_bf16x8(const f32x2& a, const f32x2& b, const f32x2& c, const f32x2& e, float s0,
                                           float s1) {
  u32x4 v = {pack_bf16x2(a[0] * s0, a[1] * s0), pack_bf16x2(b[0] * s0, b[1] * s0), pack_bf16x2(c[0] * s1, c[1] * s1),
             pack_bf16x2(e[0] * s1, e[1] * s1)};
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

}  // namespace fp4
