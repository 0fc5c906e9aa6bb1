/*
 * fp4w4a16 — block-scaled 4-bit weight x bf16 activation products (W4A16) on gfx950.
 *
 * The operation (EdgeRock-4B-NVFP4 model card, description; Nanbeige4.2-3B-NVFP4A16
 * card, header and serving notes; ROCmFP4 design page, sections 01-03 and the
 * format comparison table):
 *
 *     y[m][n] = sum_k x[m][k] * W[n][k]        (y fp32, x bf16, W never materialised)
 *
 *   NVFP4:          W[n][k] = e2m1(q) * e4m3(s[n][k/16]) * g
 *   ROCmFP4 Dual:   W[n][k] = codebook10(q) * ue4m3(s_half) * g   (one scale per 16)
 *   ROCmFP4 FAST:   W[n][k] = codebook10(q) * ue4m3(s_block) * g  (one scale per 32)
 *   Q4_0:           W[n][k] = (q - 8) * fp16(d_block) * g            (one scale per 32)
 *
 * with e2m1 in {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6}, codebook10 in {0, +-1, +-2,
 * +-3, +-4, +-6, +-8, +-10}, g the per-matrix FP32 global scale (1.0 for ROCmFP4 and Q4_0).
 * The library computes level*scale exactly, applies g last (fl32(fl32(level*scale)*g)),
 * and accumulates in FP32.
 *
 * Conventions for every entry point:
 *  - All pointers except `q_bytes`/`s_bytes` of fp4_layout_bytes are DEVICE pointers
 *    owned by the caller; the library keeps none of them after returning and allocates
 *    no memory.
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *    asynchronously; a return of FP4_OK means the launch was accepted.
 *  - Arguments are validated before anything is enqueued; a negative status is returned
 *    and nothing runs. A launch the HIP runtime rejects returns FP4_ERR_HIP (each launch's
 *    own return code is checked; errors left by earlier, unrelated HIP calls are neither
 *    reported nor cleared). No entry point prints or aborts.
 *  - State kept between calls: per-device caches of facts about the device (compute-unit
 *    count, occupancy of each kernel variant, whether a kernel's dynamic-LDS limit has been
 *    raised), filled on first use and never changed afterwards; the tuning overrides read
 *    once from the environment at the first call (FP4_GEMV_WAVES, FP4_GEMV_U, FP4_GEMV_ONE,
 *    FP4_GEMV_RING, FP4_MIDM_WAVES, FP4_GEMM_SHORT, FP4_GEMM_SPLIT, FP4_GEMM_BAND_ROWS,
 *    FP4_GEMM_NARROW, FP4_QUANT_EXHAUSTIVE, FP4_ONE_BATCH, FP4_GEMM_SETS, FP4_GEMM_PARTS;
 *    none set by default); one 4-byte device word per GPU, a static device variable, that
 *    fp4_pack_layout uses when asked to validate (serialised by a per-device host lock); and
 *    the static device array of w4a16_gemm_noalloc (FP4_GEMM_SCRATCH_BYTES per GPU), which
 *    only that entry point touches. Apart from those two, concurrent calls on different
 *    streams share no mutable state.
 *  - Shapes: W is N x K (N outputs, K inputs); x is M x K bf16 row-major; y is M x N
 *    fp32 row-major. K must be a multiple of 16 (NVFP4) or 32 (ROCmFP4). M = 0 is a
 *    no-op. x and the planes must be 16-byte aligned; y must be 4-byte aligned and must
 *    not overlap x or the planes.
 */
#ifndef FP4W4A16_H
#define FP4W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4W4A16_ABI_VERSION 3

/* Weight formats. */
enum {
  FP4_NVFP4 = 1,        /* E2M1 nibbles, E4M3 scale per 16, FP32 global scale      */
  FP4_ROCMFP4_DUAL = 2, /* Codebook10 nibbles, two UE4M3 half-block scales, 18 B/32 */
  FP4_ROCMFP4_FAST = 3, /* Codebook10 nibbles, one UE4M3 block scale, 17 B/32        */
  FP4_Q4_0 = 4          /* stock Q4_0: levels q - 8, one FP16 block scale, 18 B/32   */
};

/* Status codes. */
enum {
  FP4_OK = 0,
  FP4_ERR_ARG = -1,          /* null pointer or unknown format                  */
  FP4_ERR_SHAPE = -2,        /* bad M, N or K                                    */
  FP4_ERR_ALIGN = -3,        /* a pointer is not aligned as required             */
  FP4_ERR_UNSUPPORTED = -4,  /* shape outside what the entry point handles       */
  FP4_ERR_INVALID_SCALE = -5,/* a scale code is NaN or infinite (fp4_pack_layout
                                with validation on)                               */
  FP4_ERR_HIP = -6           /* the HIP runtime rejected a launch or a copy      */
};

/* Version of this interface (FP4W4A16_ABI_VERSION). */
int fp4_abi_version(void);

/* Text for a status code; static storage, never NULL. */
const char* fp4_status_string(int status);

/*
 * Bytes of the two device planes ("kernel layout") that fp4_pack_layout writes for an
 * N x K matrix of format `fmt`: the nibble plane and the scale plane. Rows are padded to
 * a multiple of 16 and K to a multiple of 128; padding holds zero codes and zero scales.
 * For N a multiple of 16 and K of 128 the two planes hold exactly the canonical bytes:
 * 18, 17 and 18 bytes per 32 weights for Dual, FAST and Q4_0 (ROCmFP4 design page, format
 * comparison table: block size and density) and K/2 + K/16 bytes per row for NVFP4 (one
 * nibble per weight and one scale byte per 16: EdgeRock-4B-NVFP4 card, description).
 * q_bytes and s_bytes are HOST pointers. Errors: FP4_ERR_ARG (unknown format, null
 * pointer), FP4_ERR_SHAPE / FP4_ERR_UNSUPPORTED (N or K out of range).
 */
int fp4_layout_bytes(int fmt, int64_t N, int64_t K, size_t* q_bytes, size_t* s_bytes);

/*
 * Repack canonical packed weights into the kernel layout (load time, once per matrix; the
 * pages handle their packed data and scales once, when a checkpoint is loaded: EdgeRock-4B-
 * NVFP4 card, "Load on a CUDA GPU"; block contents from the ROCmFP4 design page, format
 * comparison table, and section 02 on the two half-block scales).
 * Canonical input (device memory):
 *   NVFP4:    src_q = wq uint8[N][K/2], byte j holds element 2j (bits 0-3) and 2j+1
 *             (bits 4-7); src_s = ws uint8[N][K/16] E4M3 scales.
 *   ROCmFP4:  src_q = blocks uint8[N][K/32][B] with B = 18 (Dual: s_lo, s_hi, qs[16]) or
 *             17 (FAST: s, qs[16]); qs[j] holds weight j (bits 0-3) and j+16 (bits 4-7);
 *             src_s must be NULL. UE4M3 bit 7 is ignored.
 *   Q4_0:     src_q = blocks uint8[N][K/32][18] = [FP16 d, little-endian; qs[16]] with the
 *             same qs order; src_s must be NULL.
 * Output: dst_q / dst_s of the sizes fp4_layout_bytes reports (16-byte aligned). The
 * layout's internal order is private to this library and may change with the ABI version.
 * validate != 0: before anything is written, every scale code is checked on the device
 * (both formats define their scales as finite numbers: EdgeRock-4B-NVFP4 card, description,
 * which gives E4M3 scale bytes; ROCmFP4 design page, section 02, where the scale bytes are
 * E4M3 without a sign, and section 03, whose search ranges over finite scale values only).
 * An E4M3 / UE4M3 code whose low 7 bits are all ones (NaN), or a Q4_0 FP16
 * scale with an all-ones exponent (infinity or NaN), makes the call return
 * FP4_ERR_INVALID_SCALE and leave dst_q / dst_s untouched. Validation waits for `stream`
 * (the call returns only after the check has run) and is meant for load time.
 * validate == 0: no check and no wait; such codes then decode to NaN (or infinity) as the
 * format defines them.
 * Errors: FP4_ERR_ARG (unknown format; null src_q, dst_q or dst_s; src_s null for NVFP4 or
 * non-null otherwise), FP4_ERR_SHAPE / FP4_ERR_UNSUPPORTED (N, K), FP4_ERR_ALIGN (dst not
 * 16-byte aligned), FP4_ERR_INVALID_SCALE, FP4_ERR_HIP.
 */
int fp4_pack_layout(int fmt, int64_t N, int64_t K, const void* src_q, const void* src_s,
                    void* dst_q, void* dst_s, int validate, void* stream);

/*
 * Decode-shaped product, 1 <= M <= 16 (one token, or one token plus n-gram draft tokens:
 * Nanbeige4.2-3B-NVFP4A16 card, serving notes; its speed is set by the weight bytes read:
 * same card, speed notes, and Gemma-4-E4B-it-ROCmFP4-GGUF card, bandwidth sanity check).
 * y = x * W^T with W as defined at the top (EdgeRock-4B-NVFP4 card, description; ROCmFP4
 * design page, sections 01 and 02). Streams each nibble and scale byte
 * once, decodes to exact bf16 levels, contracts against x on the matrix cores, applies
 * the group scales to the FP32 partial sums, reduces the K split inside the workgroup and
 * multiplies by g. Up to M = 8 a wave issues all of its loads at once where that fits the chip
 * in one round of workgroups. Otherwise, from M = 5 on, it runs the mid-M kernel of
 * w4a16_midm (each wave's chunks in a chain); for Q4_0 only its one-block form (M <= 16), in
 * which the scales are folded per group as in the GEMV.
 * q/s are fp4_pack_layout output (device); x is M x K bf16 bit patterns and y M x N fp32,
 * both row-major on the device. Deterministic (no atomics). Errors: FP4_ERR_ARG,
 * FP4_ERR_SHAPE (M < 0, N or K), FP4_ERR_UNSUPPORTED (M > 16, K > 2^24), FP4_ERR_ALIGN,
 * FP4_ERR_HIP.
 */
int w4a16_gemv(int fmt, int64_t M, int64_t N, int64_t K, const void* q, const void* s,
               float global_scale, const void* x_bf16, float* y, void* stream);

/*
 * Several decode-shaped products in one launch (the per-launch cost dominates decode matrices
 * of a few MB, whose weight bytes set the decode speed: Nanbeige4.2-3B-NVFP4A16 card, speed notes). Each item is one
 * matrix with its own planes, x, y, N, K and global scale; all share fmt and M (1 <= M <= 16).
 * Typical use: the q|k|v or gate|up projections of one token, which read the same x, or any
 * list of independent products. Each y equals what w4a16_gemv would produce to within the
 * product tolerance (the K split may differ, so the summation order can). `items` is a HOST
 * array, read before the call returns; at most FP4_GEMV_MAX_ITEMS items. Each item is checked
 * as w4a16_gemv checks its arguments; the first failing item's status is returned and nothing
 * runs. M = 0 or count = 0 is a no-op. y buffers must not overlap each other or any input.
 */
#define FP4_GEMV_MAX_ITEMS 32
typedef struct fp4_gemv_item {
  const void* q;        /* fp4_pack_layout nibble plane (device) */
  const void* s;        /* fp4_pack_layout scale plane (device) */
  const void* x_bf16;   /* x[M][K], bf16 bit patterns (device) */
  float* y;             /* y[M][N], fp32 (device) */
  int64_t N;
  int64_t K;
  float global_scale;
} fp4_gemv_item;

int w4a16_gemv_batched(int fmt, int64_t M, int count, const fp4_gemv_item* items, void* stream);

/*
 * Prefill-shaped product, any M >= 1, intended for M >= 64 (a prompt of many tokens against
 * the same packed weights; W as defined at the top: EdgeRock-4B-NVFP4 card, description;
 * ROCmFP4 design page, sections 01 and 02, and the technical-boundaries note that the levels
 * are exact integers, which lets level*scale be exact in bf16): stages x tiles and packed
 * weight tiles in LDS, decodes each weight once per workgroup into exact bf16 level*scale
 * MFMA operands, contracts with bf16 MFMA in FP32 and multiplies by g in the epilogue. For
 * M <= 128 (192) the tiles may be 128 (192) rows high; 128-row tiles of small grids run two
 * wave sets over alternate stages of K whose two sums are added in a fixed order.
 * When y has few tiles (at most half the device's compute units) and K spans at least 6
 * chunks of 128, K may be split in two: the call enqueues a kernel that zeroes y, then the
 * product, whose two halves add their g-scaled sums into y with FP32 atomics. Two addends
 * onto zero give the same sum in either order, so the result is still bit-reproducible; it
 * differs from the whole-K sum only by rounding. Both kernels run on `stream`.
 * Q4_0 gives FP4_ERR_UNSUPPORTED (its level*scale is not exact in bf16). Other errors:
 * FP4_ERR_ARG, FP4_ERR_SHAPE, FP4_ERR_UNSUPPORTED (K > 2^22), FP4_ERR_ALIGN, FP4_ERR_HIP.
 * Equivalent to w4a16_gemm_ws with no workspace.
 */
int w4a16_gemm(int fmt, int64_t M, int64_t N, int64_t K, const void* q, const void* s,
               float global_scale, const void* x_bf16, float* y, void* stream);

/*
 * w4a16_gemm with a caller workspace (device memory, 16-byte aligned, owned by the caller and
 * used only while the call's kernels run on `stream`; it needs no initial contents). Grids that
 * leave compute units idle (the small-N prefill shapes, e.g. a 2560 x 9728 projection at
 * M = 65..256: the band between the decode and prefill shapes of the Nanbeige4.2-3B-NVFP4A16
 * card's serving notes) split K into P parts (2 <= P <= 16) instead of the two-part atomic split:
 * each part writes its g-scaled sum to plane p of the workspace (P planes of M x N floats) and a
 * second kernel on `stream` adds the planes into y in the order p = 0 .. P - 1, so the result is
 * bit-reproducible and differs from the whole-K sum only by rounding. workspace_bytes at least
 * w4a16_gemm_workspace_bytes() gives the split the launch rules choose; a smaller workspace gives
 * the largest split that fits (possibly none, as w4a16_gemm); NULL means none. Errors as
 * w4a16_gemm, and FP4_ERR_ALIGN for a misaligned workspace. Calls that share a workspace must be
 * ordered on one stream.
 */
int w4a16_gemm_ws(int fmt, int64_t M, int64_t N, int64_t K, const void* q, const void* s,
                  float global_scale, const void* x_bf16, float* y, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * Workspace bytes that w4a16_gemm_ws would use for this shape on the current device (0 when it
 * would not split K into parts), or a negative status for arguments w4a16_gemm would reject
 * (pointers aside). At most 64 KiB per compute unit of the device.
 */
int64_t w4a16_gemm_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K);

/*
 * For callers that cannot allocate device memory (code under graph capture, serving loops,
 * harnesses that forbid allocation): w4a16_gemm_ws with the workspace taken from a static device
 * array of FP4_GEMM_SCRATCH_BYTES on each GPU (its address is looked up once per device, on the
 * first call there; no allocation, ever). Outputs equal w4a16_gemm_ws's with a workspace of
 * w4a16_gemm_workspace_bytes(). Shapes whose split would need more than FP4_GEMM_SCRATCH_BYTES
 * (only possible on devices with more than 256 compute units) give FP4_ERR_UNSUPPORTED and
 * nothing runs. Every call on a GPU uses that GPU's one array: calls that overlap in time on one
 * GPU (on different streams, or from different threads without ordering) race on it and may give
 * wrong results; order them on one stream. Other errors as w4a16_gemm.
 */
#define FP4_GEMM_SCRATCH_BYTES (16u << 20)
int w4a16_gemm_noalloc(int fmt, int64_t M, int64_t N, int64_t K, const void* q, const void* s,
                       float global_scale, const void* x_bf16, float* y, void* stream);

/*
 * Mid-sized M, 1 <= M <= 64 (the band between the decode and prefill shapes,
 * e.g. speculative-decoding verification of many drafts or small batches, Nanbeige4.2-3B-NVFP4A16
 * card, serving notes): the GEMV's layout and in-workgroup K split, with each weight decoded once
 * into exact bf16 level*scale and reused by up to four 16-row blocks of x on the matrix cores.
 * Deterministic. Arguments and errors as w4a16_gemv; M > 64 gives FP4_ERR_UNSUPPORTED.
 */
int w4a16_midm(int fmt, int64_t M, int64_t N, int64_t K, const void* q, const void* s,
               float global_scale, const void* x_bf16, float* y, void* stream);

/* Dispatch on M: M <= 16 -> w4a16_gemv, 17 <= M <= 64 -> w4a16_midm, otherwise
 * w4a16_gemm. w4a16_matmul_ws: the same with w4a16_gemm_ws above 64, and for 48 <= M <= 64 on
 * matrices of at least 20 M weights (N K >= 20 * 2^20, not Q4_0) the GEMM with K parts too when the
 * workspace holds them (there it is faster than the mid-M kernel); w4a16_matmul_workspace_bytes gives
 * the workspace it can use (0: none), or a negative status for arguments it would reject. */
int w4a16_matmul(int fmt, int64_t M, int64_t N, int64_t K, const void* q, const void* s,
                 float global_scale, const void* x_bf16, float* y, void* stream);
int w4a16_matmul_ws(int fmt, int64_t M, int64_t N, int64_t K, const void* q, const void* s,
                    float global_scale, const void* x_bf16, float* y, void* workspace,
                    size_t workspace_bytes, void* stream);
int64_t w4a16_matmul_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K);

/*
 * Dequantize the kernel layout to FP32 W[N][K] (the pages' dequant-at-load, EdgeRock card,
 * section on loading on a CUDA GPU): W = fl32(fl32(level*scale)*g), bit-exact. For checking and tools.
 */
int fp4_dequant_f32(int fmt, int64_t N, int64_t K, const void* q, const void* s,
                    float global_scale, float* w, void* stream);

/*
 * Device packer, NVFP4 data-free round-to-nearest (Nanbeige4.2-3B-NVFP4A16 card,
 * "Creation"; EdgeRock card, description): w fp32[N][K] -> canonical wq uint8[N][K/2],
 * ws uint8[N][K/16] and g (one float written to DEVICE memory g_out):
 *   g = fl32(amax / 2688); s = E4M3 RNE of blockmax / (6 g) (FP64 divide, saturating at
 *   448); each weight takes the nearest E2M1 magnitude of |w| / (e4m3(s) g), ties to the
 *   even code; the sign bit is set only for nonzero magnitudes. amax = 0 gives g = 1 and
 *   all-zero codes. g_out doubles as the amax accumulator while the call runs.
 */
int fp4_quantize_nvfp4(int64_t N, int64_t K, const float* w, void* wq, void* ws, float* g_out,
                       void* stream);

/*
 * Device packer, ROCmFP4 exhaustive finite-UE4M3 MSE scale search (ROCmFP4 design page,
 * section 03): for each 16-weight half (Dual) or 32-weight block (FAST), every UE4M3 code
 * 0x00..0x7E is scored by E = sum v_i (|w_i| - L_i s)^2 in FP64 in index order, L_i the
 * nearest Codebook10 level (ties to the even level, clipping at 10); the smallest E wins,
 * ties broken by distance from the start code (E4M3 RNE of max|w|/10) then by the lower
 * code. importance (v) may be NULL (all ones). Output: canonical blocks uint8[N][K/32][B].
 * The candidates are visited outward from the start code with safe pruning (same section: work that cannot
 * change the selected scale may be skipped): a direction is dropped once a lower bound of E made of E's own
 * terms (weights that must clip to level 10 below the scale, or round to 0 above it) reaches the best error,
 * so the result is the exhaustive winner. Groups with a non-finite weight or a negative or NaN importance
 * score every candidate.
 */
int fp4_quantize_rocmfp4(int fmt, int64_t N, int64_t K, const float* w, const float* importance,
                         void* blocks, void* stream);

/*
 * Device packer, stock Q4_0 with the signed abs-max scale (ROCmFP4 design page, format
 * comparison table, stock Q4_0 column): w fp32[N][K] -> canonical Q4_0 blocks
 * uint8[N][K/32][18] = [FP16 d (little-endian), qs[16]], qs[j] = code j | code j+16 << 4.
 * Per block m = the first weight of largest magnitude, d = m / -8, stored as FP16 (RNE);
 * code = floor(w / d + 8.5) clipped to 0..15 in FP64 with the unrounded d; d = 0 gives
 * code 8. Q4_0 runs through w4a16_gemv, w4a16_gemv_batched and fp4_dequant_f32; the
 * matrix-core paths (w4a16_midm, w4a16_gemm) return FP4_ERR_UNSUPPORTED for it because its
 * level*scale products are not exact in bf16.
 */
int fp4_quantize_q4_0(int64_t N, int64_t K, const float* w, void* blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4W4A16_H */
