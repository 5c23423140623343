/*
 * w4a4.h — C ABI of the W4A4 quantized linear layer for AMD MI355X (gfx950).
 *
 * The layer (SERQ page, "Resumen técnico" §1-3; OffQ page, "Metodología"
 * steps 2-3):
 *   1. rotate every row of the activation X [M, K] by a block Hadamard
 *      transform over contiguous groups of b channels (Sylvester matrix,
 *      whose first row is all ones, scaled by 1/sqrt(b));
 *   2. quantize each rotated row ("on the fly", per token) to symmetric int4
 *      with an absmax scale;
 *   3. multiply the int4 codes by pre-quantized int4 weight codes W [N, K]
 *      (int32 accumulation) and dequantize with the activation and weight
 *      scales;
 *   4. optionally add the single low-rank compensation term X . A . B of
 *      rank r on the unrotated X.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers:   every data pointer is a DEVICE pointer owned by the caller,
 *             row-major and contiguous, aligned to 16 bytes.  The library
 *             never allocates, frees or keeps a pointer past the call.
 * Streams:    `stream` is a hipStream_t passed as void* (NULL = the null
 *             stream).  Every call only enqueues work on that stream and
 *             returns; buffers must stay alive until the stream has run it.
 *             A non-OK status means nothing was enqueued.
 * Sizes:      M (tokens) and N (output channels) may be 0 (nothing is
 *             enqueued); K must be a positive multiple of 64 and at most
 *             16384 (the rotation kernel holds a row of K values in one
 *             workgroup); the in-GEMM residual form also needs
 *             8 K + (r rounded up to 128) < 2^17.
 * dtypes:     W4A4_F32 = float32, W4A4_F16 = IEEE binary16.
 * Packing:    int4 codes are two's-complement nibbles, element 2j in the low
 *             nibble of byte j: a [R, K] code matrix is stored as uint8
 *             [R, K/2].  Produced codes are always in [-7, 7]; the GEMM also
 *             multiplies -8 correctly.
 * Rotation:   had_block b is 0 or 1 for "no rotation" (input already
 *             rotated), otherwise a power of two, at most 4096, dividing K.
 * Quantizer:  s = max|x~| / 7 in float32 (IEEE division); each code is
 *             clamp(rint(x~ / s), -7, 7) with the quotient rounded to float32
 *             and ties to even; a zero scale gives all-zero codes.
 * Errors:     no exceptions cross the ABI; every call returns a w4a4_status.
 * Threads:    the library is stateless apart from a per-device cache of the
 *             device check and, for w4a4_qlinear_forward_noalloc only, one
 *             fixed scratch array per device that every such call on that
 *             device shares (its calls must not overlap); all other calls are
 *             reentrant.
 */
#ifndef W4A4_H
#define W4A4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A4_ABI_VERSION 1

typedef enum {
  W4A4_OK = 0,
  W4A4_ERR_INVALID_ARG = 1, /* null required pointer, bad dtype, negative size,
                               K not positive, rank > 0 without A or B */
  W4A4_ERR_UNSUPPORTED = 2, /* shape outside the kernels' domain (K not a
                               multiple of 64 or above 16384, bad Hadamard
                               block or weight group, rank above 256 or an
                               fp16 rank not a multiple of 8), or a device
                               that is not gfx950 / no device */
  W4A4_ERR_MISALIGNED = 3,  /* a pointer not aligned to 16 bytes */
  W4A4_ERR_WORKSPACE = 4,   /* workspace smaller than required */
  W4A4_ERR_HIP = 5          /* a HIP runtime error while launching */
} w4a4_status;

typedef enum { W4A4_F32 = 0, W4A4_F16 = 1 } w4a4_dtype;

/* Layouts of activation codes.
 *   W4A4_CODES_PACKED: [M, K/2] uint8, two nibbles per byte (see Packing).
 *   W4A4_CODES_I8:     [M, K] int8, one code per byte; inside every group of
 *                      8 consecutive channels the bytes hold channels
 *                      0,2,4,6,1,3,5,7 of the group.  This is the K order in
 *                      which the GEMM widens packed weight nibbles, so these
 *                      codes feed the int8 matrix instructions unchanged; it
 *                      is the layout w4a4_qlinear_forward uses internally. */
typedef enum {
  W4A4_CODES_PACKED = 0,
  W4A4_CODES_I8 = 1,
  W4A4_CODES_I8_TILED = 2,
  W4A4_CODES_PACKED_TILED = 3,
  W4A4_CODES_PACKED_TILED_OB = 4,
  W4A4_CODES_F6_TILED = 5
} w4a4_codes_layout;

/* Tiled layouts (K a multiple of 128).  Rows are taken in blocks of 16 and K
 * in iterations of 128 codes; every (row block, iteration) tile is stored
 * contiguously, row blocks outermost, in the order in which one 64-lane
 * wave reads it: lane l = 16 g + r holds row r of the block.  Rows past the
 * end of the last block are padding with unspecified bytes.
 *   W4A4_CODES_I8_TILED (activations, [ceil(M/16)*16, K] bytes): tile
 *     (b, t) is 2048 bytes at (b*(K/128) + t)*2048; inside it, for
 *     h in {0,1}, g in {0..3}, r in {0..15}, the 16 bytes at
 *     ((4h + g)*16 + r)*16 are the W4A4_CODES_I8 bytes of codes
 *     [128t + 32g + 16h, +16) of row 16b + r.
 *   W4A4_WEIGHTS_TILED (weights, [ceil(N/16)*16, K/2] bytes): tile (b, t) is
 *     1024 bytes at (b*(K/128) + t)*1024; inside it, for g in {0..3},
 *     r in {0..15}, the 16 bytes at (16g + r)*16 are the packed bytes
 *     [64t + 16g, +16) of row 16b + r.
 *   W4A4_CODES_PACKED_TILED (activations, [ceil(M/16)*16, K/2] bytes): the
 *     packed codes of W4A4_CODES_PACKED in the W4A4_WEIGHTS_TILED layout.
 * With these layouts every 1 KB of a GEMM operand tile is one contiguous
 * copy, which the strided row-major layouts cannot offer; tiled weights are
 * used with tiled activation codes (int8 or packed). */
typedef enum {
  W4A4_WEIGHTS_ROWMAJOR = 0,
  W4A4_WEIGHTS_TILED = 1,
  W4A4_WEIGHTS_TILED_OB = 2,
  W4A4_WEIGHTS_TILED_F6 = 3
} w4a4_weight_layout;

/* Offset-binary tiled layouts: the same 16-row x 128-code tiles, with one
 * code of every byte stored as q + 8 (0..15) so that the GEMM isolates each
 * nibble with a single AND per dword instead of a shift and an AND.  Each
 * buffer is followed by one int32 per padded row.
 *   W4A4_CODES_PACKED_TILED_OB (activations, [ceil(M/16)*16, K/2] bytes and
 *     then ceil(M/16)*16 int32): every W4A4_CODES_PACKED_TILED byte XOR 0x08
 *     (low nibble: the even channel's code + 8; high nibble: the odd
 *     channel's signed code); int32 m after the tiles: the sum of row m's
 *     codes at odd channels.
 *   W4A4_WEIGHTS_TILED_OB (weights, [ceil(N/16)*16, K/2] bytes and then
 *     ceil(N/16)*16 int32): every W4A4_WEIGHTS_TILED byte with its nibbles
 *     swapped and the new low nibble XOR 8 (low nibble: the odd channel's
 *     code + 8; high nibble: the even channel's signed code); int32 n after
 *     the tiles: the sum of row n's codes at even channels.
 * In a product of the two, the GEMM pairs each high (signed, times 16) nibble
 * with the other operand's low (offset) nibble of the same channel, so its
 * int32 accumulator holds 16 sum_k qx qw + 128 (row sum + column sum), which
 * the epilogue corrects exactly.  Offset-binary weights are produced from
 * tiled ones by w4a4_weights_tiled_to_ob and serve per-channel weight scales
 * (w_group 0) of the int4 layer and GEMM. */

/* FP6 tiled layouts: the same 4-bit codes (SERQ page, "Resumen técnico"
 * §1-2), each stored as the FP6 E2M3 number of equal value (OCP
 * microscaling formats: sign bit 5, exponent bits 4:3 with bias 1, mantissa
 * bits 2:0; every integer in [-7, 7] is exact, e.g. 3 = 0b010100 and
 * -7 = 0b111110; code 0 may be stored as either zero, 0b000000 or
 * 0b100000).  They are the operand format of the gfx950 FP6 matrix
 * instruction, whose float32 sums of these products are exact integers, so
 * the GEMM takes them with no conversion; they cost 6 bits per code instead
 * of 4.  Rows in blocks of 16, K (a multiple of 128) in steps of 128; tile
 * (b, t) is 1536 bytes at (b*(K/128) + t)*1536.  Lane l = 16g + r of a tile
 * holds codes [128t + 32g, +32) of row 16b + r as 192 bits, field p (bits
 * [6p, 6p+6)) being code 128t + 32g + p/2 + 16*(p%2); the tile's bytes
 * [16l, 16l + 16) are the lane's bits [0, 128), its bytes
 * [1024 + 8l, 1024 + 8l + 8) the bits [128, 192).
 *   W4A4_CODES_F6_TILED (activations, [ceil(M/16)*16, 3K/4] bytes)
 *   W4A4_WEIGHTS_TILED_F6 (weights, [ceil(N/16)*16, 3K/4] bytes)
 * Produced by w4a4_quantize_act_int4 and w4a4_quantize_weight_int4, used
 * together by w4a4_qgemm_w4a4 and by the int4 layer (per-channel or grouped
 * weight scales, any M, not the 8-bit activations of W4A8). */

/* ABI version of the loaded library (W4A4_ABI_VERSION when built). */
int w4a4_abi_version(void);

/* Static, human-readable name of a status code. */
const char* w4a4_status_string(int status);

/* HIP error code (hipError_t) behind the last W4A4_ERR_HIP returned on this
 * thread, 0 if none. */
int w4a4_last_hip_error(void);

/*
 * Block Hadamard rotation (OffQ page, "Metodología" steps 2-3).
 *   x      [M, K] in dtype x_dtype.
 *   x_rot  [M, K] float32 output: every block of b contiguous channels of a
 *          row becomes block . H_b / sqrt(b), computed in float32 by a fast
 *          Walsh-Hadamard transform.
 *   had_block must be a power of two >= 2.
 */
int w4a4_hadamard_rotate(const void* x, int x_dtype, float* x_rot,
                         int64_t M, int64_t K, int64_t had_block, void* stream);

/*
 * Per-token symmetric int4 quantization of activations, with the block
 * Hadamard rotation fused in front (SERQ page, "Resumen técnico" §1-2: 4-bit
 * activations quantized on the fly; OffQ page, steps 2-3).
 *   x        [M, K] in dtype x_dtype.
 *   had_block 0/1: x is already rotated (codes then follow the quantizer rule
 *            exactly); otherwise the rotation above is applied first.
 *   xq       output codes in codes_layout ([M, K/2] packed, [M, K] int8 or
 *            tiled int8).
 *   x_scale  [M] float32 output, one scale per row.
 *   The input must be finite: a row holding a NaN or an infinity gets
 *   unspecified codes and scale.
 */
int w4a4_quantize_act_int4(const void* x, int x_dtype, int64_t M, int64_t K,
                           int64_t had_block, uint8_t* xq, int codes_layout,
                           float* x_scale, void* stream);
/*   With W4A4_CODES_PACKED_TILED_OB, xq holds ceil(M/16)*16 * (K/2 + 4)
 *   bytes: the offset-binary tiles and then the per-row sums of the codes at
 *   odd channels (rows M and above: unspecified). */

/*
 * 8-bit form of the activation quantizer, for W4A8 layers: the layers a
 * phase-aware mixed-precision policy keeps at 8-bit activations while the
 * weights stay 4-bit (DynamicPTQ page, "Metodología" §2).  Same rotation and
 * rule as w4a4_quantize_act_int4 with the code range [-127, 127]:
 * s = max|x~| / 127, q = clamp(rint(x~ / s), -127, 127).
 *   codes_layout must be W4A4_CODES_I8 or W4A4_CODES_I8_TILED (one signed
 *   code per byte, in those layouts' byte order); other layouts return
 *   W4A4_ERR_INVALID_ARG.  The codes feed w4a4_qgemm_w4a4 unchanged.
 */
int w4a4_quantize_act_int8(const void* x, int x_dtype, int64_t M, int64_t K,
                           int64_t had_block, uint8_t* xq, int codes_layout,
                           float* x_scale, void* stream);

/*
 * Offline weight preparation: rotation (had_block > 1) and symmetric
 * round-to-nearest int4 (DynamicPTQ page, "Resultados": RTN weights).
 *   w        [N, K] in dtype w_dtype.
 *   w_group  0: one scale per output channel; otherwise a power of two >= 64
 *            dividing K: one scale per group of w_group channels along K.
 *   wq       packed codes in w_layout: [N, K/2] row-major, or tiled.
 *   w_scale  [N] or [N, K/w_group] output in dtype scale_dtype.  The scale is
 *            rounded to scale_dtype first and the codes are taken against the
 *            stored value.
 */
int w4a4_quantize_weight_int4(const void* w, int w_dtype, int64_t N, int64_t K,
                              int64_t had_block, int64_t w_group, uint8_t* wq,
                              int w_layout, void* w_scale, int scale_dtype,
                              void* stream);

/*
 * First half of the low-rank term (SERQ page, "Resumen técnico" §2 item 2):
 *   t [M, rank] float32 = x [M, K] . A, with A passed transposed as
 *   At [rank, K] (row j of At is column j of A, so that it is contiguous
 *   along K like the weights).  x and At in dtype x_dtype; float32
 *   accumulation (fp16 matrix instructions for fp16 inputs).  1 <= rank <= 256.
 */
int w4a4_lowrank_project(const void* x, int x_dtype, const void* At, int64_t M,
                         int64_t K, int64_t rank, float* t, void* stream);

/*
 * int4 x int4 GEMM with the dequantizing epilogue (SERQ page, "Resumen
 * técnico" §3: 4-bit matrix multiplication in the linear layer).
 *   xq in codes_layout, x_scale [M] float32: activation codes and scales.
 *   The int8 layouts also carry the 8-bit codes of w4a4_quantize_act_int8
 *   (|code| <= 127; exact for K <= 16384).
 *   wq in w_layout, w_scale [N] (w_group 0) or [N, K/w_group] in
 *   w_scale_dtype.  Tiled weights need tiled codes (W4A4_CODES_I8_TILED or
 *   W4A4_CODES_PACKED_TILED) and a w_group of 0 or a multiple of 128.
 *   w_group 0 or a multiple of 64 dividing K.
 *   y   [M, N] float32 output, or NULL:
 *         y[m,n] = x_scale[m] * sum_j w_scale[n,j] * acc_j[m,n]
 *       where acc_j is the exact int32 product over K-group j.
 *   acc [M, N] int32 output, or NULL: the exact full-K integer product
 *       sum_k qx[m,k] * qw[n,k].
 *   At least one of y and acc must be non-NULL.
 */
int w4a4_qgemm_w4a4(const uint8_t* xq, int codes_layout, const float* x_scale,
                    const uint8_t* wq, int w_layout, const void* w_scale,
                    int w_scale_dtype, int64_t w_group, int64_t M, int64_t N,
                    int64_t K, float* y, int32_t* acc, void* stream);
/*   Offset-binary weights (W4A4_WEIGHTS_TILED_OB, w_group 0) pair with
 *   W4A4_CODES_PACKED_TILED_OB codes at any M, or with W4A4_CODES_PACKED_TILED
 *   codes for M <= 32; W4A4_CODES_PACKED_TILED_OB codes need such weights.
 *   Other combinations return W4A4_ERR_INVALID_ARG or W4A4_ERR_UNSUPPORTED. */

/*
 * Converts tiled int4 weights to the offset-binary tiled layout (a storage
 * encoding of the same codes; see W4A4_WEIGHTS_TILED_OB).
 *   wq   [ceil(N/16)*16, K/2] bytes in W4A4_WEIGHTS_TILED (K a multiple of
 *        128), as written by w4a4_quantize_weight_int4.
 *   out  ceil(N/16)*16 * (K/2 + 4) bytes: the converted tiles, then the
 *        per-row sums of the codes at even channels.  out may equal wq when
 *        that buffer has room for the sums.  Padding rows are converted like
 *        the others; their sums are unspecified.
 * Meant for weight preparation; the weight scales are unchanged.
 */
int w4a4_weights_tiled_to_ob(const uint8_t* wq, int64_t N, int64_t K, uint8_t* out,
                             void* stream);

/* Bytes of workspace qlinear_forward needs for these sizes (0 if M or N is
 * 0).  Calls that share one workspace must not overlap in time (the codes
 * and scales live there). */
size_t w4a4_qlinear_workspace_size(int64_t M, int64_t N, int64_t K, int64_t rank);

/*
 * Where w4a4_qlinear_forward (act_bits 4) or w4a8_qlinear_forward
 * (act_bits 8) leaves the activation codes and scales in its workspace, for
 * a call with the same M, N, K, rank, weight layout and w_group (for
 * inspection and testing):
 *   codes_offset  byte offset of the codes, stored in *codes_layout (a
 *                 w4a4_codes_layout: the layout the GEMM reads);
 *   scale_offset  byte offset of the float32 per-token scales [M].
 * Returns W4A4_ERR_INVALID_ARG for sizes <= 0, a bad layout or act_bits, or
 * a NULL output pointer.
 */
int w4a4_qlinear_workspace_layout(int64_t M, int64_t N, int64_t K, int64_t rank, int w_layout,
                                  int64_t w_group, int act_bits, size_t* codes_offset,
                                  int* codes_layout, size_t* scale_offset);

/*
 * The whole layer: rotate + quantize X, int4 GEMM, dequant, + X.A.B.
 *   x [M, K] in x_dtype; wq (in w_layout) / w_scale as prepared by
 *   w4a4_quantize_weight_int4 with the same had_block and w_group.  Tiled
 *   weights take the fastest GEMM (K a multiple of 128, w_group 0 or a
 *   multiple of 128).
 *   The rank-r factors are passed transposed so that both are contiguous
 *   along their contraction: At [rank, K] (At[j, k] = A[k, j]) and
 *   Bt [N, rank] (Bt[n, j] = B[j, n]), in x_dtype, or NULL when rank is 0.
 *   With fp16 inputs rank must be a multiple of 8; T = X.A is kept as an
 *   fp16 pair (hi + lo, about 22 significant bits) for the fp16 matrix
 *   instructions of the epilogue.
 *   y [M, N] float32 output.
 *   workspace: device scratch of at least w4a4_qlinear_workspace_size bytes,
 *   used for the activation codes, scales and X.A; its contents on entry do
 *   not matter.
 */
int w4a4_qlinear_forward(const void* x, int x_dtype, const uint8_t* wq,
                         int w_layout, const void* w_scale, int w_scale_dtype,
                         int64_t M, int64_t N, int64_t K, int64_t had_block,
                         int64_t w_group, const void* At, const void* Bt,
                         int64_t rank, float* y, void* workspace,
                         size_t ws_bytes, void* stream);

/*
 * w4a4_qlinear_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The activation codes, scales and X.A
 * live in a fixed array of W4A4_NOALLOC_SCRATCH_BYTES inside the library:
 * each GPU the library runs on holds its own copy from module load until the
 * process ends, and every call on that GPU uses it, so calls that overlap in
 * time on one GPU race (serialise them, e.g. on one stream).  The call
 * allocates nothing.
 *   Arguments, layouts and results as w4a4_qlinear_forward.
 *   Returns W4A4_ERR_WORKSPACE, with nothing enqueued, when
 *   w4a4_qlinear_workspace_size(M, N, K, rank) exceeds
 *   W4A4_NOALLOC_SCRATCH_BYTES (at rank 0: M * K up to about 32 Mi).
 */
#define W4A4_NOALLOC_SCRATCH_BYTES (32u << 20)
int w4a4_qlinear_forward_noalloc(const void* x, int x_dtype, const uint8_t* wq, int w_layout,
                                 const void* w_scale, int w_scale_dtype, int64_t M, int64_t N,
                                 int64_t K, int64_t had_block, int64_t w_group, const void* At,
                                 const void* Bt, int64_t rank, float* y, void* stream);

/*
 * The W4A8 layer (DynamicPTQ page, "Metodología" §2): w4a4_qlinear_forward
 * with 8-bit per-token activation codes (w4a4_quantize_act_int8's rule) on
 * the same 4-bit weights, GEMM and epilogue.  Arguments, layouts, workspace
 * and errors as w4a4_qlinear_forward.
 */
int w4a8_qlinear_forward(const void* x, int x_dtype, const uint8_t* wq,
                         int w_layout, const void* w_scale, int w_scale_dtype,
                         int64_t M, int64_t N, int64_t K, int64_t had_block,
                         int64_t w_group, const void* At, const void* Bt,
                         int64_t rank, float* y, void* workspace,
                         size_t ws_bytes, void* stream);

/*
 * MXFP4 form of the 4-bit path (SERQ page, "Metodología" item 2 and
 * "Contribuciones Clave": the path may be INT4 or MXFP4), following the OCP
 * microscaling format: every 32 consecutive elements along K share the
 * scale 2^e, stored as the E8M0 byte e + 127, with
 *   e = max(floor(log2(max|v|)) - 2, -127)   (-127 for an all-zero block);
 * each element is the FP4 E2M1 code of v / 2^e: the nearest of
 * {0, 0.5, 1, 1.5, 2, 3, 4, 6} with ties to the even encoding, saturating at
 * 6, sign of the quotient in bit 3 (negative zero included, as an IEEE
 * conversion keeps it).  Codes are packed two per byte like the int4 codes.
 */

/*
 * MXFP4 quantization with the block Hadamard rotation in front (had_block
 * 0/1: none), for activations and, offline, for weights.
 *   codes_layout W4A4_CODES_PACKED: xq [M, K/2], x_scale [M, K/32] bytes;
 *   W4A4_CODES_PACKED_TILED (K a multiple of 128): xq in the 1 KB tile
 *   layout, x_scale [ceil(M/16) * (K/128) * 64] bytes, where byte
 *   (g * 16 + r) of the 64-byte tile (b, t), at (b * (K/128) + t) * 64, is
 *   the scale of elements [128 t + 32 g, +32) of row 16 b + r.
 */
int w4a4_quantize_mxfp4(const void* x, int x_dtype, int64_t M, int64_t K, int64_t had_block,
                        uint8_t* xq, int codes_layout, uint8_t* x_scale, void* stream);

/*
 * MXFP4 GEMM on the CDNA4 scaled FP4 matrix instruction:
 *   y[m,n] = sum_blocks 2^(e_x + e_w) sum_k fp4_x[m,k] fp4_w[n,k]
 * with float32 accumulation.  xq/x_scale and wq/w_scale in the tiled
 * layouts of w4a4_quantize_mxfp4; K a multiple of 128; y [M, N] float32.
 */
int w4a4_qgemm_mxfp4(const uint8_t* xq, const uint8_t* x_scale, const uint8_t* wq,
                     const uint8_t* w_scale, int64_t M, int64_t N, int64_t K, float* y,
                     void* stream);

/*
 * The MXFP4 layer: rotate + MXFP4-quantize X, MXFP4 GEMM with weights from
 * w4a4_quantize_mxfp4 (same had_block, tiled), plus the optional rank-r term
 * as in w4a4_qlinear_forward.
 *   workspace: at least w4a4_qlinear_workspace_size(M, N, K, rank) bytes.
 *   It leaves the activation codes there in the W4A4_CODES_PACKED_TILED
 *   layout at the codes offset that w4a4_qlinear_workspace_layout reports
 *   for tiled int4 weights, and their E8M0 scale tiles (the tiled layout of
 *   w4a4_quantize_mxfp4) at the next multiple of 256 bytes after the codes'
 *   ceil(M / 16) * 16 * K / 2 bytes.
 */
int w4a4_qlinear_forward_mxfp4(const void* x, int x_dtype, const uint8_t* wq,
                               const uint8_t* w_scale, int64_t M, int64_t N, int64_t K,
                               int64_t had_block, const void* At, const void* Bt, int64_t rank,
                               float* y, void* workspace, size_t ws_bytes, void* stream);

/*
 * In-GEMM 4-bit residual of salient channels (SERQ page, "Metodología"
 * items 2-3): the weight rows that collect the most quantization error
 * (input channels, permuted offline so that they are the first r channels,
 * with the activations reordered by the previous layer) are reconstructed
 * by one 4-bit matrix R, and the layer adds X_s . R^T with X_s the same
 * 4-bit activation codes of those channels.  Here R is the rounding error of
 * those channels' weights on the step s_w / 8:
 *   e = RN(w~ - RN(s_w q)),  q_r = clamp(rint(RN(e / RN(s_w / 8))), -8, 7),
 *   y[m,n] = s_x[m] s_w[n] (sum_k q_x qw + (1/8) sum_{k<r} q_x q_r),
 * computed as one int32 sum 8 sum_k q_x qw + sum_{k<r} q_x q_r in the same
 * int8 matrix loop (r extra K columns, rounded up to 128).
 * Limits: K a multiple of 128, 0 <= r <= K and 8 K + r_pad < 131072
 * (r_pad = r rounded up to a multiple of 128), which keeps the int32 sum
 * exact for 4-bit codes.
 */

/*
 * Offline weight preparation with the residual: as w4a4_quantize_weight_int4
 * with per-channel scales (w_group 0) and W4A4_WEIGHTS_TILED output, plus
 * the residual codes of channels [0, res_rank).
 *   wq  [ceil(N/16)*16, (K + r_pad)/2] bytes: every 16-row block holds its
 *       K/128 code tiles followed by r_pad/128 residual tiles in the same
 *       1 KB tile layout (residual tile t' holds channels 128 t' ...; codes
 *       of channels r .. r_pad - 1 are 0).
 *   w_scale [N] in scale_dtype.
 */
int w4a4_quantize_weight_residual_int4(const void* w, int w_dtype, int64_t N, int64_t K,
                                       int64_t had_block, int64_t res_rank, uint8_t* wq,
                                       void* w_scale, int scale_dtype, void* stream);

/*
 * GEMM with the in-GEMM residual: xq W4A4_CODES_PACKED_TILED codes and
 * x_scale [M]; wq, w_scale from w4a4_quantize_weight_residual_int4 with the
 * same res_rank.
 *   y   [M, N] float32: s_x[m] s_w[n] (acc[m,n] / 8), or NULL;
 *   acc [M, N] int32: the exact 8 sum_k q_x qw + sum_{k<r} q_x q_r, or NULL.
 */
int w4a4_qgemm_residual(const uint8_t* xq, const float* x_scale, const uint8_t* wq,
                        const void* w_scale, int w_scale_dtype, int64_t res_rank, int64_t M,
                        int64_t N, int64_t K, float* y, int32_t* acc, void* stream);

/*
 * The layer with the in-GEMM residual: rotate + quantize X per token
 * (w4a4_quantize_act_int4's rule), then w4a4_qgemm_residual.
 *   workspace: at least w4a4_qlinear_workspace_size(M, N, K, 0) bytes.
 *   Other arguments and errors as w4a4_qlinear_forward.
 */
int w4a4_qlinear_forward_residual(const void* x, int x_dtype, const uint8_t* wq,
                                  const void* w_scale, int w_scale_dtype, int64_t res_rank,
                                  int64_t M, int64_t N, int64_t K, int64_t had_block, float* y,
                                  void* workspace, size_t ws_bytes, void* stream);

/*
 * Asymmetric group-wise activations (OffQ page, "Metodología" steps 2-3):
 * the all-ones first row of the Hadamard block turns a channel's outlier
 * into a constant offset over its group, which the zero point of a
 * per-group asymmetric quantizer absorbs.
 *
 * Activation quantizer, per token and group of `group` channels (the
 * Hadamard block), in float32:
 *   s = (max - min) / 15,  z = rint(-min / s),
 *   q = clamp(rint(x~ / s) + z, 0, 15),  so that x~ ~ s (q - z).
 * The zero point z is an int32 that is not clamped to [0, 15]: an offset
 * larger than the group's spread moves it past the code range.  A group of
 * equal values c takes the range spanned by c and 0; s = 0 gives q = z = 0.
 * Codes are stored as the signed nibble q - 8 (q with its top bit flipped),
 * in the W4A4_CODES_PACKED or W4A4_CODES_PACKED_TILED layout.
 *   x        [M, K] in x_dtype.
 *   group    a power of two in [128, 4096] dividing K.
 *   had_block 0/1: x is already rotated; otherwise equal to group.
 *   x_scale  [M, K/group] float32 output, x_zero [M, K/group] int32 output.
 */
int w4a4_quantize_act_asym_int4(const void* x, int x_dtype, int64_t M, int64_t K,
                                int64_t had_block, int64_t group, uint8_t* xq,
                                int codes_layout, float* x_scale, int32_t* x_zero,
                                void* stream);

/*
 * Offline weight group sums for the asymmetric product (OffQ page,
 * "Metodología" step 3: per-group zero points):
 *   w_gsum[n, g] = sum of the signed weight codes of row n over channels
 *   [g*group, (g+1)*group), int32 [N, K/group].
 *   wq packed in w_layout; group a multiple of 64 dividing K.
 */
int w4a4_weight_group_sums(const uint8_t* wq, int w_layout, int64_t N, int64_t K,
                           int64_t group, int32_t* w_gsum, void* stream);

/*
 * GEMM of asymmetric activation codes with int4 weights (OffQ page,
 * "Metodología" steps 2-3; SERQ page, "Resumen técnico" §3):
 *   y[m,n] = w_scale[n] * sum_g x_scale[m,g] * (sum_{k in g} q[m,k] qw[n,k]
 *                                               - x_zero[m,g] * w_gsum[n,g])
 * with q the uint4 codes (stored as q - 8) of w4a4_quantize_act_asym_int4.
 *   xq       W4A4_CODES_PACKED_TILED codes; x_scale, x_zero [M, K/group].
 *   wq       W4A4_WEIGHTS_TILED codes, w_scale [N] (per channel) in
 *            w_scale_dtype, w_gsum [N, K/group] from w4a4_weight_group_sums.
 *   group    a power of two in [128, 4096] dividing K; K a multiple of 128.
 *   y        [M, N] float32 output.  The integer sums are exact; the
 *            zero-point term is formed with about 22 significant bits.
 */
int w4a4_qgemm_asym(const uint8_t* xq, const float* x_scale, const int32_t* x_zero,
                    int64_t group, const uint8_t* wq, const void* w_scale,
                    int w_scale_dtype, const int32_t* w_gsum, int64_t M, int64_t N,
                    int64_t K, float* y, void* stream);

/*
 * The layer with asymmetric group-wise activations: rotate by Hadamard
 * blocks of had_block (a power of two in [128, 4096]), quantize each
 * (token, block) with w4a4_quantize_act_asym_int4's rule, w4a4_qgemm_asym,
 * plus the optional rank-r term as in w4a4_qlinear_forward.
 *   wq W4A4_WEIGHTS_TILED with per-channel scales (w_group 0) from
 *   w4a4_quantize_weight_int4 with the same had_block; w_gsum from
 *   w4a4_weight_group_sums with group = had_block.
 *   workspace: at least w4a4_qlinear_workspace_size(M, N, K, rank) bytes.
 *   It leaves the activation codes there in the W4A4_CODES_PACKED_TILED
 *   layout at the codes offset that w4a4_qlinear_workspace_layout reports
 *   for tiled int4 weights; the float32 group scales [M, K / had_block] at
 *   the next multiple of 256 bytes after the codes' ceil(M / 16) * 16 * K / 2
 *   bytes, and the int32 zero points [M, K / had_block] at the next multiple
 *   of 256 bytes after the scales.
 *   Other arguments and errors as w4a4_qlinear_forward.
 */
int w4a4_qlinear_forward_asym(const void* x, int x_dtype, const uint8_t* wq,
                              const void* w_scale, int w_scale_dtype,
                              const int32_t* w_gsum, int64_t M, int64_t N, int64_t K,
                              int64_t had_block, const void* At, const void* Bt,
                              int64_t rank, float* y, void* workspace,
                              size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A4_H */
