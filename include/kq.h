/*
 * kq.h -- C ABI of the KroQuant online activation quantizer for AMD Instinct
 * MI355X (gfx950).
 *
 * The method (KroQuant, arXiv 2607.21446v1):
 *   - Sec. 1, Eq. 1: an invertible transform T is applied to the activations
 *     (A -> A T) and its inverse to the weights (W -> W T^{-T}); the product
 *     A W^T is unchanged.
 *   - Sec. 3.1, Eq. 4: T is block diagonal, one 32x32 block K^(j) per group of
 *     32 consecutive channels.
 *   - Sec. 3.2, Eq. 5: each block is a Kronecker product of five 2x2 factors,
 *     K = G1 (x) G2 (x) G3 (x) G4 (x) G5; Sec. 3.5.1, Eq. 12: entry-wise,
 *     K[r][c] = prod_{k=1..5} G_k[bit_{5-k}(r)][bit_{5-k}(c)], so G1 mixes
 *     channels 16 apart and G5 neighbouring channels.
 *   - Sec. 3.1 and Sec. 4.1 "Data format" / Appendix D: the result is quantized
 *     block-wise to MXFP4: 32 E2M1 elements sharing one E8M0 scale (OCP MX).
 *
 * Number format (OCP MX v1.0 reading; the paper names the format only):
 *   shared exponent e = floor(log2(max_i |y_i|)) - 2, clamped to [-127, 127]
 *   (an all-zero block takes e = -127); scale byte = e + 127 (E8M0). Each
 *   element v = y / 2^e is rounded to the nearest of {0, 0.5, 1, 1.5, 2, 3, 4, 6}
 *   with ties to the even code, larger magnitudes saturate to 6. A code is
 *   sign << 3 | index of that magnitude (0x0 = 0 ... 0x7 = 6); the sign bit
 *   follows y, also for zeros.
 *
 * Layouts (all row-major, no padding in the outputs):
 *   A        bf16 bit patterns, [m][lda], lda >= d; d % 32 == 0
 *   codes    uint8 [m][d/2]: element 2k in the low nibble of byte k of its row
 *   scales   uint8 [m][d/32]: E8M0 byte of block j of row i at [i][j]
 *   factors  fp32 [d/32][5][2][2]: factors[j][k-1][r][c] = G_k[r][c] of block j,
 *            so factors[j][0] is G1 (channel bit 4) and factors[j][4] is G5 (bit 0)
 *
 * Conventions for every entry point that takes a stream:
 *   - Pointers named "device" point to GPU memory that the caller allocates,
 *     owns and keeps alive until the enqueued work has finished. The library
 *     allocates nothing and never synchronizes; the only state it keeps
 *     between calls is a per-device cache of the compute-unit count (read once
 *     with hipDeviceGetAttribute by the packed GEMMs to size their launches).
 *   - Work is enqueued on `stream` (NULL = the default stream) and runs
 *     asynchronously; results are valid once the stream has reached it.
 *   - Arguments are checked on the host before anything is enqueued; on an
 *     error nothing is launched and the status says why. A launch the HIP
 *     runtime rejects returns KQ_ERR_HIP; kq_last_hip_error() then gives the
 *     hipError_t value (per host thread).
 *   - With m == 0 (or d == 0) nothing is read, written or launched and KQ_OK
 *     is returned.
 *   - Inputs must be finite; NaN or Inf inputs give unspecified codes.
 *   - Outputs must not overlap inputs.
 *   - The GEMM-family entry points (kq_mxfp4_gemm*, kq_lowrank_project*,
 *     kq_dequantize_mxfp4_bf16, kq_pack_mxfp4_scales, kq_gemm_f32,
 *     kq_transform_quantize_mxfp4_gemm) refuse any size or leading dimension
 *     of 2^31 or more with KQ_ERR_UNSUPPORTED, before their finer limits.
 */
#ifndef KQ_H
#define KQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t. */
typedef struct ihipStream_t *kq_stream_t;

typedef enum {
    KQ_OK = 0,
    KQ_ERR_NULL = 1,        /* a required pointer is NULL */
    KQ_ERR_SHAPE = 2,       /* negative size, d % 32 != 0, lda < d, or size overflow */
    KQ_ERR_ALIGN = 3,       /* a pointer or leading dimension breaks the stated alignment */
    KQ_ERR_HIP = 4,         /* the HIP runtime rejected the launch */
    KQ_ERR_UNSUPPORTED = 5  /* argument combination outside what the kernels handle */
} kq_status;

/*
 * Quantize-only (T = I): codes/scales of A itself.
 * KroQuant Sec. 3.1 blockwise quantizer; Sec. 4.4 / Table 3 "Q4" kernel.
 *   A       device, bf16 bits [m][lda]; 16-byte aligned, lda % 8 == 0
 *   codes   device, [m][d/2] bytes, 16-byte aligned
 *   scales  device, [m][d/32] bytes
 * Results are bit-exact to the format definition above.
 */
kq_status kq_quantize_mxfp4(const uint16_t *A, int64_t m, int64_t d, int64_t lda,
                            uint8_t *codes, uint8_t *scales, kq_stream_t stream);

/*
 * Fused Kronecker transform + quantize: for every row a of A and block j,
 * y = a[32j : 32j+32] . K^(j) (Eq. 1's A T with Eq. 4-5 and Eq. 12), computed
 * in fp32, then quantized from fp32 as above (no rounding to bf16 in between).
 *   factors  device, fp32 [d/32][5][2][2], 16-byte aligned (layout above)
 *   y_debug  device or NULL; if given, fp32 [m][d] receives y (check mode),
 *            16-byte aligned. Codes and scales do not depend on it.
 * Other arguments as kq_quantize_mxfp4.
 *
 * Range. y is evaluated in fp32 as five stages in the factored form
 * G = [[1, p], [q, 1]] diag(G[0][0], G[1][1]) (p = G[0][1] / G[1][1],
 * q = G[1][0] / G[0][0]; Sec. 3.2's mixed-product rule collects the diagonals
 * into one per-channel multiply). A stage grows a block's largest magnitude by
 * at most 1 + max(|p|, |q|), so a block's scale and codes are as specified
 * when max|a| prod_k (1 + max(|p_k|, |q_k|)) < 2^128 (Hadamard factors: 2^5,
 * i.e. any |a| < 2^123). For a block that breaks it, an fp32 intermediate may
 * overflow and its scale and codes are unspecified (the fp64 definition above
 * would keep y finite and clamp e at 127). Blocks of a 16-block segment
 * containing a factor with |p| or |q| > 2^20 run the plain 2x2 stages
 * instead, where the growth per stage is max_c (|G[0][c]| + |G[1][c]|).
 */
kq_status kq_transform_quantize_mxfp4(const uint16_t *A, int64_t m, int64_t d, int64_t lda,
                                      const float *factors, uint8_t *codes, uint8_t *scales,
                                      float *y_debug, kq_stream_t stream);

/*
 * Forms of the fused transform (Sec. 3.5.1 "Kernel variants": the block product
 * y = a K as a dense 32x32 product with K materialized from Eq. 12, or, this
 * library's default, as stages of the 2x2 factors):
 *   KQ_FORM_BUTTERFLY  five in-register 2x2 stages (what kq_transform_quantize_mxfp4 runs)
 *   KQ_FORM_MFMA       K materialized per block as three bf16 terms (exact for
 *                      fp32 K) on bf16 matrix instructions, operands loaded directly
 *   KQ_FORM_MFMA_LDS   the same through LDS-staged row-major tiles; needs
 *                      d % 512 == 0, otherwise the butterfly form runs
 * The matrix forms accumulate in fp32 in another order: the same tolerance
 * against the exact transform, not bit-identical to the butterfly form. Their
 * range condition: max|a| prod_k max_c (|G_k[0][c]| + |G_k[1][c]|) < 2^128.
 */
typedef enum { KQ_FORM_BUTTERFLY = 0, KQ_FORM_MFMA = 1, KQ_FORM_MFMA_LDS = 2 } kq_transform_form;

/*
 * kq_transform_quantize_mxfp4 in a chosen form (a kq_transform_form value;
 * any other value: KQ_ERR_UNSUPPORTED). Arguments and rules otherwise as
 * kq_transform_quantize_mxfp4.
 */
kq_status kq_transform_quantize_mxfp4_form(const uint16_t *A, int64_t m, int64_t d, int64_t lda,
                                           const float *factors, uint8_t *codes, uint8_t *scales,
                                           float *y_debug, int form, kq_stream_t stream);

/*
 * SmoothQuant baseline (KroQuant Appendix D.2; Sec. 4.4 "Scale" kernel):
 * T = diag(1 / gamma), i.e. y_c = fl32(a_c * inv_scale[c]) (one fp32 multiply),
 * then quantize as above.
 *   inv_scale  device, fp32 [d] = 1 / gamma_c, 16-byte aligned
 * Other arguments as kq_quantize_mxfp4. Bit-exact whenever every product
 * fl32(a_c * inv_scale[c]) is finite (an overflowing product: unspecified codes).
 */
kq_status kq_smoothquant_quantize_mxfp4(const uint16_t *A, int64_t m, int64_t d, int64_t lda,
                                        const float *inv_scale, uint8_t *codes, uint8_t *scales,
                                        kq_stream_t stream);

/*
 * Quantize-only on fp32 input: the blockwise MXFP4 quantizer of Sec. 3.1
 * (format as above) applied to fp32 values, e.g. the folded weights W T^{-T}
 * of Eq. 1 before the W4A4 product of Eq. 2.
 *   X  device, fp32 [m][ldx], 16-byte aligned, ldx >= d, ldx % 4 == 0, finite
 * Other arguments as kq_quantize_mxfp4. Bit-exact.
 */
kq_status kq_quantize_mxfp4_f32(const float *X, int64_t m, int64_t d, int64_t ldx,
                                uint8_t *codes, uint8_t *scales, kq_stream_t stream);

/*
 * Weight fold W' = W T^{-T} (Eq. 1; Sec. 3.2: the inverse of a Kronecker
 * product is the Kronecker product of the 2x2 inverses). Per block,
 * w' = w . (K^(j))^{-T}, applied as five 2x2 stages with (G_k^{-1})^T in fp32.
 *   W         device, fp32 [o][d], 16-byte aligned
 *   factors   as kq_transform_quantize_mxfp4; every G_k must be invertible
 *   W_folded  device, fp32 [o][d], 16-byte aligned
 */
kq_status kq_inverse_fold_weights(const float *W, int64_t o, int64_t d, const float *factors,
                                  float *W_folded, kq_stream_t stream);

/*
 * W4A4 GEMM on MXFP4 operands (the downstream product of Eq. 2,
 * Q(A T) Q(W T^{-T})^T, used to check the quantizer's output end to end):
 *   O[i][j] = sum_k deq(A)[i][k] * deq(W)[j][k],  deq(code, scale) = E2M1(code) * 2^(scale - 127),
 * fp32 accumulation on gfx950's scaled FP4 matrix instructions.
 *   codes_a   device, [m][k/2] bytes (layout of kq_quantize_mxfp4), 16-byte aligned
 *   scales_a  device, [m][k/32]
 *   codes_w   device, [n][k/2] bytes (e.g. kq_quantize_mxfp4_f32 of the folded weights), 16-byte aligned
 *   scales_w  device, [n][k/32]
 *   O         device, fp32 [m][ldo], ldo >= n; written, not accumulated into
 * k must be a multiple of 32 (KQ_ERR_SHAPE) and k/2 a multiple of 16 (KQ_ERR_ALIGN).
 * When k is a positive multiple of 256 and the scales and O are 4-byte aligned,
 * the product runs on the 256 x 256-tile kernel of kq_mxfp4_gemm_packed, which
 * then reads these MX-layout scales directly (bit-identical to the packed-scale
 * call on the same operands); otherwise on a 128 x 128-tile kernel. Summation
 * order inside the matrix instruction is the hardware's; results agree with an
 * fp64 sum of the same dequantized products to fp32 rounding.
 */
kq_status kq_mxfp4_gemm(const uint8_t *codes_a, const uint8_t *scales_a, const uint8_t *codes_w,
                        const uint8_t *scales_w, int64_t m, int64_t n, int64_t k, float *O, int64_t ldo,
                        kq_stream_t stream);

/*
 * The same W4A4 GEMM as kq_mxfp4_gemm (identical arguments, layouts and error
 * rules) on 128 x 512 output tiles of eight waves, k advancing 128 per stage,
 * with the 32 x 32 x 64 scaled instruction (one 64-k block per instruction,
 * increasing k) as kq_mxfp4_gemm_packed: bit-identical to that one where it
 * applies (k % 256 == 0); against kq_mxfp4_gemm (128-k blocks), agreement to
 * fp32 rounding of the partial sums.
 * m rows of codes_a (k/2 bytes each) and 512 rows of codes_w must each span
 * fewer than 2^31 bytes per tile (KQ_ERR_UNSUPPORTED otherwise).
 */
kq_status kq_mxfp4_gemm_wide(const uint8_t *codes_a, const uint8_t *scales_a, const uint8_t *codes_w,
                             const uint8_t *scales_w, int64_t m, int64_t n, int64_t k, float *O, int64_t ldo,
                             kq_stream_t stream);

/*
 * Re-layout of MXFP4 scales for kq_mxfp4_gemm_packed (a format change only,
 * no arithmetic): the E8M0 bytes of Sec. 3.1's blocks, [rows][k/32] as the
 * quantizers write them, become [k/256][rows][8], i.e. the eight scale bytes
 * of one 256-wide k stage of consecutive rows are consecutive, even blocks of
 * the stage first: bytes 0-3 hold blocks 0, 2, 4, 6 and bytes 4-7 blocks 1, 3,
 * 5, 7 (the product reads the dword of its block parity and selects byte j for
 * the stage's j-th pair of blocks with the instruction's byte select).
 *   packed[(s * rows + i) * 8 + 4 p + j] = scales[i * (k/32) + 8 s + 2 j + p]
 *   (p in 0..1, j in 0..3)
 *   scales   device, [rows][k/32] bytes (no alignment needed)
 *   packed   device, rows * (k/32) bytes, 8-byte aligned; must not overlap scales
 * k % 256 == 0 (KQ_ERR_SHAPE); rows == 0 or k == 0 is a no-op.
 */
kq_status kq_pack_mxfp4_scales(const uint8_t *scales, int64_t rows, int64_t k, uint8_t *packed,
                               kq_stream_t stream);

/*
 * The W4A4 GEMM of Eq. 2 (as kq_mxfp4_gemm: O[i][j] = sum_k deq(A)[i][k]
 * deq(W)[j][k], fp32 accumulation on the scaled FP4 matrix instructions) with
 * both operands' scales in the packed layout of kq_pack_mxfp4_scales. It runs
 * on 256 x 256 output tiles with the 32 x 32 x 64 instruction (64 k per
 * instruction, increasing k), so its results agree with kq_mxfp4_gemm to fp32
 * rounding of the partial sums, and bit-for-bit whenever the fp32 sums are
 * exact. One launch: whole rounds of tiles (one per compute unit at a time),
 * and a last partial round of at most half the compute units as 256 x 128
 * halves (computed first on half the units when the counts allow, so that the
 * units' output stores do not all coincide); every output element gets the
 * same instructions either way. At most 2^30 tiles (KQ_ERR_UNSUPPORTED).
 *   codes_a          device, [m][k/2] bytes, 16-byte aligned
 *   packed_scales_a  device, packed [k/256][m][8], 16-byte aligned
 *   codes_w          device, [n][k/2] bytes, 16-byte aligned
 *   packed_scales_w  device, packed [k/256][n][8], 16-byte aligned
 *   O                device, fp32 [m][ldo], ldo >= n, 4-byte aligned; written, not
 *                    accumulated into (k == 0 writes zeros and reads no operand, which
 *                    may then be NULL)
 * k % 256 == 0 (KQ_ERR_SHAPE). 256 rows of codes, m k/32 and n k/32 scale
 * bytes and 256 rows of O must each span fewer than 2^31 bytes
 * (KQ_ERR_UNSUPPORTED).
 */
kq_status kq_mxfp4_gemm_packed(const uint8_t *codes_a, const uint8_t *packed_scales_a, const uint8_t *codes_w,
                               const uint8_t *packed_scales_w, int64_t m, int64_t n, int64_t k, float *O,
                               int64_t ldo, kq_stream_t stream);

/*
 * kq_mxfp4_gemm_packed with O written in bf16: each fp32 result of
 * kq_mxfp4_gemm_packed rounded to the nearest bf16 (ties to even), bit for bit
 * (for the bf16 activations a transformer layer passes on; half the output
 * bytes of the fp32 form).
 *   O   device, bf16 bits [m][ldo], ldo >= n, 2-byte aligned; written
 * Other arguments and rules as kq_mxfp4_gemm_packed (256 rows of O must span
 * fewer than 2^31 bytes).
 */
kq_status kq_mxfp4_gemm_packed_bf16(const uint8_t *codes_a, const uint8_t *packed_scales_a,
                                    const uint8_t *codes_w, const uint8_t *packed_scales_w, int64_t m, int64_t n,
                                    int64_t k, uint16_t *O, int64_t ldo, kq_stream_t stream);

/*
 * The layer of Sec. 3.4 Eq. 11 on the packed-scale GEMM: O = deq(A) deq(W)^T +
 * Z deq(L)^T, the low-rank term added after the product in the same kernel (Z
 * split into two bf16 terms, exact to 2^-16 relative; deq(L) exact in bf16),
 * so O is written once.
 *   codes_a ... k, O, ldo   as kq_mxfp4_gemm_packed (W here is the residual W~ - L R)
 *   Z                       device, fp32 [m][r], 16-byte aligned (kq_lowrank_project)
 *   codes_l, scales_l       device, L in MXFP4: [n][r/2] (4-byte aligned), [n][r/32]
 * r > 0, r % 32 == 0 (KQ_ERR_SHAPE); limits as kq_mxfp4_gemm_packed.
 */
kq_status kq_mxfp4_gemm_packed_lowrank(const uint8_t *codes_a, const uint8_t *packed_scales_a,
                                       const uint8_t *codes_w, const uint8_t *packed_scales_w, int64_t m, int64_t n,
                                       int64_t k, const float *Z, const uint8_t *codes_l, const uint8_t *scales_l,
                                       int64_t r, float *O, int64_t ldo, kq_stream_t stream);

/*
 * kq_mxfp4_gemm_packed_lowrank with the low-rank operands prepared once outside
 * the product (Sec. 3.4 Eq. 11's Z deq(L)^T): Z split as Zh = bf16(Z) and
 * Zl = bf16(Z - Zh) (what kq_lowrank_project_bf16_split writes) and deq(L) in
 * bf16 (exact; kq_dequantize_mxfp4_bf16 of L's codes and scales). Every output
 * is the same sum, in the same order, as kq_mxfp4_gemm_packed_lowrank's on the
 * fp32 Z that Zh + Zl split (bit-identical); the kernel moves the operands
 * straight into LDS instead of converting them per tile.
 *   codes_a .. k, O, ldo   as kq_mxfp4_gemm_packed_lowrank
 *   Zh, Zl                 device, bf16 bits [m][r], 16-byte aligned
 *   L16                    device, bf16 bits [n][r] (deq(L)), 16-byte aligned
 *   r                      r > 0, r % 32 == 0 (KQ_ERR_SHAPE)
 * Size limits as kq_mxfp4_gemm_packed_lowrank (512 r below 2^31).
 */
kq_status kq_mxfp4_gemm_packed_lowrank_split(const uint8_t *codes_a, const uint8_t *packed_scales_a,
                                             const uint8_t *codes_w, const uint8_t *packed_scales_w, int64_t m,
                                             int64_t n, int64_t k, const uint16_t *Zh, const uint16_t *Zl,
                                             const uint16_t *L16, int64_t r, float *O, int64_t ldo,
                                             kq_stream_t stream);

/*
 * The W4A4 layer with the activation transform and quantizer inside the
 * product (Sec. 1 Eq. 1-2; Sec. 3.2 Eq. 5 and Sec. 3.5.1 Eq. 12 for T; Sec. 3.1
 * for Q):
 *   O = deq(Q(A T)) deq(W)^T,
 * where Q(A T) is what kq_transform_quantize_mxfp4 writes for the same A and
 * factors, computed in the product's prologue and kept on chip, and W is
 * already in MXFP4 (e.g. kq_quantize_mxfp4_f32 of kq_inverse_fold_weights).
 * Blocks are transformed in groups of four (128 channels, one k stage); a group
 * in which every block admits the shear form uses it, else the general 2x2
 * stages, so for factors where some block lacks the shear form the activation
 * codes can differ from the standalone quantizer's at rounding ties (both
 * meet the same tolerance against the exact transform). When every block
 * admits it, O is bit-identical to kq_transform_quantize_mxfp4 followed by
 * kq_mxfp4_gemm_wide (the same product kernel).
 *   A         device, bf16 bits [m][lda], lda >= k, lda % 8 == 0, 16-byte aligned
 *   factors   device, fp32 [k/32][5][2][2] (as kq_transform_quantize_mxfp4), 16-byte aligned
 *   codes_w   device, [n][k/2] bytes, 16-byte aligned
 *   scales_w  device, [n][k/32] (4-byte aligned when k/32 % 4 == 0)
 *   O         device, fp32 [m][ldo], ldo >= n; written, not accumulated into
 * k % 32 == 0 (KQ_ERR_SHAPE); 128 rows of A (2 lda bytes each) and 512 rows of
 * codes_w must each span fewer than 2^31 bytes (KQ_ERR_UNSUPPORTED).
 */
kq_status kq_transform_quantize_mxfp4_gemm(const uint16_t *A, int64_t m, int64_t k, int64_t lda,
                                           const float *factors, const uint8_t *codes_w, const uint8_t *scales_w,
                                           int64_t n, float *O, int64_t ldo, kq_stream_t stream);

/*
 * Block-Hadamard transform + quantize: the fixed-rotation baselines the paper
 * compares against -- Sec. 1 and Table 2 (Hadamard at the MXFP4 block size,
 * n = 32) and Sec. 4.4 / Table 3 (the fast Walsh-Hadamard transform over the
 * whole power-of-two width, n = d). For every row a of A and every group of n
 * consecutive channels starting at a multiple of n,
 *   y = a[g n : g n + n] . H_n / sqrt(n),  H_n[r][c] = (-1)^popcount(r & c),
 * the normalized Sylvester matrix (Sec. 3.2 "Hadamard initialization": the
 * k-fold Kronecker power of [[1,1],[1,-1]]/sqrt(2)); at n = 32 this is the
 * Kronecker transform with every factor equal to that 2x2. y is computed in
 * fp32 and quantized as above.
 *   n        power of two with 32 <= n <= 16384 and d % n == 0 (else
 *            KQ_ERR_SHAPE; a power of two above 16384: KQ_ERR_UNSUPPORTED).
 *            Non-power-of-two widths need padding, which this call does not do.
 *   y_debug  device or NULL; fp32 [m][d] receives y (check mode), 16-byte aligned.
 * m * (d / n) must stay below 2^32 (KQ_ERR_UNSUPPORTED). Other arguments as
 * kq_quantize_mxfp4.
 */
kq_status kq_hadamard_quantize_mxfp4(const uint16_t *A, int64_t m, int64_t d, int64_t lda, int64_t n,
                                     uint8_t *codes, uint8_t *scales, float *y_debug,
                                     kq_stream_t stream);

/*
 * As kq_transform_quantize_mxfp4, also writing y rounded to bf16 (nearest,
 * ties to even): the 16-bit activation the low-rank branch of Sec. 3.4 Eq. 11
 * consumes (App. D keeps that branch's activations at 16 bits).
 *   y16  device, bf16 bits [m][d], 16-byte aligned (required)
 */
kq_status kq_transform_quantize_mxfp4_y16(const uint16_t *A, int64_t m, int64_t d, int64_t lda,
                                          const float *factors, uint8_t *codes, uint8_t *scales, uint16_t *y16,
                                          kq_stream_t stream);

/*
 * kq_transform_quantize_mxfp4 (or, with y16, kq_transform_quantize_mxfp4_y16)
 * with the E8M0 scales written straight in the layout kq_pack_mxfp4_scales
 * makes (the layout kq_mxfp4_gemm_packed* read): the same codes and the same
 * scale bytes, bit for bit, rearranged as [d/256][m][8] with the even blocks
 * of each 256-channel stage first -- Sec. 3.1's quantizer of Sec. 3.2 Eq. 5's
 * transform, its output laid out for Sec. 1 Eq. 2's product, so the layer
 * needs no separate re-layout launch.
 *   A, m, d, lda, factors, codes   as kq_transform_quantize_mxfp4
 *   packed_scales                  device, m d/32 bytes (no alignment needed)
 *   y16                            device, bf16 bits [m][d], 16-byte aligned, or
 *                                  NULL (no bf16 output)
 * d % 256 == 0 (KQ_ERR_SHAPE); m d/32 must stay below 2^31 - 16
 * (KQ_ERR_UNSUPPORTED). Error rules otherwise as kq_transform_quantize_mxfp4.
 */
kq_status kq_transform_quantize_mxfp4_packed(const uint16_t *A, int64_t m, int64_t d, int64_t lda,
                                             const float *factors, uint8_t *codes, uint8_t *packed_scales,
                                             uint16_t *y16, kq_stream_t stream);

/*
 * Low-rank branch of Eq. 11, first product: Z = X16 . Q(R)^T, fp32 accumulation
 * (bf16 matrix instructions; the decoded MXFP4 values are exact in bf16).
 *   X16       device, bf16 bits [m][ldx], ldx >= d, ldx % 8 == 0, 16-byte aligned
 *   codes_r   device, [r][d/2] (R in MXFP4, blocks along d), 16-byte aligned
 *   scales_r  device, [r][d/32]
 *   Z         device, fp32 [m][r], 16-byte aligned, written
 * d % 32 == 0, r > 0, r % 32 == 0 (KQ_ERR_SHAPE); 80 rows of X16 and 128 rows of
 * R's codes must each span fewer than 2^31 bytes (KQ_ERR_UNSUPPORTED). The same
 * Z, bit for bit, as kq_lowrank_project_bf16 on kq_dequantize_mxfp4_bf16 of R.
 */
kq_status kq_lowrank_project(const uint16_t *X16, int64_t m, int64_t d, int64_t ldx, const uint8_t *codes_r,
                             const uint8_t *scales_r, int64_t r, float *Z, kq_stream_t stream);

/*
 * As kq_lowrank_project with R already in bf16 (for example R decoded once per
 * call by kq_dequantize_mxfp4_bf16: the decode is exact, so Z is bit-identical
 * to kq_lowrank_project's), so the product spends no vector ALU time on R.
 *   R16  device, bf16 bits [r][d] contiguous, 16-byte aligned
 * Other arguments and rules as kq_lowrank_project; 80 rows of X16 and 128 rows
 * of R16 must each span fewer than 2^31 bytes (KQ_ERR_UNSUPPORTED).
 */
kq_status kq_lowrank_project_bf16(const uint16_t *X16, int64_t m, int64_t d, int64_t ldx, const uint16_t *R16,
                                  int64_t r, float *Z, kq_stream_t stream);

/*
 * kq_lowrank_project_bf16 writing Z as its bf16 split instead of fp32: Zh =
 * bf16(Z) and Zl = bf16(Z - Zh), each rounded to nearest even (Z - Zh is exact
 * in fp32), from the same fp32 sums (so Zh + Zl is Z to 2^-16 relative; the
 * operands kq_mxfp4_gemm_packed_lowrank_split reads, Sec. 3.4 Eq. 11).
 *   X16, m, d, ldx, R16, r   as kq_lowrank_project_bf16
 *   Zh, Zl                   device, bf16 bits [m][r] each (written), 16-byte aligned
 * Errors as kq_lowrank_project_bf16.
 */
kq_status kq_lowrank_project_bf16_split(const uint16_t *X16, int64_t m, int64_t d, int64_t ldx, const uint16_t *R16,
                                        int64_t r, uint16_t *Zh, uint16_t *Zl, kq_stream_t stream);

/*
 * kq_lowrank_project writing Z as its bf16 split (Zh = bf16(Z), Zl = bf16(Z - Zh),
 * as kq_lowrank_project_bf16_split) from R in MXFP4: the operands of
 * kq_mxfp4_gemm_packed_lowrank_split without a decoded copy of R (Sec. 3.4 Eq. 11).
 *   X16, m, d, ldx, codes_r, scales_r, r   as kq_lowrank_project
 *   Zh, Zl                                 device, bf16 bits [m][r] each (written), 16-byte aligned
 * Errors as kq_lowrank_project; bit-identical to kq_lowrank_project_bf16_split on
 * kq_dequantize_mxfp4_bf16 of R.
 */
kq_status kq_lowrank_project_split(const uint16_t *X16, int64_t m, int64_t d, int64_t ldx, const uint8_t *codes_r,
                                   const uint8_t *scales_r, int64_t r, uint16_t *Zh, uint16_t *Zl,
                                   kq_stream_t stream);

/*
 * MXFP4 -> bf16 (Sec. 3.1's dequantization deq(code, scale) = E2M1(code)
 * 2^(scale - 127)): every value has at most two significant bits, so it is
 * exact in bf16 whenever it is a normal or subnormal bf16 number.
 *   codes   device, [rows][k/2] bytes, 4-byte aligned
 *   scales  device, [rows][k/32]
 *   out     device, bf16 bits [rows][k], 16-byte aligned
 * k % 32 == 0 (KQ_ERR_SHAPE).
 */
kq_status kq_dequantize_mxfp4_bf16(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t k,
                                   uint16_t *out, kq_stream_t stream);

/*
 * The W4A4 layer of Eq. 11: O = deq(A) deq(W)^T + Z deq(L)^T, the low-rank term
 * added in the same kernel (Z split into two bf16 terms, exact to 2^-16
 * relative; deq(L) exact in bf16), so O is written once.
 *   codes_a ... ldo   as kq_mxfp4_gemm (W here is the residual W~ - L R)
 *   Z                 device, fp32 [m][r], 16-byte aligned (kq_lowrank_project)
 *   codes_l, scales_l device, L in MXFP4: [n][r/2] (16-byte aligned), [n][r/32]
 * r > 0, r % 32 == 0 (KQ_ERR_SHAPE). Kernel choice as kq_mxfp4_gemm: with k a
 * positive multiple of 256, that of kq_mxfp4_gemm_packed_lowrank on these
 * MX-layout scales (bit-identical to it).
 */
kq_status kq_mxfp4_gemm_lowrank(const uint8_t *codes_a, const uint8_t *scales_a, const uint8_t *codes_w,
                                const uint8_t *scales_w, int64_t m, int64_t n, int64_t k, const float *Z,
                                const uint8_t *codes_l, const uint8_t *scales_l, int64_t r, float *O, int64_t ldo,
                                kq_stream_t stream);

/*
 * fp32 GEMM: D = alpha op(A) op(B) + beta C, row-major operands; op(A) is m x k
 * (A is m x k, or k x m when transa), op(B) is k x n (B is k x n, or n x k when
 * transb). C may be NULL when beta == 0; C and D use the row strides ldc, ldd.
 * fp32 products accumulated in fp32 on the fp32 matrix instruction, two k at a
 * time in ascending k (not bit-identical to a scalar fused multiply-add chain;
 * within the usual fp32 dot-product error bound). Used by the calibration below
 * and usable on its own.
 */
kq_status kq_gemm_f32(int transa, int transb, int64_t m, int64_t n, int64_t k, float alpha, const float *A,
                      int64_t lda, const float *B, int64_t ldb, float beta, const float *C, int64_t ldc, float *D,
                      int64_t ldd, kq_stream_t stream);

/*
 * Layer-wise calibration of the Kronecker factors (Sec. 3.3, Eq. 6-10): Adam
 * on the 15 parameters per block theta[j][k][0..2] = (a, b, c) of
 * G_k = [[a, b], [c a, c b - 1/a]] (Eq. 6) against
 *   L = ||Q(A T) Q(W T^{-T})^T - A W^T||^2/(M o) + lambda_A ||Q(A T) - A T||^2/(M d)
 *     + lambda_W ||Q(W T^{-T}) - W T^{-T}||^2/(o d)                       (Eq. 7-9)
 * with a straight-through estimator: Q passes gradients unchanged inside the
 * first term, and its value is held fixed inside the other two (so they pull
 * A T and W T^{-T} toward their quantized values). Q is the MXFP4 quantizer of
 * this library (quantize, then decode).
 *   A          device, bf16 [M][d] calibration activations (M = N m rows)
 *   W          device, fp32 [o][d] layer weights
 *   workspace  device, 256-byte aligned, at least kq_calib_workspace_bytes();
 *              init fills it with A in fp32 and A W^T; step reuses it. Owned
 *              by the caller; no other allocation is made.
 * kq_calib_step (t >= 1 is Adam's step count; beta1, beta2 in [0, 1), eps, lr >= 0):
 *   theta, adam_m, adam_v  device fp32 [d/32][5][3], updated in place
 *   lambdas    device fp32 [2] = (lambda_A, lambda_W); with auto_lambda != 0 they
 *              are first set by Eq. 10 from this step's loss terms (call it so
 *              at the starting point; a term that is zero there gets weight 0)
 *   losses     device fp32 [3] = (L_out, L_A, L_W) at theta before the update
 *   grad_theta device fp32 [d/32][5][3] or NULL: dL/dtheta at theta
 * M, o, d > 0, d % 32 == 0, and M d, o d, M o below 2^31 (KQ_ERR_UNSUPPORTED).
 */
kq_status kq_calib_workspace_bytes(int64_t M, int64_t d, int64_t o, int64_t *bytes);
kq_status kq_calib_init(const uint16_t *A, int64_t M, int64_t d, const float *W, int64_t o, void *workspace,
                        int64_t workspace_bytes, kq_stream_t stream);
kq_status kq_calib_step(const float *W, int64_t M, int64_t d, int64_t o, float *theta, float *adam_m, float *adam_v,
                        int64_t t, float lr, float beta1, float beta2, float eps, float *lambdas, int auto_lambda,
                        float *losses, float *grad_theta, void *workspace, int64_t workspace_bytes,
                        kq_stream_t stream);

/*
 * Allocation-free calibration step, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): kq_calib_init followed by kq_calib_step in one call, on a
 * workspace the library holds in a device array of its own instead of a
 * caller-owned one. Results are those of kq_calib_init + kq_calib_step on the
 * same arguments (the same kernels in the same order). Each call redoes the
 * init half (A in fp32 and A W^T), so calls are independent of each other.
 *   A, W, theta ... grad_theta, stream   as kq_calib_init / kq_calib_step
 * Limit: kq_calib_workspace_bytes(M, d, o) must be at most 64 MiB
 * (KQ_ERR_UNSUPPORTED otherwise; M = 1024, d = o = 1152 takes 43.5 MiB).
 * Every call on one GPU uses that GPU's single array: calls that overlap on
 * one GPU (other streams or host threads) race and must be serialized by the
 * caller. No hipMalloc or other allocation is made; the first call on a device
 * looks up the array's address there (hipGetSymbolAddress).
 */
kq_status kq_calib_step_noalloc(const uint16_t *A, const float *W, int64_t M, int64_t d, int64_t o, float *theta,
                                float *adam_m, float *adam_v, int64_t t, float lr, float beta1, float beta2, float eps,
                                float *lambdas, int auto_lambda, float *losses, float *grad_theta,
                                kq_stream_t stream);

/* Human-readable name of a status code (static storage). */
const char *kq_status_string(kq_status s);

/* hipError_t of the last KQ_ERR_HIP returned on the calling host thread (0 if none). */
int kq_last_hip_error(void);

/*
 * Host-only: 2x2 factor entries from the paper's 15 parameters per block
 * (Sec. 3.2, Eq. 6): G = [[1,0],[c,1]] . [[a,b],[0,-1/a]] = [[a, b],[c a, c b - 1/a]].
 *   abc      host, fp64 [nblk][5][3] = (a, b, c) per factor; a != 0
 *   factors  host, fp32 [nblk][5][2][2] (the layout above)
 * Returns KQ_ERR_NULL for NULL pointers, KQ_ERR_SHAPE for nblk < 0 or a == 0.
 */
kq_status kq_factors_from_lu(const double *abc, int64_t nblk, float *factors);

#ifdef __cplusplus
}
#endif

#endif /* KQ_H */
