/*
 * mxq.h - C ABI of the MI355X (gfx950) microscaled-FP4 quantisation library.
 *
 * Every entry point takes plain pointers and sizes. Tensor pointers are device
 * pointers on the current HIP device; `stream` is a hipStream_t (NULL = the null
 * stream). Calls validate their arguments synchronously, enqueue kernels on
 * `stream` and return: results are valid once the stream has synchronised. The
 * caller owns and allocates every buffer; the library allocates no device memory
 * and keeps no global state. No C++ exception crosses this boundary.
 *
 * Layouts. Inputs are row-major [rows, cols] with a row stride `ldx` in elements
 * (ldx >= cols). Outputs are dense row-major:
 *   codes   uint8 [rows, cols/2]  two 4-bit codes per byte; element 2j in bits 0-3,
 *                                 element 2j+1 in bits 4-7
 *   scales  uint8 [rows, cols/bs] bs = 32 (MXFP4, E8M0 bytes) or 16 (NVFP4, E4M3 bytes)
 * Column-wise outputs quantise the transpose: codes [cols, rows/2], scales
 * [cols, rows/bs]; blocks run along rows, as a weight-gradient GEMM consumes them.
 *
 * Formats (OCP microscaling layouts):
 *   E2M1 element   s e1 e0 m: 0, 0.5, 1, 1.5, 2, 3, 4, 6 (and negatives)
 *   E8M0 scale     2^(byte - 127); 0xFF = NaN
 *   E4M3 (FP8)     OCP "fn": bias 7, max 448, 0x7F/0xFF = NaN
 *
 * Status codes: MXQ_OK on success; MXQ_EINVAL for a NULL pointer, an enum out of
 * range or a negative size; MXQ_ESHAPE for a dimension that is not a multiple of
 * the block size (no padding is ever applied), ldx < cols, or a tensor beyond the
 * size limits (2^40 elements, 2^30 columns); MXQ_EALIGN for a
 * pointer or row stride that breaks the stated alignment; MXQ_EUNSUPPORTED for a
 * combination not provided; MXQ_EHIP when a launch fails. rows == 0 is a no-op
 * that returns MXQ_OK. Data-dependent conditions (NaN, Inf, zeros, extreme
 * exponents) are never errors: they are encoded in the outputs as stated below.
 *
 * Sources. The operations follow the text of these pages:
 *  [HOPPER]  "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs",
 *            technical summary: section 1 (MXFP4 = 32-element blocks, E2M1;
 *            FP8 pipeline = E4M3 with 128-element blocks), section 2B (direct
 *            FP4 -> FP8 bit remap with hierarchical scale alignment), section 2C
 *            (fused, ragged, transposed-layout kernels); the Spanish summary,
 *            section 2 (kernels BF16ToFP4Row / FP4RowToFP8Row / FP4RowToFP8Col,
 *            subnormal handling, bitwise scale decoding).
 *  [MI355X]  "Pretraining large language models with MXFP4 on Native FP4
 *            Hardware": "Qu'est-ce que le MXFP4 ?" (shared E8M0 exponent = the
 *            block's maximum exponent, elements rounded to nearest) and
 *            "Expérience d'investigation" (Fprop/Dgrad/Wgrad, deterministic and
 *            random-sign Hadamard, stochastic rounding).
 *  [NVFP4]   "Pretraining Large Language Models with NVFP4", technical summary
 *            section 2A (16-element blocks, E4M3 block scale, fp32 tensor scale)
 *            and 2B (random Hadamard on Wgrad inputs, stochastic rounding).
 */
#ifndef MXQ_H_
#define MXQ_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MXQ_OK = 0,
  MXQ_EINVAL = 1,
  MXQ_ESHAPE = 2,
  MXQ_EALIGN = 3,
  MXQ_EUNSUPPORTED = 4,
  MXQ_EHIP = 5
} mxq_status;

typedef enum { MXQ_BF16 = 0, MXQ_F32 = 1 } mxq_dtype;
typedef enum { MXQ_MXFP4 = 0, MXQ_NVFP4 = 1, MXQ_NVFP4_2D = 2 } mxq_format;
typedef enum { MXQ_RNE = 0, MXQ_SR = 1, MXQ_SR16 = 2 } mxq_round;
typedef enum { MXQ_ROWWISE = 1, MXQ_COLWISE = 2, MXQ_BOTH = 3 } mxq_axis;

/*
 * mxq_quantize - block quantisation of a bf16/fp32 tensor to MXFP4 or NVFP4.
 *
 * MXFP4 ([HOPPER] section 1; [MI355X] "Qu'est-ce que le MXFP4 ?"): per block of 32
 *   E = clamp(floor(log2 max|x|) - 2, -127, 127), stored as the byte E + 127;
 *   code = sign(x) | E2M1 rounding of |x| / 2^E (nearest, ties to even, saturating
 *   at 6). A block holding NaN or +-Inf gets scale 0xFF and codes 0; an all-zero
 *   block gets scale 0 and sign-only codes.
 * NVFP4 ([NVFP4] section 2A): s_t = RN_fp32(A / 2688) with A the tensor's max |x|
 *   (*amax, or computed first when amax is NULL); per block of 16 s_b = E4M3 rounding (nearest
 *   even, saturating at 448) of the exact quotient max|x_block| / (6 s_t); code =
 *   sign | E2M1 rounding of the exact quotient |x| / (s_b s_t). s_t == 0 gives
 *   scale bytes 0 and sign-only codes, a block with s_b == 0 sign-only codes, a
 *   NaN/Inf amax (or a NaN/Inf block) scale bytes 0x7F and codes 0.
 * NVFP4_2D ([NVFP4] section 2B, 16x16 blocks for weights): as NVFP4 but one block
 *   scale per 16x16 tile (its max |x| over 256 elements), written in the NVFP4
 *   layout with the tile's byte repeated on its 16 rows (row-wise) or columns
 *   (column-wise): the column-wise output is exactly the transpose of the row-wise
 *   one, so one quantisation serves W and W^T, and mxq_dequantize reads it as
 *   NVFP4. rows % 16 == 0 and cols % 16 == 0 for any axis; round to nearest even
 *   only (MXQ_SR and MXQ_SR16 return MXQ_EUNSUPPORTED).
 * Stochastic rounding (rnd == MXQ_SR; [NVFP4] section 2B, gradients): element n
 *   (n = sr_offset + its row-major index in the tensor quantised; for column-wise
 *   outputs the index in the transpose) draws the 32-bit word n mod 4 of
 *   Philox4x32-10(counter = (n/4 lo, n/4 hi, 0, 0), key = (seed lo, seed hi)); with
 *   r its top 16 bits, lo the grid value at or below y = |x|/scale and step the gap
 *   to the next, y rounds up iff y > lo + step (r + 1/2) / 2^16; y >= 6 gives 6.
 * Stochastic rounding, halves stream (rnd == MXQ_SR16, opt-in; a cheaper random
 *   stream defined by this library, not by the pages): the same rule with r the
 *   16-bit half (n mod 2), low half for even n, of word (n mod 8) / 2 of
 *   Philox4x32-10(counter = (n/8 lo, n/8 hi, 0, 0), same key), i.e. half n mod 2 of
 *   word n / 2 of the default stream: one generator call serves eight elements.
 *   Results differ from MXQ_SR. sr_offset % 8 == 0 (else MXQ_EALIGN).
 *
 * x            device, bf16 or fp32 [rows, ldx]; 16-byte aligned, ldx*sizeof a
 *              multiple of 16 bytes.
 * axis         MXQ_ROWWISE writes codes_row/scales_row, MXQ_COLWISE codes_col/
 *              scales_col, MXQ_BOTH both from a single read of x. Unused output
 *              pointers may be NULL.
 * amax         NVFP4 / NVFP4_2D: device fp32[1] holding the tensor amax (read only), or
 *              NULL: then the call first computes the amax (as mxq_amax) into the
 *              tensor_scale slot, turns it into s_t there and quantises from it, all
 *              on `stream` (no allocation; tensor_scale must then be non-NULL, else
 *              MXQ_EINVAL). Sharded callers pass the all-reduced amax instead.
 * tensor_scale NVFP4 / NVFP4_2D: device fp32[1] receiving s_t (may be NULL when amax
 *              is given). amax and tensor_scale are 4-byte aligned.
 * Shapes: cols % bs == 0 for row-wise; rows % bs == 0 for column-wise outputs.
 */
mxq_status mxq_quantize(const void* x, mxq_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                        mxq_format fmt, mxq_axis axis, mxq_round rnd, uint64_t sr_seed,
                        uint64_t sr_offset, uint8_t* codes_row, uint8_t* scales_row,
                        uint8_t* codes_col, uint8_t* scales_col, const float* amax,
                        float* tensor_scale, void* stream);

/*
 * mxq_dequantize - codes + scales back to bf16 / fp32 ([HOPPER] Spanish summary
 * section 2: dequantisation with bitwise scale decoding).
 * Each output is the exact value v(code) * scale rounded once to the output type
 * (round to nearest even, overflow to Inf; MXFP4 values with scale bytes <= 252
 * are always exact). MXFP4: scale = 2^(byte - 127). NVFP4: scale = E4M3(byte) *
 * (*tensor_scale). A NaN scale gives the quiet NaN 0x7FC0 / 0x7FC00000.
 * codes [rows, cols/2], scales [rows, cols/bs], y [rows, cols] of out_dt, dense.
 * tensor_scale: device fp32[1], NVFP4 only. cols % bs == 0. NVFP4_2D outputs are
 * read as NVFP4 (the layout is the same).
 */
mxq_status mxq_dequantize(const uint8_t* codes, const uint8_t* scales, mxq_format fmt,
                          int64_t rows, int64_t cols, const float* tensor_scale, void* y,
                          mxq_dtype out_dt, void* stream);

/*
 * mxq_fp8_to_mxfp4 - direct FP8 -> MXFP4 quantisation with no bf16 intermediate
 * ([HOPPER] abstract and section 2B). Input: E4M3 q8 [rows, cols] with one fp32
 * scale per 1x128 group, s128 [rows, cols/128]; a scale is read through its
 * exponent field only (2^(field - 127); a power of two is used as is; field 255
 * makes the group NaN). Output: the MXFP4 quantisation (as mxq_quantize) of the
 * exact values e4m3(q) * scale: codes [rows, cols/2], e8m0 [rows, cols/32].
 * cols % 128 == 0. Rows are independent, so ragged per-expert segments are
 * quantised by one call over their concatenation or by one call per segment with
 * identical results.
 */
mxq_status mxq_fp8_to_mxfp4(const uint8_t* q8, const float* s128, int64_t rows, int64_t cols,
                            uint8_t* codes, uint8_t* e8m0, void* stream);

/*
 * mxq_mxfp4_to_fp8 - MXFP4 -> FP8 E4M3 with one scale per 1x128 group
 * ([HOPPER] section 2B; Spanish summary, FP4RowToFP8Row and subnormal handling).
 * Per group of four 32-blocks with exponents E_0..E_3: S = max E_j; the fp32
 * output scale is 2^(S - 127) (byte 0 gives the fp32 subnormal 2^-127); every
 * element becomes the E4M3 value nearest to v(code) * 2^(E_j - S) (ties to even,
 * subnormals materialised, sign and -0 kept). Exact whenever the exponents of the
 * blocks with nonzero codes lie within 8 of each other. A group with a 0xFF
 * exponent gives scale NaN (0x7FC00000) and codes 0x7F.
 * codes [rows, cols/2], e8m0 [rows, cols/32] -> q8 [rows, cols], s128 [rows, cols/128].
 * cols % 128 == 0.
 */
mxq_status mxq_mxfp4_to_fp8(const uint8_t* codes, const uint8_t* e8m0, int64_t rows, int64_t cols,
                            uint8_t* q8, float* s128, void* stream);

/*
 * mxq_fp4_row_to_fp8_col - MXFP4 rows -> FP8 columns in one pass (dequantise,
 * transpose, requantise) for the weight gradient of MoE experts ([HOPPER] section
 * 2C: fused kernel, ragged per-expert token counts through precomputed offsets, no
 * padding; Spanish summary, FP4RowToFP8Col).
 * codes [rows, cols/2] + e8m0 [rows, cols/32]: row-wise MXFP4 of X whose rows are
 * tokens, expert e owning rows [offsets[e], offsets[e+1]).
 * q8_col [cols, ld_q8]: E4M3 of X^T; row c holds column c of X at bytes
 * [0, rows) (the experts' segments side by side); bytes [rows, ld_q8) are not
 * written.
 * s_col [cols, ld_s] fp32: per row c, one scale per 128-token group; expert e's
 * groups start at index sum_{e' < e} ceil(n_e' / 128), the last group of an expert
 * holds its remaining n_e mod 128 tokens. Entries past the last group are not
 * written. Scale rule (not fixed by the pages): s = 2^k, k the smallest integer
 * with max|x| / 2^k <= 448 (k = 0 for an all-zero group); codes are the E4M3
 * values nearest to x / s (ties to even, subnormals kept, -0 kept). A group that
 * meets an E8M0 0xFF block gets scale NaN (0x7FC00000) and codes 0x7F.
 * offsets: device int64 [n_experts + 1], offsets[0] = 0, nondecreasing,
 * offsets[n_experts] = rows. They are read on the device; values outside [0, rows]
 * are clamped, so malformed offsets give unspecified output but no access outside
 * the buffers.
 * Requirements: cols % 32 == 0, rows < 2^31, 1 <= n_experts <= 4096,
 * ld_q8 >= rows with ld_q8 % 16 == 0, ld_s >= (rows + 127 * n_experts) / 128
 * (integer division: enough for any split of the rows). codes and q8_col 16-byte
 * aligned, s_col 4-byte, offsets 8-byte.
 */
mxq_status mxq_fp4_row_to_fp8_col(const uint8_t* codes, const uint8_t* e8m0, int64_t rows, int64_t cols,
                                  const int64_t* offsets, int64_t n_experts, uint8_t* q8_col,
                                  int64_t ld_q8, float* s_col, int64_t ld_s, void* stream);

/*
 * mxq_rht_quantize - 16-point random-sign Hadamard transform fused ahead of
 * quantisation ([MI355X] "Expérience d'investigation": deterministic H16 and
 * random-sign Hadamard; [NVFP4] section 2B: random Hadamard on Wgrad inputs).
 * Every aligned 16-element chunk along the block axis (columns for row-wise
 * outputs, rows for column-wise outputs) is replaced by y = (1/4) H16 (s * x),
 * H16 the Sylvester matrix H[i][j] = (-1)^popcount(i & j), s_i = -1 where bit i of
 * the sign mask mxq_rht_signs(rht_seed) is set (one sign vector per tensor, drawn
 * from the seed). y is computed in fp32 (butterfly stages 1, 2, 4, 8, then the
 * exact scaling by 1/4) and quantised without an intermediate bf16 rounding.
 * Arguments otherwise as mxq_quantize; rows % 32 (MXFP4) or % 16 (NVFP4) == 0 when
 * a column-wise output is requested.
 * NVFP4 (the pages' wgrad recipe): the tensor scale belongs to the transformed
 * tensor, so amax is the amax of y along the requested axis (mxq_rht_amax), or NULL
 * to have it computed first into the tensor_scale slot (as mxq_quantize does); the
 * row- and column-wise transforms have different amaxes, so axis must be
 * MXQ_ROWWISE or MXQ_COLWISE (MXQ_BOTH returns MXQ_EUNSUPPORTED). tensor_scale
 * receives s_t of y.
 */
mxq_status mxq_rht_quantize(const void* x, mxq_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                            mxq_format fmt, mxq_axis axis, uint64_t rht_seed, mxq_round rnd,
                            uint64_t sr_seed, uint64_t sr_offset, uint8_t* codes_row,
                            uint8_t* scales_row, uint8_t* codes_col, uint8_t* scales_col,
                            const float* amax, float* tensor_scale, void* stream);

/*
 * mxq_rht_quantize_mask - mxq_rht_quantize with the 16-bit sign mask given
 * directly instead of its seed: sign_mask 0 is the deterministic H16 transform of
 * [MI355X] "Expérience d'investigation"; mxq_rht_quantize(seed) equals this call
 * with sign_mask = mxq_rht_signs(seed).
 */
mxq_status mxq_rht_quantize_mask(const void* x, mxq_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                                 mxq_format fmt, mxq_axis axis, uint16_t sign_mask, mxq_round rnd,
                                 uint64_t sr_seed, uint64_t sr_offset, uint8_t* codes_row,
                                 uint8_t* scales_row, uint8_t* codes_col, uint8_t* scales_col,
                                 const float* amax, float* tensor_scale, void* stream);

/*
 * mxq_rht_apply - the transform alone: y = (1/4) H16 (s * x) on every aligned
 * 16-chunk of each row (s from sign_mask, e.g. mxq_rht_signs(rht_seed)), written as
 * fp32 [rows, cols] (dense). cols % 16 == 0.
 */
mxq_status mxq_rht_apply(const void* x, mxq_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                         uint16_t sign_mask, float* y, void* stream);

/*
 * mxq_rht_amax - the tensor amax of the transformed tensor, max |y| with
 * y = (1/4) H16 (s * x) taken along the rows (axis MXQ_ROWWISE, cols % 16 == 0) or
 * along the columns (MXQ_COLWISE, rows % 16 == 0, cols % 8 == 0), computed as
 * mxq_rht_quantize computes y (fp32 butterfly; s from sign_mask, e.g.
 * mxq_rht_signs(rht_seed)). This is the amax NVFP4 with the Hadamard transform
 * takes ([NVFP4] section 2B). Writes fp32 amax_out[0] (device); NaN/Inf propagate
 * as in mxq_amax; rows == 0 writes 0. MXQ_BOTH: MXQ_EINVAL.
 */
mxq_status mxq_rht_amax(const void* x, mxq_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                        mxq_axis axis, uint16_t sign_mask, float* amax_out, void* stream);

/*
 * mxq_amax - the tensor amax max|x| that NVFP4's tensor scale needs ([NVFP4]
 * section 2A). Writes fp32 amax_out[0] (device); a NaN or Inf anywhere gives a
 * non-finite value (NaN wins over Inf). rows == 0 writes 0.
 */
mxq_status mxq_amax(const void* x, mxq_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                    float* amax_out, void* stream);

/* Host helper: the Hadamard sign mask of a seed (bit i set: s_i = -1), bits 0..15
 * of word 0 of Philox4x32-10(key = (seed lo, seed hi), counter = 0). The pages ask
 * for one random sign vector per tensor but fix no generator; this map is the
 * library's definition ([MI355X] "Expérience d'investigation"). */
uint16_t mxq_rht_signs(uint64_t rht_seed);

/* Host helper: a static, human-readable name for a status code. */
const char* mxq_status_string(mxq_status s);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H_ */
