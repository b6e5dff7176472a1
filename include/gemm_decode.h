/*
 * gemm_decode.h -- C ABI of libgemm_decode.so: block-quantized weight x
 * activation products for LLM decode (batch-1 GEMV) and prefill (small-M /
 * M-token GEMM) on AMD Instinct MI355X (gfx950).
 *
 * Conventions for every entry point below
 * ---------------------------------------
 *  - Pointers named in a "device" argument are HIP device (or host-coherent)
 *    memory owned by the caller; the library never allocates, frees or keeps
 *    a pointer after returning. Inputs are read only; outputs are fully
 *    overwritten (never accumulated into).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls only enqueue work: results are valid once the caller has
 *    synchronised with `stream`.
 *  - Sizes are int64_t element counts. Every argument is validated on the
 *    host before any HIP call; on a validation failure nothing is launched
 *    and a negative status is returned, so every status except GD_EHIP can
 *    be produced on a machine without a GPU.
 *  - No entry point aborts, throws, or silently switches to another code
 *    path: a shape a kernel cannot run is an error.
 *  - gemm_decode_last_error() returns a thread-local description of the last
 *    non-zero status raised on the calling thread.
 *
 * Page citations name the page's title and the section on it:
 *   "browseml-gpu.js" (browseML on the GPU, exactly),
 *   "block_q8_matmul_nt.wgsl" (kopitiam-gpu),
 *   "BonsaiのWebGPUカーネルを読み解く" (habakan blog, on PrismML's Bonsai
 *    WebGPU demo),
 *   "web-xpu-ops" (package README),
 *   "roofline.html" (Decode roofline — your GPU).
 */
#ifndef GEMM_DECODE_H
#define GEMM_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status */
#define GD_OK       0
#define GD_EINVAL  (-1) /* null pointer, non-positive or overflowing size     */
#define GD_ESHAPE  (-2) /* a size is not a multiple of the format's block      */
#define GD_EALIGN  (-3) /* a pointer is not aligned as the layout requires     */
#define GD_EHIP    (-4) /* HIP reported an error (launch, configuration)        */
#define GD_ERANGE  (-5) /* a size exceeds a documented kernel limit            */

/* Short constant name of a status code ("GD_OK", "GD_EINVAL", ...). */
const char *gemm_decode_status_string(int status);
/* Thread-local text describing the last failure on this thread ("" if none). */
const char *gemm_decode_last_error(void);
/* ABI version of this header (incremented on incompatible changes). */
int gemm_decode_abi_version(void);
#define GEMM_DECODE_ABI_VERSION 4

/* ====================================================================
 * Q1_0 . q8_0  ("browseml-gpu.js": header comment "The arithmetic, as the
 * reference does it", Q1_DOT_WGSL, Q1_MM_WGSL, packQ1, packQ8)
 * ====================================================================
 * Wire formats (as the page defines them):
 *  - Q1_0 weight block, 18 bytes per 128 weights: f16 d0 little-endian,
 *    then 128 sign bits, element j in byte 2 + j/8, bit j%8; bit 1 means
 *    +d0, bit 0 means -d0. A row of K weights is K/128 consecutive blocks;
 *    rows follow each other ("AoS" weights).
 *  - q8_0 activation block, 34 bytes per 32 activations: f16 d1, then 32
 *    int8. Activation column c is K/32 consecutive blocks starting at byte
 *    c*(K/32)*34.
 *
 * Result (bit-exact, one correct bit pattern per output): for each row and
 * accumulation lane l = 0..7 over blocks i in order,
 *   s      = sum_{e=4l}^{4l+3} (bit(32k+e) ? q_e : -q_e)   (int8 negation
 *            wraps: -(-128) = -128), k = sub-block 0..3 (activation block 4i+k)
 *   ab_l   = d1_k*s for k = 0, then ab_l = ab_l + d1_k*s for k = 1..3
 *   acc_l  = fma(d0_i, ab_l, acc_l)       (acc_l starts at +0)
 *   y      = ((acc0+acc4)+(acc2+acc6)) + ((acc1+acc5)+(acc3+acc7)).
 * f16 scales are decoded exactly, subnormals included.
 *
 * Q1 planes (the library's resident weight layout, written once by
 * q1_repack and read by the GEMV; the page's packQ1 repacks for the same
 * reason). With R64 = rows rounded up to 64, nb = K/128 and nb8 = nb rounded
 * up to 8:
 *  - bits plane, R64*nb*16 bytes, 16-byte aligned: u32 index
 *    ((((r/64)*nb + i)*2 + h)*64 + r%64)*2 + m holds, for half h (lanes
 *    4h..4h+3) and word m (sub-blocks 2m, 2m+1) of block i of row r, the sign
 *    bits of elements 32k + 4l + j with l = 4h + jj (jj = 0..3),
 *    k = 2m + kk (kk = 0..1), j = 0..3, at bit (8*jj + 2 + 4*kk + j) mod 32.
 *    (Each 4-bit group, pre-shifted by 2, indexes a 16-entry table of 4-byte
 *    products; the two halves are read by two different waves.)
 *  - scale plane, R64*nb8*2 bytes, 16-byte aligned: u16 index
 *    ((r/64)*(nb8/8) + i/8)*512 + (r%64)*8 + i%8 holds the f16 bits of d0
 *    of block i of row r.
 *  - Padding rows (r >= rows) and padding blocks (i >= nb) are zero.
 * ==================================================================== */

/* Sizes in bytes of the two Q1 planes for a rows x K weight (host only, no
 * GPU needed). Errors: GD_EINVAL (null out pointer, rows < 1, K < 1,
 * overflow), GD_ESHAPE (K % 128 != 0). */
int q1_planes_bytes(int64_t rows, int64_t K, size_t *bits_bytes, size_t *scale_bytes);

/* One-time repack of AoS Q1_0 weights into the Q1 planes (integer byte
 * moves; "browseml-gpu.js", packQ1).
 *   w_aos       device, rows*(K/128)*18 bytes, 2-byte aligned.
 *   bits_plane  device, q1_planes_bytes(...).bits_bytes, 16-byte aligned.
 *   scale_plane device, q1_planes_bytes(...).scale_bytes, 16-byte aligned.
 * Every byte of both planes is written (padding with zeros). Errors:
 * GD_EINVAL, GD_ESHAPE (K % 128), GD_EALIGN, GD_EHIP. */
int q1_repack(const void *w_aos, int64_t rows, int64_t K,
              void *bits_plane, void *scale_plane, void *stream);

/* y = W . a for n_act q8_0 activation columns, bit-exact as above.
 *   bits_plane, scale_plane  device Q1 planes of a rows x K weight (q1_repack).
 *   a_q8   device, n_act*(K/32)*34 bytes of q8_0 blocks, 2-byte aligned.
 *   y      device f32 [n_act][rows] (column c at y + c*rows, as Q1_MM_WGSL's
 *          O[col*rows + row]), 4-byte aligned.
 * n_act = 1 is the batch-1 decode GEMV; n_act > 1 (the small-M product)
 * keeps every column's bits: one launch runs every column as its own GEMV
 * (each re-reads the weights, mostly from cache).
 * Limits: rows <= 2^31 - 64, n_act <= 65535. Errors: GD_EINVAL, GD_ESHAPE
 * (K % 128), GD_EALIGN, GD_ERANGE, GD_EHIP. */
int q1_q8_gemv(const void *bits_plane, const void *scale_plane, const void *a_q8,
               float *y, int64_t rows, int64_t K, int64_t n_act, void *stream);

/* One independent batch-1 problem of a grouped launch. */
typedef struct gd_q1_problem {
    const void *bits_plane;   /* device Q1 bits plane, 16-byte aligned     */
    const void *scale_plane;  /* device Q1 scale plane, 16-byte aligned    */
    const void *a_q8;         /* device q8_0 activation (one column)       */
    float *y;                 /* device f32 [its rows]                      */
    int64_t rows;             /* its rows, 1 .. the launch's rows; 0 (or a
                                 value outside that range) means the
                                 launch's rows. Planes are sized for it.   */
} gd_q1_problem;

/* `count` independent batch-1 Q1_0 . q8_0 GEMVs with a common K in one
 * launch, each with its own weights, row count, activation and output; the
 * same kernel body and the same bits as q1_q8_gemv with n_act = 1.
 *   problems  device array of `count` gd_q1_problem, 8-byte aligned. The
 *             pointers and row counts inside it are read by the kernel and
 *             cannot be validated by the host: they must satisfy
 *             q1_q8_gemv's rules for that problem's rows.
 *   rows      the largest row count of the problems (sets the grid).
 * Limits: 1 <= count <= 65535. Errors: GD_EINVAL, GD_ESHAPE, GD_EALIGN,
 * GD_ERANGE, GD_EHIP. */
int q1_q8_gemv_grouped(const gd_q1_problem *problems, int64_t count,
                       int64_t rows, int64_t K, void *stream);

/* ====================================================================
 * Sign-bit prefill GEMM  ("BonsaiのWebGPUカーネルを読み解く", figure on
 * PrismML's decode/prefill kernels: q1_bits holds the sign bits of 32
 * weights per u32, q1_scales one scale per 32 weights, bit 1 -> +1.0,
 * bit 0 -> -1.0; prefill is the compute-bound M-token case)
 * ====================================================================
 *   y[m][n] = sum_g scales[n][g] * sum_{j<32} x[m][32g+j] * (bit_j ? +1 : -1)
 *   x       device f32 [M][K] row-major, 16-byte aligned, finite. The
 *           product runs on fp16 matrix cores: each row of x is scaled, in
 *           each eighth of K (ceil(K/256) groups), by the power of two that
 *           brings its largest |x| there into [2^14, 2^15), each output's
 *           scales by the power of two that does the same for its largest
 *           |scale|, and both are split into a high and a low
 *           fp16 part (x = xh + xl, s = sh + sl, each within 2^-22 of its
 *           value while normal in fp16); a 32-weight group contributes
 *           xh*sh + xl*sh + xh*sl of its signed products, accumulated in
 *           f32 on the matrix cores per eighth of K; each eighth's sum is
 *           unscaled exactly and the eight are added in a fixed order.
 *           Error within 1e-5 of ||y||_inf (about 5e-7 on N(0,1)
 *           activations and |N(0,0.02)| scales at K = 4096).
 *   w_bits  device u32 [N][K/32], bit j of word g = weight 32g+j (LSB
 *           first), 4-byte aligned.
 *   w_scales device f32 [N][K/32], 4-byte aligned.
 *   y       device f32 [M][N], 4-byte aligned.
 *   workspace  device scratch of at least q1_sign_gemm_workspace_bytes(M,
 *           N, K) bytes, 16-byte aligned, owned by the caller. A first
 *           kernel writes the split activations and the weights in the
 *           matrix-core layout (see q1_sign_pack) into it for the second;
 *           calls that share it must be ordered on one stream. Its contents
 *           on entry do not matter and on return are unspecified.
 * Requires K % 32 == 0. Errors: GD_EINVAL, GD_ESHAPE, GD_EALIGN, GD_ERANGE
 * (M, N or K above 2^31 - 1, workspace too small), GD_EHIP. */
int q1_sign_gemm(const float *x, const uint32_t *w_bits, const float *w_scales,
                 float *y, int64_t M, int64_t N, int64_t K,
                 void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes q1_sign_gemm needs: 4*K per token (tokens padded to a
 * multiple of 16) plus 32 per padded token (an exponent per eighth of K),
 * plus 16 per output and pair of 32-weight groups (ceil(K/64) pairs), plus
 * 4 per output. Host only.
 * Errors: GD_EINVAL, GD_ESHAPE (K % 32 != 0), GD_ERANGE. */
int q1_sign_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t *bytes);

/* Bytes of the packed sign-bit weights written by q1_sign_pack:
 * 32 * N * ceil(K/64) + 4 * N. Host only. Errors: GD_EINVAL, GD_ESHAPE,
 * GD_ERANGE. */
int q1_sign_packed_bytes(int64_t N, int64_t K, size_t *bytes);

/* One-time repack of the page's sign words and scales (the layouts
 * q1_sign_gemm takes) for the calls below, in three sections (P = 16 * N *
 * ceil(K/64) bytes each for the first two):
 *   [0, P)      for the table kernels (q1_sign_gemv, q1_sign_gemm_lut4):
 *               for each output n and pair of 32-weight groups (g, g+1),
 *               g even, the u32x4 {bits[n][g], bits[n][g+1], scale[n][g],
 *               scale[n][g+1]} (scales as f32 bit patterns) at index
 *               (g/2)*N + n, a missing group g+1 = K/32 having bits 0 and
 *               scale 0, so the words of one group pair for consecutive
 *               outputs are contiguous;
 *   [P, 2P)     for the matrix-core GEMM: for each group g and output n the
 *               u32x2 {bits[n][g], sh | sl << 16} at index g*N + n, sh and
 *               sl the fp16 high and low parts of scale[n][g] * 2^c_n;
 *   [2P, 2P+4N) the int32 c_n per output: the exponent that puts the
 *               output's largest |scale| in [2^14, 2^15) (0 if all are 0).
 *   w_bits, w_scales  as for q1_sign_gemm, 4-byte aligned.
 *   w_packed          device, q1_sign_packed_bytes(N, K) bytes, 16-byte
 *                     aligned; written whole.
 * Errors: GD_EINVAL, GD_ESHAPE, GD_EALIGN, GD_ERANGE, GD_EHIP. */
int q1_sign_pack(const uint32_t *w_bits, const float *w_scales, int64_t N, int64_t K,
                 void *w_packed, void *stream);

/* q1_sign_gemm on weights packed once by q1_sign_pack (no per-call
 * regrouping launch); same numerics and bits as q1_sign_gemm. The workspace
 * holds only the split activations and row exponents: at least
 * 4*K*M16 + 32*M16 bytes (M16 = M rounded up to 16), so any size
 * q1_sign_gemm_workspace_bytes(M, N, K) returns is enough. x, w_packed and
 * workspace 16-byte aligned, y 4-byte. Errors: GD_EINVAL, GD_ESHAPE,
 * GD_EALIGN, GD_ERANGE, GD_EHIP. */
int q1_sign_gemm_packed(const float *x, const void *w_packed, float *y,
                        int64_t M, int64_t N, int64_t K,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Sign-bit decode GEMV (the page's decode kernel, one token at a time):
 * y[m][n] = sum_g scale[n][g] * sum_{j<32} s(n, 32g+j) x[m][32g+j] for each
 * of M activation rows, from packed weights. Each workgroup turns the row
 * into LDS tables of the signed sums of every 4 consecutive elements (16
 * per 4), so a nibble of signs costs one table read and one add; partial
 * sums round in f32 (within 1e-5 of ||y||_inf of the exact sum).
 *   x  device f32 [M][K], 16-byte aligned; y device f32 [M][N], 4-byte.
 * Requires K % 32 == 0, 1 <= M <= 65535. Every row reads the weights once
 * more: meant for a few tokens (use q1_sign_gemm(_packed) for prefill).
 * Errors: GD_EINVAL, GD_ESHAPE, GD_EALIGN, GD_ERANGE, GD_EHIP. */
int q1_sign_gemv(const float *x, const void *w_packed, float *y,
                 int64_t M, int64_t N, int64_t K, void *stream);

/* The page's LUT4 prefill GEMM (binary-lut4-matmul: 16 partial sums of
 * every 4 activations in workgroup memory, one read per nibble, reused over
 * a 16-token x 512-output tile), kept as the comparator of the matrix-core
 * GEMM: same y and contract as q1_sign_gemv, for any M. */
int q1_sign_gemm_lut4(const float *x, const void *w_packed, float *y,
                      int64_t M, int64_t N, int64_t K, void *stream);

/* ====================================================================
 * Block-scaled int8 matmul_nt  ("block_q8_matmul_nt.wgsl": PACKING,
 * ACCUMULATION ORDER, quant_at, main)
 * ====================================================================
 *   y[r][c] = sum_b scales[c][b] * sum_{t<32} x[r][32b+t] * q[c][32b+t]
 *   x       device f32 [m][k] row-major, 16-byte aligned.
 *   quants  device u32 [n][k/4]: element t of row c in byte t%4 of word
 *           c*k/4 + t/4 (little-endian), two's-complement int8; 16-byte
 *           aligned.
 *   scales  device f32 [n][k/32], 4-byte aligned.
 *   y       device f32 [m][n], 4-byte aligned.
 * Requires k % 32 == 0 (an error, where the page's kernel would silently
 * drop a tail) and k % 16 == 0 rows of quants on 16-byte boundaries (implied
 * by k % 32 == 0). x must be finite. Results agree with the page's order
 * within 1e-5 of ||y||_inf. For 2 <= m <= 16 and k <= 1024 the block
 * sub-totals run on fp16 matrix cores: each activation row is scaled by a
 * power of two that brings its largest |x| into [2^14, 2^15), split into
 * high and low fp16 parts, and the sub-total is scaled back exactly, so
 * rows of any finite magnitude keep ~22 bits. Limits: m <= 16 and
 * m*k <= 16384 (the activation rows are staged whole in LDS). Errors:
 * GD_EINVAL, GD_ESHAPE, GD_EALIGN, GD_ERANGE, GD_EHIP. */
int blockq8_matmul_nt(const float *x, const uint32_t *quants, const float *scales,
                      float *y, int64_t m, int64_t k, int64_t n, void *stream);

/* ====================================================================
 * Ternary bitplane GEMV  ("BonsaiのWebGPUカーネルを読み解く", section on
 * Bonsai: P bit set where w = +1, N bit set where w = -1, and
 * dot = 2(pc(P&X) - pc(N&X)) - pc(P) + pc(N) for a binary plane X)
 * ====================================================================
 * The int8 activation enters as its eight two's-complement bit planes B_b
 * (x = sum_{b<7} 2^b B_b - 128 B_7), so the integer dot is a weighted sum of
 * per-plane popcount identities and is exact.
 * ==================================================================== */

/* Bit planes of an int8 activation vector (or `count` vectors).
 *   x_q     device int8 [count][K], 16-byte aligned.
 *   planes  device u32 [count][8][K/32]: word m of plane b holds bit b of
 *           the two's-complement bytes x_q[32m .. 32m+31], element 32m+j at
 *           bit j. 16-byte aligned.
 * Requires K % 32 == 0, 1 <= count <= 65535. Errors: GD_EINVAL, GD_ESHAPE,
 * GD_EALIGN, GD_ERANGE, GD_EHIP. */
int ternary_act_bitplanes(const int8_t *x_q, int64_t count, int64_t K,
                          uint32_t *planes, void *stream);

/* dot[r] = sum_k w[r][k] * x[k] (exact int32) and y[r] = (float)dot[r] * s
 * with s = w_scale * x_scale rounded once to f32.
 *   w_pos, w_neg  device u32 [rows][K/32], bit j of word m = element 32m+j;
 *                 16-byte aligned. An element with both bits set counts as 0.
 *   x_planes      device u32 [8][K/32] from ternary_act_bitplanes, 16-byte
 *                 aligned.
 *   y             device f32 [rows]; dot_out device int32 [rows] or NULL.
 * Requires K % 32 == 0 and K <= 65536 (so |dot| <= 128*K < 2^24 and
 * f32(dot) is exact; the planes, 8*K/8 bytes, are staged whole in LDS). Errors: GD_EINVAL,
 * GD_ESHAPE, GD_EALIGN, GD_ERANGE, GD_EHIP. */
int ternary_gemv(const uint32_t *w_pos, const uint32_t *w_neg, float w_scale,
                 const uint32_t *x_planes, float x_scale, float *y, int32_t *dot_out,
                 int64_t rows, int64_t K, void *stream);

typedef struct gd_ternary_problem {
    const uint32_t *w_pos;     /* device u32 [rows][K/32]  */
    const uint32_t *w_neg;     /* device u32 [rows][K/32]  */
    const uint32_t *x_planes;  /* device u32 [8][K/32]     */
    float *y;                  /* device f32 [rows]        */
    int32_t *dot_out;          /* device int32 [rows] or NULL */
    float w_scale;
    float x_scale;             /* used when x_scale_dev is NULL */
    const float *x_scale_dev;  /* device f32 (e.g. from ternary_quantize_act) or NULL;
                                  when set, the activation scale is read from it */
} gd_ternary_problem;

/* `count` independent ternary GEMVs of one shape in one launch (one decode
 * step's projections of a given shape); same kernel body and bits as
 * ternary_gemv, the scale product w_scale * x_scale taken with the scale
 * read from x_scale_dev where that is set. `problems` is a device array (8-byte aligned) whose inner
 * pointers must satisfy ternary_gemv's rules. Limits: 1 <= count <= 65535.
 * Errors: GD_EINVAL, GD_ESHAPE, GD_EALIGN, GD_ERANGE, GD_EHIP. */
int ternary_gemv_grouped(const gd_ternary_problem *problems, int64_t count,
                         int64_t rows, int64_t K, void *stream);

/* ====================================================================
 * Activation quantization  ("web-xpu-ops", operator table: quantize, and
 * the reciprocal and rounding rows of its q4 format table, which state the
 * same convention)
 * ====================================================================
 * The step before each GEMV. Per group (a token for the ternary path, a
 * 32-element block for q8_0): absmax = max |x|; codes are Math.round of
 * x * (127/absmax), the reciprocal formed in f64, ties toward +infinity
 * (floor(v) + (v - floor(v) >= 0.5) in f64), clamped to [-127, 127]; the
 * scale is the f64 quotient absmax/127 rounded to f32. A group whose absmax
 * is 0 gets scale 0 and zero codes. Inputs must be finite (NaN or infinity
 * give unspecified codes). Codes and scales are bit-exact with this rule.
 * ==================================================================== */

/* f32 activations -> q8_0 blocks in the layout q1_q8_gemv reads
 * ("browseml-gpu.js", packQ8: 34 bytes, f16 d then 32 int8 codes). The
 * pages fix the block, not its quantizer: the rule above is applied to each
 * block of 32, and d is the f32 scale rounded to f16 (nearest even).
 *   x     device f32 [n][K], 16-byte aligned.
 *   a_q8  device, n * (K/32) * 34 bytes (column c at byte c * (K/32) * 34),
 *         2-byte aligned; written whole.
 * Requires K % 32 == 0, n >= 1, n * K/32 <= 2^34. Errors: GD_EINVAL,
 * GD_ESHAPE, GD_EALIGN, GD_ERANGE, GD_EHIP. */
int q8_0_quantize(const float *x, void *a_q8, int64_t n, int64_t K, void *stream);

/* f32 activations -> per-token int8 codes (the rule above over each token's
 * K values), written as the bit planes ternary_gemv reads, and the scales.
 *   x        device f32 [count][K], 16-byte aligned.
 *   planes   device u32 [count][8][K/32], the layout of
 *            ternary_act_bitplanes; 4-byte aligned (ternary_gemv itself
 *            needs 16).
 *   x_scale  device f32 [count] (for gd_ternary_problem.x_scale_dev).
 * Requires K % 32 == 0, 1 <= count <= 2^31 - 1, K <= 2^30. Errors:
 * GD_EINVAL, GD_ESHAPE, GD_EALIGN, GD_ERANGE, GD_EHIP. */
int ternary_quantize_act(const float *x, int64_t count, int64_t K, uint32_t *planes,
                         float *x_scale, void *stream);

/* ====================================================================
 * Split-K decode attention  ("BonsaiのWebGPUカーネルを読み解く", section on
 * split-K flash decode attention: per split a running maximum, denominator
 * and rescaled output; a merge that rescales every split to the global
 * maximum)
 * ====================================================================
 * One decode token: for query head h and its KV head kv = h / (n_heads /
 * n_kv_heads), s_j = scale * q[h] . k[kv][j] over positions j < kv_len, and
 * out[h] = sum_j exp(s_j - max s) v[kv][j] / sum_j exp(s_j - max s). The
 * pages leave the score scale to the caller (1/sqrt(head_dim) is usual).
 * f32 throughout; within 1e-5 of ||out||_inf of the f64 definition.
 * ==================================================================== */

/* Workspace bytes attn_decode_splitk needs: num_splits * n_heads *
 * (head_dim + 2) * 4, num_splits = 0 meaning the split count the call picks
 * for that shape. Host only. Errors as attn_decode_splitk's validation. */
int attn_decode_workspace_bytes(int64_t n_heads, int64_t n_kv_heads, int64_t head_dim,
                                int64_t kv_len, int64_t num_splits, size_t *bytes);

/*   q         device f32 [n_heads][head_dim], 16-byte aligned.
 *   k_cache,  device f32 [n_kv_heads][kv_stride][head_dim]: position j of KV
 *   v_cache   head kv at row kv * kv_stride + j; rows j < kv_len are read.
 *             16-byte aligned.
 *   out       device f32 [n_heads][head_dim], 4-byte aligned.
 *   num_splits  number of key ranges run in parallel (each ceil(kv_len /
 *             num_splits) keys, trailing splits may be empty); 0 picks about
 *             512 workgroups in all, at least 64 keys each.
 *   workspace device, attn_decode_workspace_bytes(...) bytes, 16-byte
 *             aligned: per split and head the running output, maximum and
 *             denominator, read by the merge launch of the same call.
 * Requires head_dim == 128, n_heads % n_kv_heads == 0 with n_heads /
 * n_kv_heads in {1, 2, 4, 8}, kv_len >= 1, kv_stride >= kv_len,
 * num_splits <= 65535. Errors: GD_EINVAL, GD_ESHAPE, GD_EALIGN, GD_ERANGE,
 * GD_EHIP. */
int attn_decode_splitk(const float *q, const float *k_cache, const float *v_cache, float *out,
                       int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, int64_t kv_len,
                       int64_t kv_stride, float scale, int64_t num_splits,
                       void *workspace, size_t workspace_bytes, void *stream);

/* attn_decode_splitk without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops or harnesses
 * that forbid hipMalloc). Same arguments, validation, kernels and results
 * as attn_decode_splitk; the split partials go to a scratch array inside the
 * library (GD_ATTN_NOALLOC_MAX_BYTES per device, held from the first call on
 * that device until the process ends). The call allocates nothing. Requires
 * num_splits * n_heads * (head_dim + 2) * 4 <= GD_ATTN_NOALLOC_MAX_BYTES
 * (num_splits = 0: the split count the call picks), else GD_ERANGE before
 * any launch. Calls on one device share its scratch: calls that overlap on
 * one device (several streams, several host threads) race; order them.
 * Errors: GD_EINVAL, GD_ESHAPE, GD_EALIGN, GD_ERANGE, GD_EHIP. */
#define GD_ATTN_NOALLOC_MAX_BYTES (4 * 1024 * 1024)
int attn_decode_splitk_noalloc(const float *q, const float *k_cache, const float *v_cache, float *out,
                               int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, int64_t kv_len,
                               int64_t kv_stride, float scale, int64_t num_splits, void *stream);

/* ====================================================================
 * Measurement kernels  ("roofline.html": the FILL kernel writes a non-zero,
 * incompressible pattern so reads reach real DRAM; the read kernel streams
 * 16-byte words through an XOR into a sink)
 * ==================================================================== */

/* Fill `bytes` (multiple of 16, 16-byte aligned) with a hash of the 16-byte
 * word index and `seed`. Errors: GD_EINVAL, GD_ESHAPE, GD_EALIGN, GD_EHIP. */
int gemm_decode_fill(void *buf, size_t bytes, uint32_t seed, void *stream);

/* Read `bytes` (multiple of 16, 16-byte aligned) `passes` times with
 * 16-byte loads, XOR-reducing into sink (device u32 [sink_words], written).
 * Errors: GD_EINVAL, GD_ESHAPE, GD_EALIGN, GD_ERANGE, GD_EHIP. */
int gemm_decode_stream_read(const void *buf, size_t bytes, int32_t passes,
                            uint32_t *sink, int64_t sink_words, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_DECODE_H */
