/*
 * oracle.c -- the CPU oracle for the block-quantized weight x activation
 * products. TEST INFRASTRUCTURE ONLY: it is loaded by tests/, by
 * __graft_entry__.smoke() and by bench.py's cpu_baseline leg, and by nothing
 * else. It shares no source, header, table or helper with the HIP library
 * (gemm_decode_amd/csrc); the two meet only on input bytes.
 *
 * Plain, slow, obviously correct: every function is a direct loop nest in the
 * order the pages state, with no blocking, fusion or reordering. Compiled with
 * -O2 -ffp-contract=off -fno-fast-math and the default x86-64 SSE rounding
 * (round to nearest even, no flush-to-zero), so every float operation written
 * here is exactly one IEEE operation. Threads (OpenMP) only split independent
 * outputs; each output's arithmetic is the same sequence on any thread count.
 *
 * Sources (page title, then section):
 *   [P1] "browseml-gpu.js" (browseML on the GPU, exactly): header comment
 *        "The arithmetic, as the reference does it", Q1_DOT_WGSL, Q1_MM_WGSL,
 *        packQ1, packQ8.
 *   [P2] "block_q8_matmul_nt.wgsl" (kopitiam-gpu): PACKING, ACCUMULATION
 *        ORDER, quant_at, main.
 *   [P3] "BonsaiのWebGPUカーネルを読み解く" (habakan blog): the ternary
 *        popcount identity in the section on Bonsai; the figure on PrismML's
 *        decode/prefill kernels (q1_bits / q1_scales, q1_signs4_unit).
 *   [P4] "web-xpu-ops": "The reference is the point" (f64 reference).
 *
 * Parity pins live in tests/test_oracle_*.py; every function below is pinned
 * by at least one of them (closed forms, integer-exact special cases,
 * brute force in f64/int64 via numpy, invariants).
 */

#include <math.h>
#include <stdint.h>
#include <string.h>
#include <omp.h>

#define QK1 128
#define QK8 32
#define Q1_BYTES 18
#define Q8_BYTES 34

int gdo_max_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------
 * f16 -> f32, exactly. [P1] decodes f16 scales with integer operations,
 * subnormals included: value = (-1)^s * m * 2^-24 for exponent field 0,
 * (-1)^s * (1024 + m) * 2^(e - 25) for 1 <= e <= 30, and Inf/NaN for e = 31
 * (NaN keeps the mantissa in the top of the f32 mantissa). Every f16 value is
 * exactly representable in f32 and ldexp of a small integer is exact.
 * ------------------------------------------------------------------------ */
float gdo_f16_to_f32(uint16_t h)
{
    uint32_t s = (h >> 15) & 1u, e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
    float v;
    if (e == 31u) {
        uint32_t bits = (s << 31) | 0x7f800000u | (m << 13);
        memcpy(&v, &bits, 4);
        return v;
    }
    if (e == 0u)
        v = ldexpf((float)m, -24);
    else
        v = ldexpf((float)(1024u + m), (int)e - 25);
    return s ? -v : v;
}

/* The negation [P1] applies to a quant whose sign bit is 0 is an int8
 * negation, which wraps: -128 has no positive counterpart in int8 and stays
 * -128 (Q1_DOT_WGSL, the comment on the sign select). */
static int32_t neg_i8_wrapping(int32_t q)
{
    return q == -128 ? -128 : -q;
}

/* The signed, wrapped quant the method adds for one element: q itself when
 * the element's sign bit is 1, its int8 negation when it is 0. */
static int32_t signed_quant(int bit, int8_t q)
{
    return bit ? (int32_t)q : neg_i8_wrapping(q);
}

/* f16 scale stored little-endian at p. */
static float scale_at(const uint8_t *p)
{
    return gdo_f16_to_f32((uint16_t)(p[0] | (p[1] << 8)));
}

/* ------------------------------------------------------------------------
 * Q1_0 . q8_0, form F1: from the array-of-structs bytes of both operands.
 *
 * [P1] header comment: per 128 weights a f16 d0 and 128 sign bits; per 32
 * activations a f16 d1 and 32 int8. For block i and accumulation lane l=0..7:
 *   s      = sum over e=4l..4l+3 of (bit(32k+e) ? q_e : neg_i8_wrapping(q_e))
 *   ab[l]  = d1*s            (k = 0)     -- exact in f32 (11 + 10 bits)
 *   ab[l]  = ab[l] + d1*s    (k = 1..3)  -- one rounding per add
 *   acc[l] = fma(d0, ab[l], acc[l])      -- correctly rounded fused op
 * and finally ((a0+a4)+(a2+a6)) + ((a1+a5)+(a3+a7)).
 * Activation column c's block b is at a + (c*(K/32) + b)*34; output is
 * y[c*rows + r] (Q1_MM_WGSL's O[col*rows + row]).
 * ------------------------------------------------------------------------ */
void gdo_q1_q8_gemv_aos(const uint8_t *w, const uint8_t *a, float *y,
                        int64_t rows, int64_t K, int64_t n_act, int nthreads)
{
    const int64_t nb = K / QK1;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static) collapse(2)
    for (int64_t c = 0; c < n_act; c++) {
        for (int64_t r = 0; r < rows; r++) {
            const uint8_t *act = a + c * (K / QK8) * Q8_BYTES;   /* column c */
            const uint8_t *wrow = w + r * nb * Q1_BYTES;          /* row r */
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int64_t i = 0; i < nb; i++) {
                const uint8_t *blk = wrow + i * Q1_BYTES;
                /* The block's integer sums first (exact in int32): s[k][l]
                 * over the four elements 4l..4l+3 of sub-block k, where
                 * element t of sub-block k is weight 32k + t of the block,
                 * whose sign bit sits at bit (32k+t)%8 of byte 2+(32k+t)/8. */
                int32_t s[4][8];
                float d1[4];
                memset(s, 0, sizeof s);
                for (int k = 0; k < 4; k++) {
                    const uint8_t *ablk = act + (4 * i + k) * Q8_BYTES;
                    d1[k] = scale_at(ablk);
                    for (int t = 0; t < 32; t++) {
                        const int j = 32 * k + t;
                        const int bit = (blk[2 + j / 8] >> (j % 8)) & 1;
                        s[k][t / 4] += signed_quant(bit, (int8_t)ablk[2 + t]);
                    }
                }
                /* Then the float chain of each lane in the stated order:
                 * ab = d1_0*s_0, + d1_1*s_1, + d1_2*s_2, + d1_3*s_3 (each
                 * product exact, each add rounded), and one fused step. */
                const float d0 = scale_at(blk);
                for (int l = 0; l < 8; l++) {
                    float ab = d1[0] * (float)s[0][l];
                    for (int k = 1; k < 4; k++) ab = ab + d1[k] * (float)s[k][l];
                    acc[l] = fmaf(d0, ab, acc[l]);
                }
            }
            y[c * rows + r] = ((acc[0] + acc[4]) + (acc[2] + acc[6])) +
                              ((acc[1] + acc[5]) + (acc[3] + acc[7]));
        }
    }
}

/* ------------------------------------------------------------------------
 * [P1] packQ1: per weight block its scale as f32 (exact) and its 128 bits as
 * four little-endian u32 taken from bytes 2+4k..5+4k.
 * ------------------------------------------------------------------------ */
void gdo_pack_q1_p1(const uint8_t *w, int64_t rows, int64_t K, float *d, uint32_t *b)
{
    const int64_t nb = K / QK1;
    for (int64_t i = 0; i < rows * nb; i++) {
        const uint8_t *o = w + i * Q1_BYTES;
        d[i] = gdo_f16_to_f32((uint16_t)(o[0] | (o[1] << 8)));
        for (int k = 0; k < 4; k++) {
            const uint8_t *p = o + 2 + 4 * k;
            b[i * 4 + k] = (uint32_t)p[0] | ((uint32_t)p[1] << 8) |
                           ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
        }
    }
}

/* [P1] packQ8: per activation block its scale as f32 and its quants four to
 * a little-endian u32; column c's block b at index c*(K/32) + b. */
void gdo_pack_q8_p1(const uint8_t *a, int64_t n_act, int64_t K, float *d, uint32_t *q)
{
    const int64_t nb8 = K / QK8;
    for (int64_t c = 0; c < n_act; c++) {
        for (int64_t b = 0; b < nb8; b++) {
            const uint8_t *o = a + (c * nb8 + b) * Q8_BYTES;
            d[c * nb8 + b] = gdo_f16_to_f32((uint16_t)(o[0] | (o[1] << 8)));
            for (int w = 0; w < 8; w++) {
                const uint8_t *p = o + 2 + 4 * w;
                q[(c * nb8 + b) * 8 + w] = (uint32_t)p[0] | ((uint32_t)p[1] << 8) |
                                           ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
            }
        }
    }
}

/* ------------------------------------------------------------------------
 * Q1_0 . q8_0, form F2: the same arithmetic on [P1]'s packed layouts, one
 * chain per (row, lane l) as Q1_MM_WGSL runs it: lane l reads the nibble
 * (word_k >> 4l) & 0xf and the l-th quant word of each activation block;
 * the eight chains are then added in the fixed tree. Must equal F1 bit for
 * bit, which pins the packing and the lane <-> element mapping.
 * ------------------------------------------------------------------------ */
void gdo_q1_q8_gemv_p1packed(const float *wd, const uint32_t *wb,
                             const float *ad, const uint32_t *aq, float *y,
                             int64_t rows, int64_t K, int64_t n_act, int nthreads)
{
    const int64_t nb = K / QK1;
    const int64_t nb8 = K / QK8;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static) collapse(2)
    for (int64_t c = 0; c < n_act; c++) {
        for (int64_t r = 0; r < rows; r++) {
            const float *act_d = ad + c * nb8;              /* column c's block scales */
            const uint32_t *act_q = aq + c * nb8 * 8;       /* its quant words, 8 per block */
            float lane_acc[8];
            for (int l = 0; l < 8; l++) {
                float acc = 0.f;
                for (int64_t i = 0; i < nb; i++) {
                    const uint32_t *signs = wb + (r * nb + i) * 4;   /* packQ1: word k = sub-block k */
                    float prod[4];
                    for (int k = 0; k < 4; k++) {
                        const uint32_t nib = (signs[k] >> (4 * l)) & 0xfu;   /* lane l's four signs */
                        const uint32_t quad = act_q[(4 * i + k) * 8 + l];    /* lane l's four quants */
                        int32_t s = 0;
                        for (int e = 0; e < 4; e++)
                            s += signed_quant((int)((nib >> e) & 1u), (int8_t)(uint8_t)(quad >> (8 * e)));
                        prod[k] = act_d[4 * i + k] * (float)s;
                    }
                    const float ab = ((prod[0] + prod[1]) + prod[2]) + prod[3];
                    acc = fmaf(wd[r * nb + i], ab, acc);
                }
                lane_acc[l] = acc;
            }
            y[c * rows + r] = ((lane_acc[0] + lane_acc[4]) + (lane_acc[2] + lane_acc[6])) +
                              ((lane_acc[1] + lane_acc[5]) + (lane_acc[3] + lane_acc[7]));
        }
    }
}

/* ------------------------------------------------------------------------
 * Sign-bit GEMM y = x @ w^T, plain definition in f64 ([P4], "The reference is
 * the point": accumulate in f64). [P3]'s packed format: bit j of u32
 * bits[n][g] is weight 32g+j of row n, bit 1 -> +1, bit 0 -> -1, and
 * scales[n][g] multiplies the 32 weights of group g:
 *   y[m][n] = sum_g scales[n][g] * sum_j x[m][32g+j] * sign(n, 32g+j),
 * rounded to f32 once.
 * ------------------------------------------------------------------------ */
void gdo_sign_gemm_f64(const float *x, const uint32_t *bits, const float *scales,
                       float *y, int64_t M, int64_t N, int64_t K, int nthreads)
{
    const int64_t G = K / 32;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static) collapse(2)
    for (int64_t m = 0; m < M; m++) {
        for (int64_t n = 0; n < N; n++) {
            double acc = 0.0;
            for (int64_t g = 0; g < G; g++) {
                uint32_t word = bits[n * G + g];
                double sub = 0.0;
                for (int j = 0; j < 32; j++) {
                    double xv = (double)x[m * K + 32 * g + j];
                    sub += ((word >> j) & 1u) ? xv : -xv;
                }
                acc += (double)scales[n * G + g] * sub;
            }
            y[m * N + n] = (float)acc;
        }
    }
}

/* The same product with f32 arithmetic in group order (sub-total of the 32
 * signed activations in sequence, then acc = acc + scale*sub): one of the
 * orders the page's fragments allow, kept to size the tolerance. */
void gdo_sign_gemm_f32(const float *x, const uint32_t *bits, const float *scales,
                       float *y, int64_t M, int64_t N, int64_t K, int nthreads)
{
    const int64_t G = K / 32;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static) collapse(2)
    for (int64_t m = 0; m < M; m++) {
        for (int64_t n = 0; n < N; n++) {
            float acc = 0.f;
            for (int64_t g = 0; g < G; g++) {
                uint32_t word = bits[n * G + g];
                float sub = 0.f;
                for (int j = 0; j < 32; j++) {
                    float xv = x[m * K + 32 * g + j];
                    sub = sub + (((word >> j) & 1u) ? xv : -xv);
                }
                float t = scales[n * G + g] * sub;
                acc = acc + t;
            }
            y[m * N + n] = acc;
        }
    }
}

/* ------------------------------------------------------------------------
 * Block-Q8 matmul_nt y = x @ w^T, [P2] main in its stated order, in f32 with
 * every product and add rounded separately (the reading recorded for the
 * unstated contraction): for each (row, col) acc = 0; per block b of 32,
 * block_sum = 0; block_sum = block_sum + x*quant for t = 0..31 in order;
 * acc = acc + scales[col][b]*block_sum. quant_at: byte t%4 of word t/4,
 * sign-extended ([P2], PACKING).
 * ------------------------------------------------------------------------ */
static float quant_at(const uint32_t *quants, int64_t index)
{
    uint32_t word = quants[index / 4];
    uint32_t byte = (word >> ((index % 4) * 8)) & 0xffu;
    return (float)(int32_t)(int8_t)(uint8_t)byte;
}

void gdo_blockq8_f32(const float *x, const uint32_t *quants, const float *scales,
                     float *y, int64_t m, int64_t k, int64_t n, int nthreads)
{
    const int64_t bpr = k / 32;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static) collapse(2)
    for (int64_t row = 0; row < m; row++) {
        for (int64_t col = 0; col < n; col++) {
            float acc = 0.f;
            for (int64_t b = 0; b < bpr; b++) {
                float block_sum = 0.f;
                for (int t = 0; t < 32; t++) {
                    float p = x[row * k + b * 32 + t] * quant_at(quants, col * k + b * 32 + t);
                    block_sum = block_sum + p;
                }
                float sb = scales[col * bpr + b] * block_sum;
                acc = acc + sb;
            }
            y[row * n + col] = acc;
        }
    }
}

/* ------------------------------------------------------------------------
 * Ternary bitplane GEMV ([P3], section on Bonsai). Weights w in {-1,0,+1} as
 * P (w=+1) and N (w=-1) planes, u32 [rows][K/32], element 32m+j at bit j.
 *
 * T1: the direct integer sum dot = sum_k w_k * x_k (int64), brute force.
 *
 * T2: the page's identity, dot = 2(pc(P&X) - pc(N&X)) - pc(P) + pc(N), for a
 * binary plane X. For int8 x it is applied to the eight bit planes X_b of the
 * offset-binary code u = x + 128 (u = sum_b 2^b X_b): each plane gives
 * D_b = sum_k w_k (2 X_bk - 1), so sum_b 2^b D_b = sum_k w_k (2u_k - 255)
 * = 2 dot + pc(P) - pc(N), i.e. dot = (sum_b 2^b D_b - pc(P) + pc(N)) / 2.
 * The output is y = (float)dot * s with s = w_scale * x_scale rounded once.
 * ------------------------------------------------------------------------ */
void gdo_ternary_dot_direct(const uint32_t *P, const uint32_t *N, const int8_t *x,
                            int64_t *dot, int64_t rows, int64_t K)
{
    const int64_t W = K / 32;
    for (int64_t r = 0; r < rows; r++) {
        int64_t acc = 0;
        for (int64_t kk = 0; kk < K; kk++) {
            int p = (P[r * W + kk / 32] >> (kk % 32)) & 1;
            int q = (N[r * W + kk / 32] >> (kk % 32)) & 1;
            int w = p - q;
            acc += (int64_t)w * (int64_t)x[kk];
        }
        dot[r] = acc;
    }
}

void gdo_ternary_gemv(const uint32_t *P, const uint32_t *N, float w_scale,
                      const int8_t *x, float x_scale, float *y, int32_t *dot32,
                      int64_t rows, int64_t K, int nthreads)
{
    const int64_t W = K / 32;
    if (nthreads < 1) nthreads = 1;
    const float s = w_scale * x_scale;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        int64_t sum = 0;       /* sum_b 2^b D_b */
        int64_t pcP = 0, pcN = 0;
        for (int64_t m = 0; m < W; m++) {
            uint32_t p = P[r * W + m], n = N[r * W + m];
            pcP += __builtin_popcount(p);
            pcN += __builtin_popcount(n);
            for (int b = 0; b < 8; b++) {
                uint32_t X = 0;
                for (int j = 0; j < 32; j++) {
                    uint32_t u = (uint32_t)((int32_t)x[m * 32 + j] + 128);
                    X |= ((u >> b) & 1u) << j;
                }
                int64_t D = 2 * ((int64_t)__builtin_popcount(p & X) -
                                 (int64_t)__builtin_popcount(n & X)) -
                            __builtin_popcount(p) + __builtin_popcount(n);
                sum += D * ((int64_t)1 << b);
            }
        }
        int64_t twice = sum - pcP + pcN;
        int64_t dot = twice / 2;
        if (dot32) dot32[r] = (int32_t)dot;
        y[r] = (float)dot * s;
    }
}

/* ------------------------------------------------------------------------
 * Activation quantization.
 *
 * [P4] "web-xpu-ops", operator table entry "quantize" and the q4 format
 * table (its reciprocal and rounding rows, which name quantize's own
 * convention): per row, absmax to int8 symmetric in [-127, 127]; the
 * reciprocal 127/absmax is formed in f64; each code is Math.round of
 * x * (127/absmax), i.e. floor(v) + (v - floor(v) >= 0.5), ties toward
 * +infinity, clamped to [-127, 127]; the scale is absmax/127. A row whose
 * absmax is 0 gets scale 0 and all-zero codes. Inputs must be finite.
 * ------------------------------------------------------------------------ */
static int32_t math_round_code(double v)
{
    double f = floor(v);
    double q = f + ((v - f) >= 0.5 ? 1.0 : 0.0);
    if (q > 127.0) q = 127.0;
    if (q < -127.0) q = -127.0;
    return (int32_t)q;
}

void gdo_quantize_absmax_int8(const float *x, int64_t M, int64_t K, int8_t *q, float *scale)
{
    for (int64_t r = 0; r < M; r++) {
        const float *xr = x + r * K;
        double amax = 0.0;
        for (int64_t j = 0; j < K; j++) {
            double a = fabs((double)xr[j]);
            if (a > amax) amax = a;
        }
        if (amax == 0.0) {
            for (int64_t j = 0; j < K; j++) q[r * K + j] = 0;
            scale[r] = 0.0f;
            continue;
        }
        double inv = 127.0 / amax;
        for (int64_t j = 0; j < K; j++) q[r * K + j] = (int8_t)math_round_code((double)xr[j] * inv);
        scale[r] = (float)(amax / 127.0);
    }
}

/* f32 -> IEEE binary16, round to nearest even: the value is written as an
 * integer significand in units of the target spacing 2^(E-10) (E the binade,
 * at least -14, where the spacing of the subnormals is reached), rounded by
 * rint() under the default nearest-even mode; a carry into 2048 moves one
 * binade up, and E > 15 is infinity. NaN becomes a quiet NaN. */
uint16_t gdo_f32_to_f16(float f)
{
    uint16_t s = signbit(f) ? 0x8000u : 0u;
    if (isnan(f)) return (uint16_t)(s | 0x7e00u);
    if (isinf(f)) return (uint16_t)(s | 0x7c00u);
    double a = fabs((double)f);
    if (a == 0.0) return s;
    int E;
    frexp(a, &E);
    E -= 1;                                  /* a in [2^E, 2^(E+1)) */
    if (E < -14) E = -14;
    double m = rint(ldexp(a, 10 - E));       /* exact scaling, then one rounding */
    if (m >= 2048.0) {
        m = 1024.0;
        E += 1;
    }
    if (E > 15) return (uint16_t)(s | 0x7c00u);
    if (m < 1024.0) return (uint16_t)(s | (uint16_t)m);   /* subnormal */
    return (uint16_t)(s | (uint16_t)(((uint32_t)(E + 15) << 10) | ((uint32_t)m - 1024u)));
}

/* q8_0 activation blocks in [P1]'s 34-byte format (f16 d, then 32 int8
 * codes; packQ8 reads d from the first two bytes, little-endian). The pages
 * fix the block but not how it is quantized; reading: the [P4] per-row rule
 * above applied to each block of 32 elements (codes from 127/absmax in f64
 * and Math.round), with d = f16_RNE(f32(absmax / 127)). A block whose
 * absmax is 0 is all zero. x is [n][K] f32, K a multiple of 32; out is
 * n * (K/32) blocks. */
void gdo_quantize_q8_0(const float *x, int64_t n, int64_t K, uint8_t *out)
{
    const int64_t nb = K / QK8;
    for (int64_t c = 0; c < n; c++) {
        for (int64_t i = 0; i < nb; i++) {
            const float *xb = x + c * K + i * QK8;
            uint8_t *o = out + (c * nb + i) * Q8_BYTES;
            double amax = 0.0;
            for (int j = 0; j < QK8; j++) {
                double a = fabs((double)xb[j]);
                if (a > amax) amax = a;
            }
            uint16_t d = 0;
            int8_t codes[QK8];
            if (amax == 0.0) {
                memset(codes, 0, sizeof codes);
            } else {
                double inv = 127.0 / amax;
                for (int j = 0; j < QK8; j++) codes[j] = (int8_t)math_round_code((double)xb[j] * inv);
                d = gdo_f32_to_f16((float)(amax / 127.0));
            }
            o[0] = (uint8_t)(d & 0xffu);
            o[1] = (uint8_t)(d >> 8);
            memcpy(o + 2, codes, QK8);
        }
    }
}
