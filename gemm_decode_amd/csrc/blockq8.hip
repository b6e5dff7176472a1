// blockq8.hip -- block-scaled int8 matmul_nt y = x @ w^T on gfx950 (page
// "block_q8_matmul_nt.wgsl": PACKING -- four int8 per u32, element t in byte
// t%4 of word t/4, sign-extended; ACCUMULATION ORDER -- the block scale
// multiplies each 32-element block's sub-total once).
//
// Mapping (VALU path). Sixteen lanes share an output feature (a row of w)
// and split its k range in 16-byte pieces of 16 quants, so a wave reads 256
// contiguous bytes of each of four rows per load. The activation rows are
// staged once per workgroup in LDS. Each lane forms the sub-total of its 16
// quants against every activation row, scales it by its block's scale and
// accumulates; the sixteen partials of a row are then added across lanes.
// This regroups the page's f32 order (16-element pieces instead of
// 32-element blocks, a different final sum order); the results agree with
// that order within 1e-5 of ||y||_inf.
#include "gd_device.h"
#include "gd_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerRow = 16;
constexpr int kRowsPerPass = kThreads / kLanesPerRow;   // 16
constexpr int kPasses = 8;
constexpr int kRowsPerWG = kRowsPerPass * kPasses;      // 128
constexpr int kMaxXFloats = 16384;                      // 64 KiB of staged activations

// Sign-extended byte b of word w, as f32.
__device__ __forceinline__ float sbyte(uint32_t w, int b) {
    return static_cast<float>(static_cast<int32_t>(w << (24 - 8 * b)) >> 24);
}

template <int M>
__global__ __launch_bounds__(kThreads) void blockq8_valu_kernel(const float *__restrict__ x,
                                                                const uint32_t *__restrict__ quants,
                                                                const float *__restrict__ scales,
                                                                float *__restrict__ y, int m, int64_t k,
                                                                int64_t n) {
    extern __shared__ float xs[];
    for (int64_t i = threadIdx.x; i < static_cast<int64_t>(m) * k; i += kThreads) xs[i] = x[i];
    __syncthreads();
    const int lane = threadIdx.x % kLanesPerRow;
    const int rsub = threadIdx.x / kLanesPerRow;
    const int64_t chunks = k / 16;
    const int64_t bpr = k / 32;
    for (int pass = 0; pass < kPasses; pass++) {
        const int64_t c = static_cast<int64_t>(blockIdx.x) * kRowsPerWG + pass * kRowsPerPass + rsub;
        float acc[M];
#pragma unroll
        for (int r = 0; r < M; r++) acc[r] = 0.0f;
        if (c < n) {
            const uint4 *qrow = reinterpret_cast<const uint4 *>(quants + c * (k / 4));
            const float *srow = scales + c * bpr;
            for (int64_t ch = lane; ch < chunks; ch += kLanesPerRow) {
                const uint4 q4 = qrow[ch];
                const float sc = srow[ch >> 1];
                const uint32_t qw[4] = {q4.x, q4.y, q4.z, q4.w};
                float qf[16];
#pragma unroll
                for (int t = 0; t < 16; t++) qf[t] = sbyte(qw[t >> 2], t & 3);
#pragma unroll
                for (int r = 0; r < M; r++) {
                    if (r < m) {
                        const float4 *xr = reinterpret_cast<const float4 *>(xs + r * k + ch * 16);
                        float s = 0.0f;
#pragma unroll
                        for (int v = 0; v < 4; v++) {
                            const float4 xv = xr[v];
                            s = __builtin_fmaf(xv.x, qf[4 * v + 0], s);
                            s = __builtin_fmaf(xv.y, qf[4 * v + 1], s);
                            s = __builtin_fmaf(xv.z, qf[4 * v + 2], s);
                            s = __builtin_fmaf(xv.w, qf[4 * v + 3], s);
                        }
                        acc[r] = __builtin_fmaf(sc, s, acc[r]);
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < M; r++) {
            float v = acc[r];
            v += __shfl_xor(v, 1, kLanesPerRow);
            v += __shfl_xor(v, 2, kLanesPerRow);
            v += __shfl_xor(v, 4, kLanesPerRow);
            v += __shfl_xor(v, 8, kLanesPerRow);
            if (lane == 0 && c < n && r < m) y[r * n + c] = v;
        }
    }
}

// ---------------------------------------------------------------- m = 1
// Decode GEMV (one activation row). Thirty-two lanes share an output
// feature; lane j owns chunks c = j + 32t (t < kCPL) of 16 quants, the same
// positions in every row, so its slice of x (up to 32 floats) stays in
// registers for all its rows. Each quant byte is
// converted sign-extended (one v_cvt_f32_i32 with an SDWA byte select and
// sext, as the page's quant_at reads it) and multiplied into the chunk's
// sum, so the f32 error follows sum |x*q| whatever the mean of x. x is read
// from HBM once per workgroup into LDS. A wave covers two rows per step and
// keeps the loads of the next three steps in flight (four register sets
// rotated by name).
constexpr int kLPR = 32;                // lanes per row
constexpr int kCPL = 2;                 // chunks per lane: k <= 16*kLPR*kCPL = 1024
constexpr int kGemvThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef const u32x4 __attribute__((address_space(1))) *gq_t;
typedef const float __attribute__((address_space(1))) *gf_t;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef const f32x4 __attribute__((address_space(1))) *gx_t;

struct RowBuf {
    u32x4 q[kCPL];
    float s[kCPL];
};

__global__ __launch_bounds__(kGemvThreads) void blockq8_gemv_kernel(const float *x_g, const uint32_t *quants_g,
                                                                     const float *scales_g,
                                                                     float *__restrict__ y, int64_t k, int64_t n,
                                                                     int64_t steps_per_wave) {
    const gq_t quants = (gq_t)quants_g;
    const gf_t scales = (gf_t)scales_g;
    const gx_t xq = (gx_t)x_g;                               // x as 16-byte words
    const int lane = threadIdx.x % kLPR;
    const int sub = (threadIdx.x % 64) / kLPR;               // row within the wave's pair
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * kGemvThreads + threadIdx.x) / 64;
    const int chunks = static_cast<int>(k / 16);
    const int64_t bpr = k / 32;
    const int64_t row0 = wave * 2 * steps_per_wave;          // rows row0 + 2i + sub

    auto load = [&](int64_t i, RowBuf &b) {
        // Steps past this wave's last are clamped to that step (a cache
        // hit; never stored), not run into the next wave's rows, which
        // would be fetched a second time.
        const int64_t ic = i < steps_per_wave ? i : steps_per_wave - 1;
        int64_t r = row0 + 2 * ic + sub;
        r = r < n ? r : n - 1;
#pragma unroll
        for (int t = 0; t < kCPL; t++) {
            int c = lane + kLPR * t;
            c = c < chunks ? c : chunks - 1;                     // masked by x = 0 below
            b.q[t] = gd::ld_stream(&quants[r * chunks + c]);
            b.s[t] = gd::ld_stream(&scales[r * bpr + c / 2]);
        }
    };
    // x once per workgroup into LDS (read before the quant loads, which the
    // in-order load counter would otherwise make it wait for)
    __shared__ f32x4 xl[kLPR * kCPL * 4];                    // k <= 1024 floats
    for (int i = threadIdx.x; i < chunks * 4; i += kGemvThreads) xl[i] = xq[i];
    RowBuf b0, b1, b2, b3;
    load(0, b0);
    load(1, b1);
    load(2, b2);
    __syncthreads();

    float xv[kCPL][16];
#pragma unroll
    for (int t = 0; t < kCPL; t++) {
        const int c = lane + kLPR * t;
        const int cc = c < chunks ? c : chunks - 1;
        const float keep = c < chunks ? 1.0f : 0.0f;
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const f32x4 w = xl[cc * 4 + v];
#pragma unroll
            for (int e = 0; e < 4; e++) xv[t][4 * v + e] = w[e] * keep;
        }
    }
    auto row_dot = [&](const RowBuf &b) {
        float acc = 0.0f;
#pragma unroll
        for (int t = 0; t < kCPL; t++) {
            float s = 0.0f;
#pragma unroll
            for (int wq = 0; wq < 4; wq++) {
                const uint32_t w = b.q[t][wq];
                s = __builtin_fmaf(xv[t][4 * wq + 0], sbyte(w, 0), s);
                s = __builtin_fmaf(xv[t][4 * wq + 1], sbyte(w, 1), s);
                s = __builtin_fmaf(xv[t][4 * wq + 2], sbyte(w, 2), s);
                s = __builtin_fmaf(xv[t][4 * wq + 3], sbyte(w, 3), s);
            }
            acc = __builtin_fmaf(b.s[t], s, acc);
        }
        acc += __shfl_xor(acc, 1, kLPR);
        acc += __shfl_xor(acc, 2, kLPR);
        acc += __shfl_xor(acc, 4, kLPR);
        acc += __shfl_xor(acc, 8, kLPR);
        acc += __shfl_xor(acc, 16, kLPR);
        return acc;
    };
    auto store = [&](int64_t i, float v) {
        const int64_t r = row0 + 2 * i + sub;
        if (lane == 0 && i < steps_per_wave && r < n) y[r] = v;
    };
    for (int64_t i = 0; i < steps_per_wave; i += 4) {
        load(i + 3, b3);
        store(i, row_dot(b0));
        load(i + 4, b0);
        store(i + 1, row_dot(b1));
        load(i + 5, b1);
        store(i + 2, row_dot(b2));
        load(i + 6, b2);
        store(i + 3, row_dot(b3));
    }
}

// ---------------------------------------------------------------- 2 <= m <= 16
// Small-M GEMM on the matrix cores. One v_mfma_f32_16x16x32_f16 spans
// exactly one 32-element block (K = 32), so its output is the block's
// sub-total for a 16 x 16 tile of (activation row, output feature) and the
// block scale is applied once to it, as in the page's order.
//   A = x, row i = lane % 16, k slice 8*(lane/16) .. +7 of the block, as an
//       f16 pair hi + lo (x = hi + lo to 22 bits) after scaling each row by
//       a power of two 2^e that puts its largest |x| in [2^14, 2^15); the
//       sub-total is scaled back by 2^-e before the block scale.
//   B = w, column j = lane % 16 (output feature n0 + j), same k slice: one
//       8-byte load per lane per block. Bytes become f16 exactly: the byte
//       of q + 128 under the exponent byte 0x64 is the f16 1024 + q + 128,
//       and one packed f16 add of -1152 leaves q.
//   D lane l holds rows 4*(l/16) + r (r < 4) of column l % 16.
// A wave owns one 16-feature tile and issues the loads of all its blocks
// (k <= 1024, at most 32) before the activations are staged; a workgroup of
// twelve waves stages the activations once, in MFMA operand order in LDS.
constexpr int kMfmaWaves = 12;
constexpr int kMfmaThreads = 64 * kMfmaWaves;
constexpr int kMfmaMaxK = 1024;
constexpr int kScStride = 33;          // padded row of staged block scales
constexpr int kAhead = 12;             // weight blocks in flight per lane

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef const u32x2 __attribute__((address_space(1))) *gq2_t;

// Four f16 values q (two's-complement bytes of w) as two packed f16 pairs.
__device__ __forceinline__ void q8_to_half4(uint32_t w, uint32_t &lo, uint32_t &hi) {
    const uint32_t u = w ^ 0x80808080u;                                     // q + 128
    const uint32_t a = (u & 0xffu) | ((u & 0xff00u) << 8) | 0x64006400u;   // bytes 0, 1
    const uint32_t b = ((u >> 16) & 0xffu) | ((u >> 8) & 0xff0000u) | 0x64006400u;
    const half2v bias = {static_cast<_Float16>(-1152.0f), static_cast<_Float16>(-1152.0f)};
    lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, a) + bias);
    hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, b) + bias);
}

template <int NB>
__global__ __launch_bounds__(kMfmaThreads) void blockq8_mfma_kernel(const float *x_g, const uint32_t *quants_g,
                                                                     const float *scales_g, float *__restrict__ y,
                                                                     int m, int nb, int64_t n) {
    __shared__ __attribute__((aligned(16))) half8 xop[NB][2][64];   // [block][hi, lo][lane]
    __shared__ float sc[kMfmaWaves][16][kScStride];                  // [wave][feature][block]
    __shared__ float wmax[kMfmaWaves][16];
    __shared__ int rexp[16];
    constexpr int kSlots = 64 * NB;                                  // (block, k slice, row) triples
    constexpr int kSlotIters = (kSlots + kMfmaThreads - 1) / kMfmaThreads;

    const gx_t xg = (gx_t)x_g;
    const gq2_t quants = (gq2_t)quants_g;
    const gf_t scales = (gf_t)scales_g;
    const int tid = threadIdx.x;
    const int l = tid % 64;
    const int wv = tid / 64;
    const int j = l % 16;
    const int g = l / 16;
    const int64_t k = 32 * static_cast<int64_t>(nb);
    const int64_t n0 = (static_cast<int64_t>(blockIdx.x) * kMfmaWaves + wv) * 16;

    // 1. activation slots, read first so that waiting for them does not wait
    //    for the weight loads issued after them (loads complete in order)
    const int mm = tid % 16;                       // row of every slot of this thread
    const int mmc = mm < m ? mm : m - 1;
    const float keep = mm < m ? 1.0f : 0.0f;
    f32x4 xv[kSlotIters][2];
#pragma unroll
    for (int it = 0; it < kSlotIters; it++) {
        const int s = tid + it * kMfmaThreads;
        int b = s / 64;
        b = b < nb ? b : nb - 1;
        const int64_t off = (mmc * k + 32 * b + 8 * ((s % 64) / 16)) / 4;
        xv[it][0] = xg[off] * keep;
        xv[it][1] = xg[off + 1] * keep;
    }
    // 2. this wave's block scales: rows n0 .. n0+15, two rows per load
    float sv[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        int64_t r = n0 + 2 * i + l / 32;
        r = r < n ? r : n - 1;
        const int b = (l % 32) < nb ? (l % 32) : nb - 1;
        sv[i] = scales[r * nb + b];
    }
    // 3. this lane's feature, 8 bytes at k slice g per block: the first
    //    kAhead blocks now, each later one when the block kAhead before it is
    //    consumed. A window keeps the data arriving in the order it is used;
    //    issuing every block at once (all waves on the chip do) lets the
    //    first ones arrive anywhere in the whole stream.
    const int64_t row = n0 + j < n ? n0 + j : n - 1;
    auto wload = [&](int b) {
        const int bc = b < nb ? b : nb - 1;
        return quants[row * (k / 8) + 4 * bc + g];   // plain: the line's other 24 bytes come later
    };
    u32x2 wq[NB];
#pragma unroll
    for (int b = 0; b < (kAhead < NB ? kAhead : NB); b++) wq[b] = wload(b);

    // 4. per-row power of two: largest |x| of each row over the workgroup
    float amax = 0.0f;
#pragma unroll
    for (int it = 0; it < kSlotIters; it++)
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
            for (int e = 0; e < 4; e++) amax = fmaxf(amax, fabsf(xv[it][h][e]));
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    if (l < 16) wmax[wv][l] = amax;
#pragma unroll
    for (int i = 0; i < 8; i++)   // blocks past nb get scale 0 (computed, contribute 0)
        if (l % 32 < NB) sc[wv][2 * i + l / 32][l % 32] = (l % 32) < nb ? sv[i] : 0.0f;
    __syncthreads();
    float rm = 0.0f;
#pragma unroll
    for (int w = 0; w < kMfmaWaves; w++) rm = fmaxf(rm, wmax[w][mm]);
    const int ex = rm > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(rm) : 0;
    if (tid < 16) rexp[tid] = ex;
#pragma unroll
    for (int it = 0; it < kSlotIters; it++) {
        const int s = tid + it * kMfmaThreads;
        if (s < kSlots) {   // blocks past nb are staged as zero
            half8 hv, lv;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const float v = s < 64 * nb ? __builtin_ldexpf(xv[it][e / 4][e % 4], ex) : 0.0f;
                hv[e] = static_cast<_Float16>(v);
                lv[e] = static_cast<_Float16>(v - static_cast<float>(hv[e]));
            }
            xop[s / 64][0][s % 64] = hv;
            xop[s / 64][1][s % 64] = lv;
        }
    }
    __syncthreads();

    // 5. one block per step: sub-total on the matrix cores, then the scale.
    //    Every one of the NB blocks is computed (the ones past nb have zero
    //    activations and scale), so the steps carry no branches and the
    //    compiler overlaps consecutive blocks. The row's 2^-e is applied once
    //    at the end: in the normal range scaling by a power of two commutes
    //    with rounding, so this equals unscaling each sub-total first.
    floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int b = 0; b < NB; b++) {
        if (b + kAhead < NB) wq[b + kAhead] = wload(b + kAhead);
        union { uint32_t u[4]; half8 h; } bw;
        q8_to_half4(wq[b][0], bw.u[0], bw.u[1]);
        q8_to_half4(wq[b][1], bw.u[2], bw.u[3]);
        floatx4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(xop[b][0][l], bw.h, floatx4{0.0f, 0.0f, 0.0f, 0.0f},
                                                           0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(xop[b][1][l], bw.h, d, 0, 0, 0);
        const float s = sc[wv][j][b];
#pragma unroll
        for (int r = 0; r < 4; r++) acc[r] = __builtin_fmaf(s, d[r], acc[r]);
    }
    if (n0 + j < n) {
#pragma unroll
        for (int r = 0; r < 4; r++)
            if (4 * g + r < m) y[(4 * g + r) * n + n0 + j] = __builtin_ldexpf(acc[r], -rexp[4 * g + r]);
    }
}

template <int NB>
void launch_mfma(const float *x, const uint32_t *q, const float *s, float *y, int m, int64_t k, int64_t n,
                 hipStream_t st) {
    const int64_t tiles = (n + 15) / 16;
    const int64_t gx = (tiles + kMfmaWaves - 1) / kMfmaWaves;
    hipLaunchKernelGGL(blockq8_mfma_kernel<NB>, dim3(static_cast<uint32_t>(gx)), dim3(kMfmaThreads), 0, st, x, q,
                       s, y, m, static_cast<int>(k / 32), n);
}

template <int M>
void launch_valu(const float *x, const uint32_t *q, const float *s, float *y, int m, int64_t k, int64_t n,
                 hipStream_t st) {
    const int64_t gx = (n + kRowsPerWG - 1) / kRowsPerWG;
    const size_t lds = static_cast<size_t>(m) * k * sizeof(float);
    hipLaunchKernelGGL(blockq8_valu_kernel<M>, dim3(static_cast<uint32_t>(gx)), dim3(kThreads), lds, st, x, q, s,
                       y, m, k, n);
}

}  // namespace

using namespace gd;

extern "C" int blockq8_matmul_nt(const float *x, const uint32_t *quants, const float *scales, float *y, int64_t m,
                                 int64_t k, int64_t n, void *stream) {
    GD_REQUIRE(x && quants && scales && y, GD_EINVAL, "blockq8_matmul_nt: null pointer");
    GD_REQUIRE(m >= 1 && k >= 1 && n >= 1, GD_EINVAL, "blockq8_matmul_nt: m (%lld), k (%lld), n (%lld) must be >= 1",
               (long long)m, (long long)k, (long long)n);
    GD_REQUIRE(k % 32 == 0, GD_ESHAPE, "blockq8_matmul_nt: k (%lld) must be a multiple of 32", (long long)k);
    GD_REQUIRE(m <= 16, GD_ERANGE, "blockq8_matmul_nt: m (%lld) above 16", (long long)m);
    GD_REQUIRE(m * k <= kMaxXFloats, GD_ERANGE, "blockq8_matmul_nt: m*k (%lld) above %d", (long long)(m * k),
               kMaxXFloats);
    GD_REQUIRE(n <= (INT64_C(1) << 31), GD_ERANGE, "blockq8_matmul_nt: n above 2^31");
    GD_REQUIRE(aligned(quants, 16), GD_EALIGN, "blockq8_matmul_nt: quants must be 16-byte aligned");
    GD_REQUIRE(aligned(x, 16), GD_EALIGN, "blockq8_matmul_nt: x must be 16-byte aligned");
    GD_REQUIRE(aligned(scales, 4) && aligned(y, 4), GD_EALIGN,
               "blockq8_matmul_nt: scales and y must be 4-byte aligned");
    hipStream_t st = as_stream(stream);
    const int mi = static_cast<int>(m);
    if (m == 1 && k <= 16 * kLPR * kCPL) {
        // steps per wave (a multiple of 4) for about 2048 waves: eight per CU
        // (two workgroups of four) on 256 CUs. Measured at k=960, n=49152:
        // 12 steps per wave 10.9 us; 8 steps (12 waves per CU) 12.1 us, the
        // per-wave prologue (x staging, the first three steps' loads) then
        // weighing more; 16 steps (six waves per CU, uneven) 12.2 us.
        const int64_t pairs = (n + 1) / 2;                        // 2 rows per wave step
        int64_t spw = (pairs + 2047) / 2048;
        spw = (spw + 3) / 4 * 4;
        const int64_t waves = (pairs + spw - 1) / spw;
        const int64_t blocks = (waves * 64 + kGemvThreads - 1) / kGemvThreads;
        hipLaunchKernelGGL(blockq8_gemv_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kGemvThreads), 0, st, x,
                           quants, scales, y, k, n, spw);
    } else if (m >= 2 && k <= kMfmaMaxK) {
        if (k <= 256)
            launch_mfma<8>(x, quants, scales, y, mi, k, n, st);
        else if (k <= 512)
            launch_mfma<16>(x, quants, scales, y, mi, k, n, st);
        else
            launch_mfma<32>(x, quants, scales, y, mi, k, n, st);
    } else if (m == 1)
        launch_valu<1>(x, quants, scales, y, mi, k, n, st);
    else if (m <= 2)
        launch_valu<2>(x, quants, scales, y, mi, k, n, st);
    else if (m <= 4)
        launch_valu<4>(x, quants, scales, y, mi, k, n, st);
    else if (m <= 8)
        launch_valu<8>(x, quants, scales, y, mi, k, n, st);
    else
        launch_valu<16>(x, quants, scales, y, mi, k, n, st);
    return check_launch("blockq8_matmul_nt");
}
