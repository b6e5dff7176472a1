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
    GD_REQUIRE(aligned(x, 4) && aligned(scales, 4) && aligned(y, 4), GD_EALIGN,
               "blockq8_matmul_nt: x, scales and y must be 4-byte aligned");
    hipStream_t st = as_stream(stream);
    const int mi = static_cast<int>(m);
    if (m == 1)
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
