// sign_gemm.hip -- sign-bit prefill GEMM y = x @ w^T on gfx950 matrix cores
// (page "BonsaiのWebGPUカーネルを読み解く", figure on PrismML's kernels:
// q1_bits packs the sign bits of 32 weights per u32, bit 1 -> +1.0 and
// 0 -> -1.0, with one q1_scales entry per 32 weights; prefill over many
// tokens is the compute-bound case and the page's third path hands it to the
// GPU's cooperative matrix instructions).
//
// Numerics. The +-1 weights are exact in fp16. Each x is split as
// x = hi + lo + e with hi = fp16(x), lo = fp16(x - hi) (x - hi is exact in
// f32), |e| <= 2^-22 |x| for normal-range values. Per 32-weight group g two
// v_mfma_f32_16x16x32_f16 (hi pass, then lo pass into the same f32
// accumulator) give the group's signed sum exactly up to f32 accumulation;
// the group scale is then applied on the VALU: acc = fma(scale[n][g], D, acc).
// The result is within ~1e-7 of ||y||_inf of the f64 definition.
//
// Tiling. A workgroup of four waves computes a 128 x 128 tile of y, each wave
// a 64 x 64 sub-tile as 4 x 4 MFMA tiles of 16 x 16. Per group the workgroup
// stages x's 128 x 32 slice (split into hi/lo fp16) and the 128 sign words
// (expanded to fp16 +-1) in LDS.
#include "gd_internal.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTM = 128, kTN = 128, kKS = 32;
constexpr int kRow = 40;   // LDS row stride in halves (32 + 8 padding)

__global__ __launch_bounds__(kThreads) void sign_gemm_kernel(const float *__restrict__ x,
                                                             const uint32_t *__restrict__ bits,
                                                             const float *__restrict__ scales,
                                                             float *__restrict__ y, int64_t M, int64_t N,
                                                             int64_t K) {
    __shared__ __attribute__((aligned(16))) _Float16 a_hi[kTM * kRow];
    __shared__ __attribute__((aligned(16))) _Float16 a_lo[kTM * kRow];
    __shared__ __attribute__((aligned(16))) _Float16 b_s[kTN * kRow];

    const int tid = threadIdx.x;
    const int wave = tid / 64, l = tid % 64;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kTM;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kTN;
    const int64_t G = K / 32;

    floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int li = l % 16, lk = 8 * (l / 16);

    for (int64_t g = 0; g < G; g++) {
        // ---- stage x slice [128 x 32] as hi/lo fp16
#pragma unroll
        for (int it = 0; it < 4; it++) {
            const int idx = tid + it * kThreads;          // float4 index in the tile
            const int row = idx >> 3, c4 = idx & 7;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (m0 + row < M) v = *reinterpret_cast<const float4 *>(x + (m0 + row) * K + g * 32 + c4 * 4);
            const float xv[4] = {v.x, v.y, v.z, v.w};
            _Float16 h[4], lo[4];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                h[q] = static_cast<_Float16>(xv[q]);
                lo[q] = static_cast<_Float16>(xv[q] - static_cast<float>(h[q]));
            }
            _Float16 *dh = a_hi + row * kRow + c4 * 4;
            _Float16 *dl = a_lo + row * kRow + c4 * 4;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                dh[q] = h[q];
                dl[q] = lo[q];
            }
        }
        // ---- stage sign words [128 n] as fp16 +-1 [128 x 32]
        {
            const int nrow = tid >> 1, half = tid & 1;
            uint32_t w = 0;
            if (n0 + nrow < N) w = bits[(n0 + nrow) * G + g];
            uint32_t *dst = reinterpret_cast<uint32_t *>(b_s + nrow * kRow + half * 16);
#pragma unroll
            for (int q = 0; q < 8; q++) {
                const int j = half * 16 + 2 * q;
                const uint32_t b0 = (w >> j) & 1u, b1 = (w >> (j + 1)) & 1u;
                dst[q] = 0xBC00BC00u ^ (b0 << 15) ^ (b1 << 31);   // bit 1 -> +1.0, 0 -> -1.0
            }
        }
        __syncthreads();

        float sc[4];
#pragma unroll
        for (int nt = 0; nt < 4; nt++) {
            const int64_t n = n0 + wn * 64 + nt * 16 + li;
            sc[nt] = (n < N) ? scales[n * G + g] : 0.0f;
        }
        half8 bf[4];
#pragma unroll
        for (int nt = 0; nt < 4; nt++)
            bf[nt] = *reinterpret_cast<const half8 *>(b_s + (wn * 64 + nt * 16 + li) * kRow + lk);
#pragma unroll
        for (int mt = 0; mt < 4; mt++) {
            const half8 ah = *reinterpret_cast<const half8 *>(a_hi + (wm * 64 + mt * 16 + li) * kRow + lk);
            const half8 al = *reinterpret_cast<const half8 *>(a_lo + (wm * 64 + mt * 16 + li) * kRow + lk);
#pragma unroll
            for (int nt = 0; nt < 4; nt++) {
                floatx4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bf[nt], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                d = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bf[nt], d, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; r++) acc[mt][nt][r] = __builtin_fmaf(sc[nt], d[r], acc[mt][nt][r]);
            }
        }
        __syncthreads();
    }

    // D layout of a 16x16 MFMA tile: lane l holds rows 4*(l/16) + r, column l%16.
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
#pragma unroll
        for (int nt = 0; nt < 4; nt++) {
            const int64_t n = n0 + wn * 64 + nt * 16 + li;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int64_t m = m0 + wm * 64 + mt * 16 + 4 * (l / 16) + r;
                if (m < M && n < N) y[m * N + n] = acc[mt][nt][r];
            }
        }
    }
}

}  // namespace

using namespace gd;

extern "C" int q1_sign_gemm(const float *x, const uint32_t *w_bits, const float *w_scales, float *y, int64_t M,
                            int64_t N, int64_t K, void *stream) {
    GD_REQUIRE(x && w_bits && w_scales && y, GD_EINVAL, "q1_sign_gemm: null pointer");
    GD_REQUIRE(M >= 1 && N >= 1 && K >= 1, GD_EINVAL, "q1_sign_gemm: M (%lld), N (%lld), K (%lld) must be >= 1",
               (long long)M, (long long)N, (long long)K);
    GD_REQUIRE(K % 32 == 0, GD_ESHAPE, "q1_sign_gemm: K (%lld) must be a multiple of 32", (long long)K);
    GD_REQUIRE(M <= INT64_C(2147483647) && N <= INT64_C(2147483647), GD_ERANGE, "q1_sign_gemm: M or N above 2^31-1");
    GD_REQUIRE((M + kTM - 1) / kTM <= 65535, GD_ERANGE, "q1_sign_gemm: M above 65535*128");
    GD_REQUIRE(aligned(x, 16) && aligned(w_bits, 16) && aligned(w_scales, 16) && aligned(y, 16), GD_EALIGN,
               "q1_sign_gemm: x, w_bits, w_scales and y must be 16-byte aligned");
    const dim3 grid(static_cast<uint32_t>((N + kTN - 1) / kTN), static_cast<uint32_t>((M + kTM - 1) / kTM));
    hipLaunchKernelGGL(sign_gemm_kernel, grid, dim3(kThreads), 0, as_stream(stream), x, w_bits, w_scales, y, M, N,
                       K);
    return check_launch("q1_sign_gemm");
}
