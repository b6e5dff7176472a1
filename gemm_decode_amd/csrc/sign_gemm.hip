// sign_gemm.hip -- sign-bit prefill GEMM y = x @ w^T on gfx950 matrix cores
// (page "BonsaiのWebGPUカーネルを読み解く", figure on PrismML's kernels:
// q1_bits packs the sign bits of 32 weights per u32, bit 1 -> +1.0 and
// 0 -> -1.0, with one q1_scales entry per 32 weights; prefill over many
// tokens is the compute-bound case, which the page's third path hands to the
// GPU's cooperative matrix instructions).
//
// Numerics. The +-1 weights are exact in fp16. Each x is split as
// x = hi + lo + e with hi = fp16(x), lo = fp16(x - hi) (x - hi is exact in
// f32), |e| <= 2^-22 |x| for normal-range values. Per 32-weight group g two
// v_mfma_f32_16x16x32_f16 (hi pass, then lo pass into the same f32
// accumulator) give the group's signed sum up to f32 accumulation; the group
// scale is then applied on the VALU: acc = fma(scale[n][g], D, acc). The
// result is within ~1e-7 of ||y||_inf of the f64 definition.
//
// Tiling. A workgroup of eight waves computes a 64 (tokens) x 128 (outputs)
// tile; each wave owns 32 x 32 of it (2 x 2 MFMA tiles of 16 x 16). Per step
// of two groups (K = 64) the workgroup converts x's 64 x 64 slice to hi/lo
// fp16 once into LDS (double-buffered, one barrier per step), while each lane
// expands its own sign bytes into B fragments through a 16-entry LDS table
// (one 8-byte read per 4 weights). Global loads run two steps ahead.
#include "gd_internal.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;             // 8 waves: 2 (tokens) x 4 (outputs)
constexpr int kTM = 64, kTN = 128;
constexpr int kStepGroups = 2;            // 32-weight groups per barrier
constexpr int kKS = 32 * kStepGroups;     // 64
constexpr int kRow = kKS + 8;             // LDS row stride in halves (padding)

__global__ __launch_bounds__(kThreads) void sign_gemm_kernel(const float *__restrict__ x,
                                                             const uint32_t *__restrict__ bits,
                                                             const float *__restrict__ scales,
                                                             float *__restrict__ y, int64_t M, int64_t N,
                                                             int64_t K) {
    __shared__ __attribute__((aligned(16))) _Float16 a_hi[2][kTM * kRow];
    __shared__ __attribute__((aligned(16))) _Float16 a_lo[2][kTM * kRow];
    __shared__ u32x2 lut[16];   // 4 fp16 +-1 values per 4-bit sign group

    const int tid = threadIdx.x;
    const int w = tid / 64, l = tid % 64;
    const int wm = w >> 2, wn = w & 3;    // wave: 32 tokens x 32 outputs
    const int li = l % 16, lq = l / 16;   // MFMA lane row/column, K quarter
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kTM;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kTN;
    const int G = static_cast<int>(K / 32);
    const int S = (G + kStepGroups - 1) / kStepGroups;   // steps

    if (tid < 16) {
        uint32_t h[4];
        for (int j = 0; j < 4; j++) h[j] = ((tid >> j) & 1) ? 0x3C00u : 0xBC00u;   // +1.0 / -1.0
        lut[tid] = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    }

    // Staging role: tile row sr, 8 consecutive columns at sc8 of each step's
    // 64. Rows past M, groups past G and outputs past N read clamped (valid)
    // addresses; such results are never stored (a group past G is given a zero
    // scale), so the loop has no guards.
    const int sr = tid >> 3, sc8 = (tid & 7) * 8;
    const int64_t xrow = (m0 + sr < M) ? m0 + sr : M - 1;
    const float *xrowp = x + xrow * K;
    const int64_t na = n0 + wn * 32 + li, nb_ = na + 16;
    const uint32_t *bp0 = bits + (na < N ? na : N - 1) * G;
    const uint32_t *bp1 = bits + (nb_ < N ? nb_ : N - 1) * G;
    const float *sp0 = scales + (na < N ? na : N - 1) * G;
    const float *sp1 = scales + (nb_ < N ? nb_ : N - 1) * G;

    struct StepRegs {
        float4 x0, x1;                 // staging: 8 x of one row
        uint32_t b[kStepGroups][2];    // sign words (group, output)
        float c[kStepGroups][2];       // scales
    };
    auto load = [&](int st, StepRegs &r) {
        const int sc = st < S ? st : S - 1;
        int gx = sc * kStepGroups + sc8 / 32;               // this thread's group for x
        gx = gx < G ? gx : G - 1;
        const float4 *xp = reinterpret_cast<const float4 *>(xrowp + gx * 32 + (sc8 % 32));
        r.x0 = xp[0];
        r.x1 = xp[1];
#pragma unroll
        for (int q = 0; q < kStepGroups; q++) {
            const int g = st * kStepGroups + q;
            const int gc = g < G ? g : G - 1;
            r.b[q][0] = bp0[gc];
            r.b[q][1] = bp1[gc];
            const float keep = g < G ? 1.0f : 0.0f;    // a group past G adds nothing
            r.c[q][0] = sp0[gc] * keep;
            r.c[q][1] = sp1[gc] * keep;
        }
    };
    auto stage_x = [&](int buf, const StepRegs &r) {
        const float xv[8] = {r.x0.x, r.x0.y, r.x0.z, r.x0.w, r.x1.x, r.x1.y, r.x1.z, r.x1.w};
        _Float16 hv[8], lv[8];
#pragma unroll
        for (int q = 0; q < 8; q++) {
            hv[q] = static_cast<_Float16>(xv[q]);
            lv[q] = static_cast<_Float16>(xv[q] - static_cast<float>(hv[q]));
        }
        *reinterpret_cast<half8 *>(&a_hi[buf][sr * kRow + sc8]) =
            half8{hv[0], hv[1], hv[2], hv[3], hv[4], hv[5], hv[6], hv[7]};
        *reinterpret_cast<half8 *>(&a_lo[buf][sr * kRow + sc8]) =
            half8{lv[0], lv[1], lv[2], lv[3], lv[4], lv[5], lv[6], lv[7]};
    };

    floatx4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // One step: compute step st from LDS buffer st&1 with `cur` (its sign
    // words and scales), stage step st+1's x from `nxt` into the other
    // buffer, and issue step st+2's loads into `fut`. The three register sets
    // rotate by name across an unrolled-by-three loop, never by copy (a copy
    // of just-loaded registers would wait for the load).
    auto body = [&](int st, const StepRegs &cur, const StepRegs &nxt, StepRegs &fut) {
        const int buf = st & 1;
        load(st + 2, fut);
        if (st + 1 < S) stage_x(buf ^ 1, nxt);

        floatx4 d[kStepGroups][2][2];
        half8 bf[kStepGroups][2];
#pragma unroll
        for (int q = 0; q < kStepGroups; q++)
#pragma unroll
            for (int nt = 0; nt < 2; nt++) {
                const uint32_t yb = (cur.b[q][nt] >> (8 * lq)) & 0xffu;
                const u32x2 p = lut[yb & 0xf], h = lut[yb >> 4];
                bf[q][nt] = __builtin_bit_cast(half8, u32x4{p.x, p.y, h.x, h.y});
            }
        half8 ah[kStepGroups][2], al[kStepGroups][2];
#pragma unroll
        for (int q = 0; q < kStepGroups; q++)
#pragma unroll
            for (int mt = 0; mt < 2; mt++) {
                const int off = (wm * 32 + mt * 16 + li) * kRow + q * 32 + 8 * lq;
                ah[q][mt] = *reinterpret_cast<const half8 *>(&a_hi[buf][off]);
                al[q][mt] = *reinterpret_cast<const half8 *>(&a_lo[buf][off]);
            }
        // all hi passes, then the dependent lo passes
#pragma unroll
        for (int q = 0; q < kStepGroups; q++)
#pragma unroll
            for (int mt = 0; mt < 2; mt++)
#pragma unroll
                for (int nt = 0; nt < 2; nt++)
                    d[q][mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[q][mt], bf[q][nt],
                                                                         floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < kStepGroups; q++)
#pragma unroll
            for (int mt = 0; mt < 2; mt++)
#pragma unroll
                for (int nt = 0; nt < 2; nt++)
                    d[q][mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[q][mt], bf[q][nt], d[q][mt][nt], 0, 0, 0);
        // group scales, in group order
#pragma unroll
        for (int q = 0; q < kStepGroups; q++)
#pragma unroll
            for (int mt = 0; mt < 2; mt++)
#pragma unroll
                for (int nt = 0; nt < 2; nt++)
#pragma unroll
                    for (int rr = 0; rr < 4; rr++)
                        acc[mt][nt][rr] = __builtin_fmaf(cur.c[q][nt], d[q][mt][nt][rr], acc[mt][nt][rr]);
        __syncthreads();
    };

    StepRegs ra, rb, rc;
    load(0, ra);
    load(1, rb);
    stage_x(0, ra);
    __syncthreads();   // LUT and step 0's A ready
    for (int st = 0; st < S; st += 3) {
        body(st, ra, rb, rc);
        if (st + 1 < S) body(st + 1, rb, rc, ra);
        if (st + 2 < S) body(st + 2, rc, ra, rb);
    }

    // D layout of a 16x16 MFMA tile: lane l holds rows 4*(l/16) + r, column l%16.
#pragma unroll
    for (int nt = 0; nt < 2; nt++) {
        const int64_t n = nt ? nb_ : na;
        if (n >= N) continue;
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
            for (int rr = 0; rr < 4; rr++) {
                const int64_t m = m0 + wm * 32 + mt * 16 + 4 * lq + rr;
                if (m < M) y[m * N + n] = acc[mt][nt][rr];
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
    GD_REQUIRE((M + kTM - 1) / kTM <= 65535, GD_ERANGE, "q1_sign_gemm: M above 65535*64");
    GD_REQUIRE(aligned(x, 16) && aligned(w_bits, 16) && aligned(w_scales, 16) && aligned(y, 16), GD_EALIGN,
               "q1_sign_gemm: x, w_bits, w_scales and y must be 16-byte aligned");
    const dim3 grid(static_cast<uint32_t>((N + kTN - 1) / kTN), static_cast<uint32_t>((M + kTM - 1) / kTM));
    hipLaunchKernelGGL(sign_gemm_kernel, grid, dim3(kThreads), 0, as_stream(stream), x, w_bits, w_scales, y, M, N,
                       K);
    return check_launch("q1_sign_gemm");
}
