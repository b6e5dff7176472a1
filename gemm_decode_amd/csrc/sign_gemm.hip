// sign_gemm.hip -- sign-bit prefill GEMM y = x @ w^T on gfx950 matrix cores
// (page "BonsaiのWebGPUカーネルを読み解く", figure on PrismML's kernels:
// q1_bits packs the sign bits of 32 weights per u32, bit 1 -> +1.0 and
// 0 -> -1.0, with one q1_scales entry per 32 weights; prefill over many
// tokens is the compute-bound case, which the page's third path hands to the
// GPU's cooperative matrix instructions).
//
// Numerics. Row m of x is scaled by 2^e_m, the power of two that puts its
// largest |x| in [2^14, 2^15), and split as v = hi + lo + r with
// hi = fp16(v), lo = fp16(v - hi) (v - hi is exact in f32), |r| <= 2^-22 |v|
// for normal-range values. The +-1 weights are exact in fp16. Per 32-weight
// group g two v_mfma_f32_16x16x32_f16 (hi, then lo into the same f32
// accumulator) give the group's signed sum; the group scale is applied on
// the VALU, acc = fma(scale[n][g], D, acc), and y = acc * 2^-e_m exactly.
// The result is within ~1e-7 of ||y||_inf of the f64 definition for any
// finite x.
//
// Three steps; a call on unpacked weights runs split and wpack as one launch
// (independent work, side by side), a call on packed weights split alone.
//  split: one workgroup per row (rows padded to a multiple of 16) finds e_m
//         and writes the row's hi/lo halves to the workspace, each 32-weight
//         group as one 128-byte line (its 32 hi halves, then its 32 lo
//         halves, in MFMA element order), so the GEMM converts nothing and a
//         lane's A operand is 16 contiguous bytes.
//  wpack: regroups the sign words and scales by pairs of groups (below).
//  gemm:  a workgroup of eight waves (two per SIMD) owns a 64 (tokens) x
//         128 (outputs) tile; each wave owns 32 tokens x all 128 outputs
//         (2 x 8 MFMA tiles, so every A fragment feeds eight MFMAs) over a
//         quarter of K. A operands come from the workspace; each lane loads the
//         sign words and scales of two weight rows and ds_bpermute hands
//         every lane the words of its MFMA column; each lane then expands
//         them into B fragments with two VALU ops per fp16 pair. Each
//         two-group step's loads are issued one step ahead and the loop has
//         no barrier (one at the end adds the quarters). Workgroups are mapped
//         so that one XCD runs consecutive tiles of the same token rows,
//         whose activation lines then stay in that XCD's L2.
//
// Element order inside a group. Any order gives the same sums, so A and B
// use the one that makes B cheap: element 2j + h (j < 4, h < 2) of fragment
// quarter q (lanes 16q .. 16q+15) is weight 16h + 4q + 3 - j. Shifting the
// sign word left by 12 - 4q + j puts the bits of elements 2j and 2j+1 at
// bits 15 and 31, and ((word << (12 - 4q + j)) & 0x80008000) ^ 0xbc00bc00 is
// the fp16 pair: bit 1 -> 0x3c00 (+1), bit 0 -> 0xbc00 (-1).
#include "gd_internal.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef const u32x4 __attribute__((address_space(1))) *g_u4;
typedef const f32x4 __attribute__((address_space(1))) *g_f4;
typedef const uint32_t __attribute__((address_space(1))) *g_u1;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef const u32x2 __attribute__((address_space(1))) *g_u2;
typedef const f32x2 __attribute__((address_space(1))) *g_f2;
typedef const float __attribute__((address_space(1))) *g_f1;

constexpr int kPrepThreads = 256;
constexpr int kThreads = 512;             // 8 waves: 4 (K quarters) x 2 (token halves), two per SIMD
constexpr int kTM = 64, kTN = 128;
constexpr int kStep = 2;                  // groups per load step

// ------------------------------------------------------------------- prep
// Workspace, in this order:
//  split activations: row m, group g is the 128-byte line at (m*G + g)*128:
//    halves 8q .. 8q+7 are the hi parts of fragment quarter q's elements,
//    halves 32 + 8q .. 32 + 8q+7 the lo parts (rows padded to 16, zero);
//  row exponents: one int32 per padded row;
//  weights: u32x4 at (g/2)*N + n = {bits[n][g], bits[n][g+1], scale[n][g],
//    scale[n][g+1]} for even g (a missing group g+1 = G has scale 0), so the
//    words of a group pair for consecutive outputs are contiguous.
// sign_wpack_kernel regroups the weights through LDS: a workgroup reads 64
// rows x 32 groups with 16-byte loads along the rows and writes 16 pairs x
// 64 outputs, each pair a contiguous 1 KiB run.
constexpr int kPackRows = 64, kPackGroups = 32;

// Tile (bx, by): rows 64*bx.., groups 32*by..
__device__ __forceinline__ void wpack_tile(const uint32_t *bits_g, const float *scales_g, int64_t N, int64_t G,
                                           u32x4 *__restrict__ wv, int64_t bx, int64_t by) {
    __shared__ uint32_t tb[kPackRows][kPackGroups + 1];
    __shared__ uint32_t ts[kPackRows][kPackGroups + 1];
    const int64_t n0 = bx * kPackRows;
    const int64_t g0 = by * kPackGroups;
    const int tid = threadIdx.x;
#pragma unroll
    for (int k = 0; k < kPackRows * kPackGroups / kPrepThreads; k++) {   // 8 words per thread
        const int idx = tid + k * kPrepThreads;
        const int r = idx / kPackGroups, c = idx % kPackGroups;
        const int64_t n = n0 + r, g = g0 + c;
        const bool live = n < N && g < G;
        tb[r][c] = live ? bits_g[n * G + g] : 0u;
        ts[r][c] = live ? __builtin_bit_cast(uint32_t, scales_g[n * G + g]) : 0u;
    }
    __syncthreads();
    const int64_t G2 = (G + 1) / 2;
#pragma unroll
    for (int k = 0; k < kPackRows * kPackGroups / 2 / kPrepThreads; k++) {   // 4 outputs per thread
        const int idx = tid + k * kPrepThreads;
        const int gp = idx / kPackRows, r = idx % kPackRows;
        const int64_t n = n0 + r, pair = g0 / 2 + gp;
        if (n < N && pair < G2)
            wv[pair * N + n] = u32x4{tb[r][2 * gp], tb[r][2 * gp + 1], ts[r][2 * gp], ts[r][2 * gp + 1]};
    }
}

__global__ __launch_bounds__(kPrepThreads) void sign_wpack_kernel(const uint32_t *bits_g, const float *scales_g,
                                                                  int64_t N, int64_t G, u32x4 *__restrict__ wv) {
    wpack_tile(bits_g, scales_g, N, G, wv, blockIdx.x, blockIdx.y);
}

// sign_split_kernel splits one padded row of x per workgroup; for
// K <= 32 * kSplitItems * kPrepThreads / 4 the row stays in registers
// between finding its largest |x| and converting it.
constexpr int kSplitItems = 4;   // (group, quarter) items per thread held in registers

__device__ __forceinline__ void split_row(const float *x_g, int64_t M, int64_t K, uint32_t *__restrict__ xs,
                                          int32_t *__restrict__ rexp, int64_t m) {
    const int64_t G = K / 32;
    const int tid = threadIdx.x;
    __shared__ float red[kPrepThreads / 64];
    const bool live = m < M;
    const g_f4 row = (g_f4)(x_g + (live ? m : 0) * K);
    const int64_t items = G * 4;                       // item (g, q): weights 4q.. and 16+4q.. of group g
    const bool held = items <= static_cast<int64_t>(kSplitItems) * kPrepThreads;
    f32x4 va[kSplitItems], vb[kSplitItems];
    float amax = 0.0f;
    if (live) {
        if (held) {
#pragma unroll
            for (int k = 0; k < kSplitItems; k++) {
                const int64_t it = tid + static_cast<int64_t>(k) * kPrepThreads;
                const int64_t itc = it < items ? it : items - 1;      // repeats are harmless for the max
                va[k] = row[8 * (itc / 4) + itc % 4];
                vb[k] = row[8 * (itc / 4) + 4 + itc % 4];
#pragma unroll
                for (int e = 0; e < 4; e++) amax = fmaxf(amax, fmaxf(fabsf(va[k][e]), fabsf(vb[k][e])));
            }
        } else {
            for (int64_t c = tid; c < K / 4; c += kPrepThreads) {
                const f32x4 v = row[c];
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
            }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if (tid % 64 == 0) red[tid / 64] = amax;
    __syncthreads();
    float rm = red[0];
#pragma unroll
    for (int w = 1; w < kPrepThreads / 64; w++) rm = fmaxf(rm, red[w]);
    const int e = rm > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(rm) : 0;
    if (tid == 0) rexp[m] = e;

    u32x4 *dst = reinterpret_cast<u32x4 *>(xs) + m * G * 8;
    auto emit = [&](int64_t it, const f32x4 &a, const f32x4 &b) {
        const int64_t g = it / 4;
        const int q = static_cast<int>(it % 4);
        union { _Float16 h[8]; u32x4 u; } hv, lv;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float v0 = __builtin_ldexpf(a[3 - j], e);
            const float v1 = __builtin_ldexpf(b[3 - j], e);
            hv.h[2 * j] = static_cast<_Float16>(v0);
            hv.h[2 * j + 1] = static_cast<_Float16>(v1);
            lv.h[2 * j] = static_cast<_Float16>(v0 - static_cast<float>(hv.h[2 * j]));
            lv.h[2 * j + 1] = static_cast<_Float16>(v1 - static_cast<float>(hv.h[2 * j + 1]));
        }
        dst[g * 8 + q] = hv.u;
        dst[g * 8 + 4 + q] = lv.u;
    };
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    if (held) {
#pragma unroll
        for (int k = 0; k < kSplitItems; k++) {
            const int64_t it = tid + static_cast<int64_t>(k) * kPrepThreads;
            if (it < items) emit(it, live ? va[k] : zero, live ? vb[k] : zero);
        }
    } else {
        for (int64_t it = tid; it < items; it += kPrepThreads) {
            f32x4 a = zero, b = zero;
            if (live) {
                a = row[8 * (it / 4) + it % 4];
                b = row[8 * (it / 4) + 4 + it % 4];
            }
            emit(it, a, b);
        }
    }
}

__global__ __launch_bounds__(kPrepThreads) void sign_split_kernel(const float *x_g, int64_t M, int64_t K,
                                                                  uint32_t *__restrict__ xs,
                                                                  int32_t *__restrict__ rexp) {
    split_row(x_g, M, K, xs, rexp, blockIdx.x);
}

// Both per-call preparations in one launch (they are independent): the first
// n_split workgroups split one padded row of x each, the rest regroup one
// 64 x 32 tile of the weights each (tile index = blockIdx.x - n_split, rows
// fastest), so the two run side by side instead of one after the other.
__global__ __launch_bounds__(kPrepThreads) void sign_prep_kernel(const float *x_g, int64_t M, int64_t K,
                                                                 uint32_t *__restrict__ xs, int32_t *__restrict__ rexp,
                                                                 int64_t n_split, const uint32_t *bits_g,
                                                                 const float *scales_g, int64_t N,
                                                                 u32x4 *__restrict__ wv, int64_t wpack_x) {
    const int64_t b = blockIdx.x;
    if (b < n_split) {
        split_row(x_g, M, K, xs, rexp, b);
    } else {
        const int64_t t = b - n_split;
        wpack_tile(bits_g, scales_g, N, K / 32, wv, t % wpack_x, t / wpack_x);
    }
}

// ------------------------------------------------------------------- gemm
struct StepBuf {
    u32x4 a[kStep][2][2];      // [group][m tile][hi, lo] A operands
    u32x4 w[2];                // {bits g0, bits g0+1, scale g0, scale g0+1} of outputs n0 + lane, n0 + 64 + lane
};

// Workgroup of eight waves, two per SIMD: wave w covers tokens 32*(w%2) of
// the 64-token tile, all 128 outputs (2 x 8 MFMA tiles), and quarter w/2 of
// the group pairs; the quarters meet at the end through LDS and are added
// in quarter order.
__global__ __launch_bounds__(kThreads) void sign_gemm_kernel(const uint32_t *xs_g, const int32_t *rexp,
                                                             const u32x4 *wv_g, float *__restrict__ y, int64_t M,
                                                             int64_t N, int64_t G, int64_t tiles_n, int64_t tiles,
                                                             int64_t per_xcd) {
    __shared__ floatx4 part[3][2][16][64];              // quarters 1-3, [quarter-1][token half][tile][lane]
    const int64_t wg = blockIdx.x;
    const int64_t L = (wg % 8) * per_xcd + wg / 8;     // workgroup wg runs on XCD wg % 8
    if (L >= tiles) return;                             // uniform: the whole workgroup leaves
    const int64_t tm = L / tiles_n, tn = L % tiles_n;
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / 64);   // wave-uniform
    const int l = threadIdx.x % 64;
    const int kq = w / 2, wm = w % 2;
    const int li = l % 16, lq = l / 16;

    const int64_t m16 = (M + 15) / 16;
    g_u4 xrow[2];              // this lane's A rows (tile rows 16*t + li, t clamped to the last tile), quarter lq
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
        int64_t t = tm * 4 + wm * 2 + mt;
        t = t < m16 ? t : m16 - 1;
        xrow[mt] = (g_u4)xs_g + (t * 16 + li) * G * 8 + lq;
    }
    g_u4 wrow[2];              // outputs n0 + l and n0 + 64 + l (clamped)
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int64_t n = tn * kTN + 64 * h + l;
        wrow[h] = (g_u4)wv_g + (n < N ? n : N - 1);
    }
    int bp[4];                 // ds_bpermute byte address of lane 16k + li
#pragma unroll
    for (int k = 0; k < 4; k++) bp[k] = (16 * k + li) * 4;

    const int64_t S = (G + kStep - 1) / kStep;          // group pairs of the whole K
    const int64_t Sq = (S + 3) / 4;                     // pairs per quarter (the last may have fewer)
    const int64_t first = kq * Sq;
    int64_t cnt = S - first;                            // this wave's pairs
    cnt = cnt < 0 ? 0 : (cnt > Sq ? Sq : cnt);

    // Pair i of this wave; i >= cnt reloads the last pair (never computed).
    // A missing second group of the last pair (G odd) reads group G-1 with
    // the zero scale the workspace holds for it.
    auto load = [&](int64_t i, StepBuf &r) {
        i = i < cnt ? i : (cnt > 0 ? cnt - 1 : 0);
        int64_t st = first + i;
        st = st < S ? st : S - 1;              // a wave with no pairs (cnt == 0) loads the last one
        const int64_t g0 = st * kStep;
#pragma unroll
        for (int q = 0; q < kStep; q++) {
            const int64_t g = g0 + q < G ? g0 + q : G - 1;
#pragma unroll
            for (int mt = 0; mt < 2; mt++) {
                r.a[q][mt][0] = xrow[mt][g * 8];
                r.a[q][mt][1] = xrow[mt][g * 8 + 4];
            }
        }
#pragma unroll
        for (int h = 0; h < 2; h++) r.w[h] = wrow[h][st * N];
    };

    floatx4 acc[2][8];
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int nt = 0; nt < 8; nt++) acc[mt][nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    const int sh = 12 - 4 * lq;
    auto compute = [&](const StepBuf &r) {
#pragma unroll
        for (int q = 0; q < kStep; q++) {
            // column li of n tile nt is output 16*nt + li of the tile: lane (16*nt + li) % 64 holds it
            uint32_t bw[8];
            float sc[8];
#pragma unroll
            for (int nt = 0; nt < 8; nt++) {
                bw[nt] = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(bp[nt % 4], static_cast<int>(r.w[nt / 4][q])));
                sc[nt] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(bp[nt % 4],
                                                                             static_cast<int>(r.w[nt / 4][2 + q])));
            }
            half8 bf[8];
#pragma unroll
            for (int nt = 0; nt < 8; nt++) {
                u32x4 v;
#pragma unroll
                for (int j = 0; j < 4; j++) v[j] = ((bw[nt] << (sh + j)) & 0x80008000u) ^ 0xbc00bc00u;
                bf[nt] = __builtin_bit_cast(half8, v);
            }
#pragma unroll
            for (int mt = 0; mt < 2; mt++)
#pragma unroll
                for (int n4 = 0; n4 < 8; n4 += 4) {   // four independent hi -> lo -> scale chains
                    floatx4 d[4];
#pragma unroll
                    for (int u = 0; u < 4; u++)
                        d[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, r.a[q][mt][0]),
                                                                     bf[n4 + u], floatx4{0.0f, 0.0f, 0.0f, 0.0f}, 0,
                                                                     0, 0);
#pragma unroll
                    for (int u = 0; u < 4; u++)
                        d[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, r.a[q][mt][1]),
                                                                     bf[n4 + u], d[u], 0, 0, 0);
#pragma unroll
                    for (int u = 0; u < 4; u++)
#pragma unroll
                        for (int rr = 0; rr < 4; rr++)
                            acc[mt][n4 + u][rr] = __builtin_fmaf(sc[n4 + u], d[u][rr], acc[mt][n4 + u][rr]);
                }
        }
    };

    // Scheduling barriers keep each pair's loads where they are written and
    // stop the compiler from pulling one pair's arithmetic into another's
    // (which would wait for loads that are meant to still be in flight).
    // Two register sets rotate by name over an unconditional loop body; an
    // odd last pair is peeled off after it.
    StepBuf r0, r1;
    load(0, r0);
    __builtin_amdgcn_sched_barrier(0);
    int64_t i = 0;
    for (; i + 1 < cnt; i += 2) {
        load(i + 1, r1);
        __builtin_amdgcn_sched_barrier(0);
        compute(r0);
        __builtin_amdgcn_sched_barrier(0);
        load(i + 2, r0);
        __builtin_amdgcn_sched_barrier(0);
        compute(r1);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (i < cnt) compute(r0);

    // Quarters 1-3 hand their sums to quarter 0, which adds them in order.
    if (kq > 0) {
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
            for (int nt = 0; nt < 8; nt++) part[kq - 1][wm][mt * 8 + nt][l] = acc[mt][nt];
    }
    __syncthreads();
    if (kq > 0) return;
#pragma unroll
    for (int p = 0; p < 3; p++)
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
            for (int nt = 0; nt < 8; nt++) {
                const floatx4 o = part[p][wm][mt * 8 + nt][l];
#pragma unroll
                for (int rr = 0; rr < 4; rr++) acc[mt][nt][rr] = acc[mt][nt][rr] + o[rr];
            }

    // D layout of a 16x16 MFMA tile: lane l holds rows 4*(l/16) + r, column l%16.
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int rr = 0; rr < 4; rr++) {
            const int64_t m = tm * kTM + wm * 32 + mt * 16 + 4 * lq + rr;
            if (m >= M) continue;
            const int ne = -rexp[m];
#pragma unroll
            for (int nt = 0; nt < 8; nt++) {
                const int64_t n = tn * kTN + nt * 16 + li;
                if (n < N) y[m * N + n] = __builtin_ldexpf(acc[mt][nt][rr], ne);
            }
        }
}

int workspace_size(int64_t M, int64_t N, int64_t K, int64_t *bytes) {
    const int64_t m16 = (M + 15) / 16, G2 = (K / 32 + 1) / 2;
    int64_t a, b, c, d;
    GD_REQUIRE(gd::mul_ok(m16 * 16, K, &a) && gd::mul_ok(a, 4, &b) && gd::mul_ok(G2, N, &c) &&
                   gd::mul_ok(c, 16, &d),
               GD_ERANGE, "workspace size overflows");
    *bytes = b + m16 * 16 * 4 + d;    // split activations, row exponents, regrouped weights
    return GD_OK;
}

}  // namespace

using namespace gd;

extern "C" int q1_sign_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t *bytes) {
    GD_REQUIRE(bytes, GD_EINVAL, "q1_sign_gemm_workspace_bytes: null output pointer");
    GD_REQUIRE(M >= 1 && N >= 1 && K >= 1, GD_EINVAL,
               "q1_sign_gemm_workspace_bytes: M (%lld), N (%lld) and K (%lld) must be >= 1", (long long)M,
               (long long)N, (long long)K);
    GD_REQUIRE(K % 32 == 0, GD_ESHAPE, "q1_sign_gemm_workspace_bytes: K (%lld) must be a multiple of 32",
               (long long)K);
    GD_REQUIRE(M <= INT64_C(2147483647) && N <= INT64_C(2147483647) && K <= INT64_C(2147483647), GD_ERANGE,
               "q1_sign_gemm_workspace_bytes: M, N or K above 2^31-1");
    int64_t b;
    const int st = workspace_size(M, N, K, &b);
    if (st) return st;
    *bytes = static_cast<size_t>(b);
    clear_error();
    return GD_OK;
}

namespace {

int check_mnk(const char *who, int64_t M, int64_t N, int64_t K) {
    GD_REQUIRE(M >= 1 && N >= 1 && K >= 1, GD_EINVAL, "%s: M (%lld), N (%lld), K (%lld) must be >= 1", who,
               (long long)M, (long long)N, (long long)K);
    GD_REQUIRE(K % 32 == 0, GD_ESHAPE, "%s: K (%lld) must be a multiple of 32", who, (long long)K);
    GD_REQUIRE(M <= INT64_C(2147483647) && N <= INT64_C(2147483647) && K <= INT64_C(2147483647), GD_ERANGE,
               "%s: M, N or K above 2^31-1", who);
    return GD_OK;
}

int packed_size(int64_t N, int64_t K, int64_t *bytes) {
    int64_t c;
    GD_REQUIRE(gd::mul_ok((K / 32 + 1) / 2, N, &c) && gd::mul_ok(c, 16, bytes), GD_ERANGE,
               "packed weight size overflows");
    return GD_OK;
}

// Launches split + GEMM against weights already in the packed layout.
int split_and_gemm(const float *x, const u32x4 *wv, float *y, int64_t M, int64_t N, int64_t K, void *workspace,
                   hipStream_t s, const char *who, bool split_done = false) {
    const int64_t G = K / 32;
    const int64_t m16 = (M + 15) / 16;
    uint32_t *xs = static_cast<uint32_t *>(workspace);
    int32_t *rexp = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + m16 * 16 * K * 4);
    const int64_t tiles_m = (M + kTM - 1) / kTM, tiles_n = (N + kTN - 1) / kTN;
    const int64_t tiles = tiles_m * tiles_n;
    const int64_t per_xcd = (tiles + 7) / 8;
    GD_REQUIRE(per_xcd * 8 <= INT64_C(0xffffffff), GD_ERANGE, "%s: grid too large", who);
    if (!split_done)
        hipLaunchKernelGGL(sign_split_kernel, dim3(static_cast<uint32_t>(m16 * 16)), dim3(kPrepThreads), 0, s, x, M,
                           K, xs, rexp);
    hipLaunchKernelGGL(sign_gemm_kernel, dim3(static_cast<uint32_t>(per_xcd * 8)), dim3(kThreads), 0, s, xs, rexp,
                       wv, y, M, N, G, tiles_n, tiles, per_xcd);
    return check_launch(who);
}

}  // namespace

extern "C" int q1_sign_packed_bytes(int64_t N, int64_t K, size_t *bytes) {
    GD_REQUIRE(bytes, GD_EINVAL, "q1_sign_packed_bytes: null output pointer");
    int st = check_mnk("q1_sign_packed_bytes", 1, N, K);
    if (st) return st;
    int64_t b;
    st = packed_size(N, K, &b);
    if (st) return st;
    *bytes = static_cast<size_t>(b);
    clear_error();
    return GD_OK;
}

extern "C" int q1_sign_pack(const uint32_t *w_bits, const float *w_scales, int64_t N, int64_t K, void *w_packed,
                            void *stream) {
    GD_REQUIRE(w_bits && w_scales && w_packed, GD_EINVAL, "q1_sign_pack: null pointer");
    int st = check_mnk("q1_sign_pack", 1, N, K);
    if (st) return st;
    GD_REQUIRE(aligned(w_bits, 4) && aligned(w_scales, 4) && aligned(w_packed, 16), GD_EALIGN,
               "q1_sign_pack: w_bits and w_scales must be 4-byte aligned, w_packed 16-byte");
    const int64_t G = K / 32;
    const int64_t wpack_x = (N + kPackRows - 1) / kPackRows, wpack_y = (G + kPackGroups - 1) / kPackGroups;
    GD_REQUIRE(wpack_x <= INT64_C(0xffffffff) && wpack_y <= 65535, GD_ERANGE, "q1_sign_pack: grid too large");
    hipLaunchKernelGGL(sign_wpack_kernel, dim3(static_cast<uint32_t>(wpack_x), static_cast<uint32_t>(wpack_y)),
                       dim3(kPrepThreads), 0, as_stream(stream), w_bits, w_scales, N, G,
                       static_cast<u32x4 *>(w_packed));
    return check_launch("q1_sign_pack");
}

extern "C" int q1_sign_gemm_packed(const float *x, const void *w_packed, float *y, int64_t M, int64_t N, int64_t K,
                                   void *workspace, size_t workspace_bytes, void *stream) {
    GD_REQUIRE(x && w_packed && y && workspace, GD_EINVAL, "q1_sign_gemm_packed: null pointer");
    int st = check_mnk("q1_sign_gemm_packed", M, N, K);
    if (st) return st;
    GD_REQUIRE(aligned(x, 16) && aligned(w_packed, 16) && aligned(y, 4) && aligned(workspace, 16), GD_EALIGN,
               "q1_sign_gemm_packed: x, w_packed and workspace must be 16-byte aligned, y 4-byte");
    const int64_t m16 = (M + 15) / 16;
    int64_t a, need;
    GD_REQUIRE(mul_ok(m16 * 16, K, &a) && mul_ok(a, 4, &need), GD_ERANGE, "q1_sign_gemm_packed: size overflows");
    need += m16 * 16 * 4;   // split activations and row exponents; no weight part
    GD_REQUIRE(workspace_bytes >= static_cast<size_t>(need), GD_ERANGE,
               "q1_sign_gemm_packed: workspace of %zu bytes, %lld needed", workspace_bytes, (long long)need);
    return split_and_gemm(x, static_cast<const u32x4 *>(w_packed), y, M, N, K, workspace, as_stream(stream),
                          "q1_sign_gemm_packed");
}

extern "C" int q1_sign_gemm(const float *x, const uint32_t *w_bits, const float *w_scales, float *y, int64_t M,
                            int64_t N, int64_t K, void *workspace, size_t workspace_bytes, void *stream) {
    GD_REQUIRE(x && w_bits && w_scales && y && workspace, GD_EINVAL, "q1_sign_gemm: null pointer");
    GD_REQUIRE(M >= 1 && N >= 1 && K >= 1, GD_EINVAL, "q1_sign_gemm: M (%lld), N (%lld), K (%lld) must be >= 1",
               (long long)M, (long long)N, (long long)K);
    GD_REQUIRE(K % 32 == 0, GD_ESHAPE, "q1_sign_gemm: K (%lld) must be a multiple of 32", (long long)K);
    GD_REQUIRE(M <= INT64_C(2147483647) && N <= INT64_C(2147483647) && K <= INT64_C(2147483647), GD_ERANGE,
               "q1_sign_gemm: M, N or K above 2^31-1");
    GD_REQUIRE(aligned(x, 16) && aligned(w_bits, 4) && aligned(w_scales, 4) && aligned(y, 4) &&
                   aligned(workspace, 16),
               GD_EALIGN, "q1_sign_gemm: x and workspace must be 16-byte aligned, w_bits, w_scales and y 4-byte");
    int64_t need;
    int st = workspace_size(M, N, K, &need);
    if (st) return st;
    GD_REQUIRE(workspace_bytes >= static_cast<size_t>(need), GD_ERANGE,
               "q1_sign_gemm: workspace of %zu bytes, %lld needed", workspace_bytes, (long long)need);
    const int64_t G = K / 32;
    const int64_t m16 = (M + 15) / 16;
    u32x4 *wv = reinterpret_cast<u32x4 *>(static_cast<char *>(workspace) + m16 * 16 * K * 4 + m16 * 16 * 4);
    const int64_t wpack_x = (N + kPackRows - 1) / kPackRows, wpack_y = (G + kPackGroups - 1) / kPackGroups;
    GD_REQUIRE(wpack_x <= INT64_C(0xffffffff) && wpack_y <= 65535, GD_ERANGE, "q1_sign_gemm: grid too large");
    const int64_t n_prep = m16 * 16 + wpack_x * wpack_y;
    GD_REQUIRE(n_prep <= INT64_C(0xffffffff), GD_ERANGE, "q1_sign_gemm: grid too large");
    hipStream_t s = as_stream(stream);
    uint32_t *xs = static_cast<uint32_t *>(workspace);
    int32_t *rexp = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + m16 * 16 * K * 4);
    hipLaunchKernelGGL(sign_prep_kernel, dim3(static_cast<uint32_t>(n_prep)), dim3(kPrepThreads), 0, s, x, M, K, xs,
                       rexp, m16 * 16, w_bits, w_scales, N, wv, wpack_x);
    return split_and_gemm(x, wv, y, M, N, K, workspace, s, "q1_sign_gemm", true);
}
