// sign_lut.hip -- sign-bit products by table lookup on gfx950: the decode
// GEMV (few activation rows) and the LUT4 prefill GEMM, kept as the
// comparator of the matrix-core path (page "BonsaiのWebGPUカーネルを読み解く",
// figure on PrismML's kernels: decode expands the signs to +-1 and multiplies;
// prefill computes the 16 partial sums of every 4 activations once in
// workgroup memory and replaces each 4-bit nibble of signs by one table
// read, reused across an M x N tile).
//
// Tables. For the 4 activation elements 4j..4j+3 of a 32-weight group (bits
// 4j..4j+3 of its sign word, least significant first, bit 1 -> +1),
// T[n] = sum_i (bit i of n ? x_i : -x_i). These are the page's {0,1} subset
// sums L[n] made signed (T = 2L - L[15]); they are built directly as
// T[0] = -(((x0 + x1) + x2) + x3) and T[n] = T[n without its lowest set bit]
// + 2 x_lowest. A group's signed sum is the 8 reads of its nibbles added in
// nibble order, and each output accumulates acc = fma(scale[n][g], sum_g,
// acc) over the groups in order. This differs from the f64 definition only
// by the rounding of those partial sums, far inside 1e-5 of ||y||_inf.
//
// Mapping. Weights come packed by q1_sign_pack: a u32x4 {bits g, bits g+1,
// scale g, scale g+1} at (g/2)*N + n, so one load of 64 consecutive outputs'
// words of a group pair is 1 KiB. The decode GEMV serves 64 outputs per
// workgroup (one per lane, the waves splitting K), or 16 (each output's K
// split over 32 slices) where 64 would leave the CUs short of workgroups.
// All lanes that read a table read the same 16 entries at once (at most 16
// distinct dwords, in distinct banks). A nibble's table offset is a byte of
// the word shifted by 2 in either direction, taken with one SDWA v_and_b32.
#include "gd_device.h"
#include "gd_internal.h"

namespace {

using gd::grp;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef const u32x4 __attribute__((address_space(1))) *g_u4;
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPairBytes = 1024;   // tables of one group pair: 16 nibble groups x 16 floats

// Builds the 16 entries of a nibble group from its four activation elements
// x at tab + q*16.
__device__ __forceinline__ void build_group_x(float *tab, int q, const f32x4 &x) {
    float v[16];
    v[0] = -(((x[0] + x[1]) + x[2]) + x[3]);
    const float d[4] = {2.0f * x[0], 2.0f * x[1], 2.0f * x[2], 2.0f * x[3]};   // exact
#pragma unroll
    for (int n = 1; n < 16; n++) v[n] = v[n & (n - 1)] + d[__builtin_ctz(n)];
    f32x4 *dst = reinterpret_cast<f32x4 *>(tab + q * 16);
#pragma unroll
    for (int m = 0; m < 4; m++) dst[m] = f32x4{v[4 * m], v[4 * m + 1], v[4 * m + 2], v[4 * m + 3]};
}

// The 16 nibble offsets of a group pair's two sign words.
struct PairOffsets {
    uint32_t o[2][8];
};

__device__ __forceinline__ void pair_offsets(const u32x4 &v, PairOffsets &po) {
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const uint32_t w = v[h];
        const uint32_t wl = w << 2, wr = w >> 2;   // nibble 2b at byte b of wl, nibble 2b+1 at byte b of wr
        po.o[h][0] = grp<0>(wl);
        po.o[h][1] = grp<0>(wr);
        po.o[h][2] = grp<1>(wl);
        po.o[h][3] = grp<1>(wr);
        po.o[h][4] = grp<2>(wl);
        po.o[h][5] = grp<2>(wr);
        po.o[h][6] = grp<3>(wl);
        po.o[h][7] = grp<3>(wr);
    }
}

// acc = fma(scale_g, sum of the group's 8 nibble reads, acc) for both groups
// of a pair whose tables start at t.
__device__ __forceinline__ float pair_accumulate(const char *t, const PairOffsets &po, const u32x4 &v, float acc) {
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const char *tg = t + h * 512;
        float s = *reinterpret_cast<const float *>(tg + po.o[h][0]);
#pragma unroll
        for (int j = 1; j < 8; j++) s = s + *reinterpret_cast<const float *>(tg + j * 64 + po.o[h][j]);
        // the element goes through a scalar first: a bit_cast applied to an
        // ext-vector element directly reads the vector's first word
        const uint32_t sbits = v[2 + h];
        acc = __builtin_fmaf(__builtin_bit_cast(float, sbits), s, acc);
    }
    return acc;
}

// ------------------------------------------------------------ decode GEMV
// One activation row per workgroup row (blockIdx.y), 64 outputs per
// workgroup (one per lane). The eight waves split every K chunk (64 group
// pairs, 4096 elements, 64 KiB of tables) in eighths; each lane loads all of
// its pairs of a chunk before the tables are built. The eight partial sums
// of an output are added in wave order at the end.
constexpr int kGvThreads = 512;
constexpr int kGvWaves = kGvThreads / 64;
constexpr int kGvChunkPairs = 64;
constexpr int kGvPairsPerWave = kGvChunkPairs / kGvWaves;   // 8
constexpr int kGvGroupIters = kGvChunkPairs * 16 / kGvThreads;   // nibble groups each thread builds per chunk

// The activation elements of this thread's nibble groups q = tid + kGvThreads*i
// of the chunk at pair c0 (zero past the chunk's cp pairs or past K). They are
// loaded before the chunk's weights: loads complete in order, so the table
// build then waits for these alone while the weights are still arriving.
__device__ __forceinline__ void chunk_x(const float *xr, int64_t c0, int64_t cp, int64_t K,
                                        f32x4 (&xq)[kGvGroupIters]) {
#pragma unroll
    for (int i = 0; i < kGvGroupIters; i++) {
        const int q = threadIdx.x + kGvThreads * i;
        const int64_t e = c0 * 64 + 4 * q;
        xq[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (q < cp * 16 && e < K) xq[i] = *reinterpret_cast<const f32x4 *>(xr + e);
    }
}

__global__ __launch_bounds__(kGvThreads) void sign_gemv_kernel(const float *__restrict__ x,
                                                               const u32x4 *__restrict__ wv_g,
                                                               float *__restrict__ y, int64_t N, int64_t K) {
    __shared__ float tab[kGvChunkPairs * kPairBytes / 4];
    __shared__ float part[kGvWaves][64];
    const g_u4 wv = (g_u4)wv_g;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int64_t m = blockIdx.y;
    const float *xr = x + m * K;
    const int64_t n = static_cast<int64_t>(blockIdx.x) * 64 + lane;
    const int64_t nl = n < N ? n : N - 1;   // clamped: computed, never stored
    const int64_t G2 = (K / 32 + 1) / 2;    // group pairs
    const char *tabc = reinterpret_cast<const char *>(tab);
    float acc = 0.0f;
    for (int64_t c0 = 0; c0 < G2; c0 += kGvChunkPairs) {
        const int64_t cp = (G2 - c0) < kGvChunkPairs ? (G2 - c0) : kGvChunkPairs;   // pairs in this chunk
        const int p0 = wave * kGvPairsPerWave;
        int cnt = static_cast<int>(cp) - p0;
        cnt = cnt < 0 ? 0 : (cnt > kGvPairsPerWave ? kGvPairsPerWave : cnt);   // uniform per wave
        f32x4 xq[kGvGroupIters];
        chunk_x(xr, c0, cp, K, xq);
        asm volatile("" ::: "memory");   // the activation loads go first
        u32x4 v[kGvPairsPerWave];
#pragma unroll
        for (int p = 0; p < kGvPairsPerWave; p++) {
            int64_t pg = c0 + p0 + p;
            pg = pg < G2 ? pg : G2 - 1;   // clamped: loaded, never used
            v[p] = gd::ld_stream(&wv[pg * N + nl]);   // read once (the LUT4 kernel's re-reads stay plain)
        }
        if (c0 > 0) __syncthreads();   // the previous chunk's reads are done
#pragma unroll
        for (int i = 0; i < kGvGroupIters; i++) {
            const int q = threadIdx.x + kGvThreads * i;
            if (q < cp * 16) build_group_x(tab, q, xq[i]);
        }
        __syncthreads();
        if (cnt == kGvPairsPerWave) {
#pragma unroll
            for (int p = 0; p < kGvPairsPerWave; p++) {
                PairOffsets po;
                pair_offsets(v[p], po);
                acc = pair_accumulate(tabc + (p0 + p) * kPairBytes, po, v[p], acc);
            }
        } else {
#pragma unroll
            for (int p = 0; p < kGvPairsPerWave; p++) {
                if (p < cnt) {
                    PairOffsets po;
                    pair_offsets(v[p], po);
                    acc = pair_accumulate(tabc + (p0 + p) * kPairBytes, po, v[p], acc);
                }
            }
        }
    }
    part[wave][lane] = acc;
    __syncthreads();
    if (wave == 0 && n < N) {
        float s = part[0][lane];
#pragma unroll
        for (int w = 1; w < kGvWaves; w++) s += part[w][lane];
        y[m * N + n] = s;
    }
}

// Narrow form for small N: OPW outputs per workgroup, thread t serving
// output t % OPW and K slice t / OPW of each 64-pair chunk (the chunk's
// tables 68 KiB in LDS), so N = 4096 gives 256 workgroups instead of 64.
// The slices' partial sums of an output meet in LDS and are added in slice
// order. Lanes of one slice read the same 16-entry table at once; a wave
// holds 64 / OPW slices on consecutive pairs, whose tables sit 64 bytes apart
// in bank order (each pair's tables padded by 64 bytes).
constexpr int kGvPairStride = kPairBytes + 64;   // bytes per pair's tables, padded
constexpr int kGvNarrowOutputs = 16;
constexpr int64_t kGvNarrowMaxN = 8192;

template <int OPW>
__global__ __launch_bounds__(kGvThreads) void sign_gemv_narrow_kernel(const float *__restrict__ x,
                                                                      const u32x4 *__restrict__ wv_g,
                                                                      float *__restrict__ y, int64_t N, int64_t K) {
    constexpr int kSlices = kGvThreads / OPW;
    constexpr int kPairsPerSlice = kGvChunkPairs / kSlices;
    __shared__ __attribute__((aligned(16))) char tab[kGvChunkPairs * kGvPairStride];
    __shared__ float part[kSlices][OPW];
    const g_u4 wv = (g_u4)wv_g;
    const int o = threadIdx.x % OPW, sl = threadIdx.x / OPW;
    const int64_t m = blockIdx.y;
    const float *xr = x + m * K;
    const int64_t n = static_cast<int64_t>(blockIdx.x) * OPW + o;
    const int64_t nl = n < N ? n : N - 1;   // clamped: computed, never stored
    const int64_t G2 = (K / 32 + 1) / 2;    // group pairs
    float acc = 0.0f;
    for (int64_t c0 = 0; c0 < G2; c0 += kGvChunkPairs) {
        const int64_t cp = (G2 - c0) < kGvChunkPairs ? (G2 - c0) : kGvChunkPairs;   // pairs in this chunk
        // this slice's pairs: sl, sl + kSlices, ... (consecutive slices on
        // consecutive pairs, whose padded tables fall in different banks)
        f32x4 xq[kGvGroupIters];
        chunk_x(xr, c0, cp, K, xq);
        asm volatile("" ::: "memory");   // the activation loads go first
        u32x4 v[kPairsPerSlice];
#pragma unroll
        for (int p = 0; p < kPairsPerSlice; p++) {
            int64_t pg = c0 + sl + kSlices * p;
            pg = pg < G2 ? pg : G2 - 1;   // clamped: loaded, never used
            v[p] = gd::ld_stream(&wv[pg * N + nl]);   // read once (the LUT4 kernel's re-reads stay plain)
        }
        if (c0 > 0) __syncthreads();   // the previous chunk's reads are done
#pragma unroll
        for (int i = 0; i < kGvGroupIters; i++) {   // nibble group q % 16 of pair q / 16
            const int q = threadIdx.x + kGvThreads * i;
            if (q < cp * 16) build_group_x(reinterpret_cast<float *>(tab + (q / 16) * kGvPairStride), q % 16, xq[i]);
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < kPairsPerSlice; p++) {
            const int pl = sl + kSlices * p;   // pair within the chunk (uniform per slice)
            if (pl < cp) {
                PairOffsets po;
                pair_offsets(v[p], po);
                acc = pair_accumulate(tab + pl * kGvPairStride, po, v[p], acc);
            }
        }
    }
    part[sl][o] = acc;
    __syncthreads();
    if (static_cast<int>(threadIdx.x) < OPW && n < N) {
        float s = part[0][o];
#pragma unroll
        for (int k = 1; k < kSlices; k++) s += part[k][o];
        y[m * N + n] = s;
    }
}

// ------------------------------------------------------- LUT4 prefill GEMM
// A workgroup owns 16 tokens x 512 outputs (eight waves, one output per
// lane, 16 accumulators per lane). Per K chunk of 8 group pairs (512
// elements) the tables of all 16 tokens are built (128 KiB), then each
// lane's nibble offsets are extracted once per pair and serve all 16 tokens.
constexpr int kL4Threads = 512;
constexpr int kL4Tokens = 16;
constexpr int kL4ChunkPairs = 8;
constexpr int kL4TokenBytes = kL4ChunkPairs * kPairBytes;   // 8 KiB
constexpr int kL4GroupIters = kL4Tokens * kL4ChunkPairs * 16 / kL4Threads;   // table groups per thread and chunk

__global__ __launch_bounds__(kL4Threads) void sign_lut4_kernel(const float *__restrict__ x,
                                                               const u32x4 *__restrict__ wv_g,
                                                               float *__restrict__ y, int64_t M, int64_t N,
                                                               int64_t K) {
    __shared__ float tab[kL4Tokens * kL4TokenBytes / 4];
    const g_u4 wv = (g_u4)wv_g;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kL4Tokens;
    const int64_t n = static_cast<int64_t>(blockIdx.x) * kL4Threads + threadIdx.x;
    const int64_t nl = n < N ? n : N - 1;
    const int64_t G2 = (K / 32 + 1) / 2;
    const char *tabc = reinterpret_cast<const char *>(tab);
    float acc[kL4Tokens];
#pragma unroll
    for (int t = 0; t < kL4Tokens; t++) acc[t] = 0.0f;
    for (int64_t c0 = 0; c0 < G2; c0 += kL4ChunkPairs) {
        const int cp = static_cast<int>((G2 - c0) < kL4ChunkPairs ? (G2 - c0) : kL4ChunkPairs);   // uniform
        // the activation elements of this thread's table groups first (loads
        // complete in order: the build then waits for these alone); tokens
        // past M get zero tables (never stored)
        f32x4 xg[kL4GroupIters];
#pragma unroll
        for (int j = 0; j < kL4GroupIters; j++) {
            const int i = threadIdx.x + kL4Threads * j;
            const int t = i / (cp * 16), q = i % (cp * 16);
            const int64_t m = m0 + t;
            const int64_t e = c0 * 64 + 4 * q;
            xg[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (i < kL4Tokens * cp * 16 && m < M && e < K) xg[j] = *reinterpret_cast<const f32x4 *>(x + m * K + e);
        }
        asm volatile("" ::: "memory");
        u32x4 v[kL4ChunkPairs];
#pragma unroll
        for (int p = 0; p < kL4ChunkPairs; p++) {
            int64_t pg = c0 + p;
            pg = pg < G2 ? pg : G2 - 1;
            v[p] = wv[pg * N + nl];
        }
        if (c0 > 0) __syncthreads();
#pragma unroll
        for (int j = 0; j < kL4GroupIters; j++) {
            const int i = threadIdx.x + kL4Threads * j;
            if (i < kL4Tokens * cp * 16) build_group_x(tab + (i / (cp * 16)) * (kL4TokenBytes / 4), i % (cp * 16), xg[j]);
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < kL4ChunkPairs; p++) {
            if (p < cp) {
                PairOffsets po;
                pair_offsets(v[p], po);
#pragma unroll
                for (int t = 0; t < kL4Tokens; t++)
                    acc[t] = pair_accumulate(tabc + t * kL4TokenBytes + p * kPairBytes, po, v[p], acc[t]);
            }
        }
    }
    if (n < N) {
#pragma unroll
        for (int t = 0; t < kL4Tokens; t++)
            if (m0 + t < M) y[(m0 + t) * N + n] = acc[t];
    }
}

int check_args(const char *who, const float *x, const void *w_packed, const float *y, int64_t M, int64_t N,
               int64_t K) {
    GD_REQUIRE(x && w_packed && y, GD_EINVAL, "%s: null pointer", who);
    GD_REQUIRE(M >= 1 && N >= 1 && K >= 1, GD_EINVAL, "%s: M (%lld), N (%lld), K (%lld) must be >= 1", who,
               (long long)M, (long long)N, (long long)K);
    GD_REQUIRE(K % 32 == 0, GD_ESHAPE, "%s: K (%lld) must be a multiple of 32", who, (long long)K);
    GD_REQUIRE(N <= INT64_C(2147483647) && K <= INT64_C(2147483647), GD_ERANGE, "%s: N or K above 2^31-1", who);
    GD_REQUIRE(gd::aligned(x, 16) && gd::aligned(w_packed, 16) && gd::aligned(y, 4), GD_EALIGN,
               "%s: x and w_packed must be 16-byte aligned, y 4-byte", who);
    return GD_OK;
}

}  // namespace

using namespace gd;

extern "C" int q1_sign_gemv(const float *x, const void *w_packed, float *y, int64_t M, int64_t N, int64_t K,
                            void *stream) {
    int st = check_args("q1_sign_gemv", x, w_packed, y, M, N, K);
    if (st) return st;
    GD_REQUIRE(M <= 65535, GD_ERANGE, "q1_sign_gemv: M (%lld) above 65535", (long long)M);
    // Up to N = 8192 the narrow form (16 outputs per workgroup, four times
    // the workgroups: about 20 % faster at 4096 x 4096); above it 64 outputs
    // per workgroup already give 224+ workgroups and build fewer tables (16
    // or 32 outputs per workgroup measured 41 % and 4 % slower at
    // 14336 x 4096, and 56 outputs, 256 workgroups, 1 % faster).
    const u32x4 *wp = static_cast<const u32x4 *>(w_packed);
    if (N <= kGvNarrowMaxN)
        hipLaunchKernelGGL(sign_gemv_narrow_kernel<kGvNarrowOutputs>,
                           dim3(static_cast<uint32_t>((N + kGvNarrowOutputs - 1) / kGvNarrowOutputs),
                                static_cast<uint32_t>(M)),
                           dim3(kGvThreads), 0, as_stream(stream), x, wp, y, N, K);
    else
        hipLaunchKernelGGL(sign_gemv_kernel, dim3(static_cast<uint32_t>((N + 63) / 64), static_cast<uint32_t>(M)),
                           dim3(kGvThreads), 0, as_stream(stream), x, wp, y, N, K);
    return check_launch("q1_sign_gemv");
}

extern "C" int q1_sign_gemm_lut4(const float *x, const void *w_packed, float *y, int64_t M, int64_t N, int64_t K,
                                 void *stream) {
    int st = check_args("q1_sign_gemm_lut4", x, w_packed, y, M, N, K);
    if (st) return st;
    const int64_t gx = (N + kL4Threads - 1) / kL4Threads, gy = (M + kL4Tokens - 1) / kL4Tokens;
    GD_REQUIRE(gy <= 65535, GD_ERANGE, "q1_sign_gemm_lut4: M (%lld) too large", (long long)M);
    hipLaunchKernelGGL(sign_lut4_kernel, dim3(static_cast<uint32_t>(gx), static_cast<uint32_t>(gy)),
                       dim3(kL4Threads), 0, as_stream(stream), x, static_cast<const u32x4 *>(w_packed), y, M, N, K);
    return check_launch("q1_sign_gemm_lut4");
}
