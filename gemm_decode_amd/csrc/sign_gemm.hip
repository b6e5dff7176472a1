// sign_gemm.hip -- sign-bit prefill GEMM y = x @ w^T on gfx950 matrix cores
// (page "BonsaiのWebGPUカーネルを読み解く", figure on PrismML's kernels:
// q1_bits packs the sign bits of 32 weights per u32, bit 1 -> +1.0 and
// 0 -> -1.0, with one q1_scales entry per 32 weights; prefill over many
// tokens is the compute-bound case, which the page's third path hands to the
// GPU's cooperative matrix instructions).
//
// Numerics. Each row m of x, in each eighth p of K, is scaled by 2^e_mp, the
// power of two that puts its largest |x| there in [2^14, 2^15); each output
// n's scales by 2^c_n, the power of two that does the same for its largest
// |scale|. Both are split as v = h + l + r with h = fp16(v), l = fp16(v - h)
// (v - h is exact in f32), |r| <= 2^-22 |v| while v is normal in fp16. The
// group scale rides in the B operand: B = +-sh (bit 1 / bit 0) and +-sl. Per
// 32-weight group three v_mfma_f32_16x16x32_f16 add xh*sh, xl*sh and xh*sl
// (the xl*sl term, 2^-22 relative, is dropped) into the tile's f32
// accumulator; nothing else touches it. Each eighth's sums are unscaled
// exactly (ldexp by -(e_mp + c_n)) and the eight are added in a fixed order.
// Within 1e-5 of ||y||_inf of the f64 definition (about 5e-7 on the prefill
// workload).
//
// Matrix-core time on gfx950 is the budget: each 16x16x32 fp16 MFMA holds a
// SIMD for 16 cycles, and VALU instructions issued beside a wave's MFMAs do
// not overlap them (measured: each adds about 4 cycles), so the kernel keeps
// VALU per MFMA low.
//
// Three steps; a call on unpacked weights runs split and bpack as one launch
// (independent work, side by side), a call on packed weights split alone.
//  split: workgroup (16-row tile, eighth of K) finds the tile rows' exponents
//         there and writes their hi/lo halves to the workspace in MFMA
//         operand order (below), so the GEMM converts nothing and a wave's
//         A operand of one 16-row tile and group is one contiguous 1 KiB.
//  bpack: the per-output exponent and each group's {sign word, sh | sl<<16}.
//  gemm:  a workgroup of eight waves (two per SIMD, one workgroup per CU)
//         owns a 64 (tokens) x 128 (outputs) tile; wave w runs all 4 x 8
//         MFMA tiles over eighth w of the groups, so a B fragment (14 VALU
//         ops from the sign and scale words) feeds twelve MFMAs and an A
//         fragment 24. Each group's loads are issued one group ahead; the
//         group's packed words (1 KiB for 128 outputs, one 16-byte load per
//         lane) reach the lanes that need them through a per-wave LDS slot,
//         staged a group ahead too. The eighths meet in LDS at the end.
//         Workgroups are mapped so that one XCD runs consecutive tiles of the
//         same token rows, whose operands then stay in that XCD's L2.
//
// Element order inside a group. Any order gives the same sums, so A and B
// use the one that makes B cheap: element 2j + i (j < 4, i < 2) of fragment
// quarter q (lanes 16q .. 16q+15) is weight 16i + 4q + 3 - j. Shifting the
// sign word left by 12 - 4q + j puts the bits of elements 2j and 2j+1 at
// bits 15 and 31, and (~(word << (12 - 4q + j)) & 0x80008000) ^ (h | h << 16)
// is the fp16 pair +-h: bit 1 -> +h, bit 0 -> -h.
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

constexpr int kPrepThreads = 512;
constexpr int kThreads = 512;             // 8 waves: the K eighths of one 64 x 128 tile
constexpr int kTM = 64, kTN = 128;
constexpr int kKParts = kThreads / 64;    // K parts of the GEMM (one per wave), each with its own row exponents
constexpr int kBufFlags = 0x00020000;     // raw 32-bit dword format (gfx9 buffer descriptor word 3)

// ------------------------------------------------------------------- prep
// Workspace, in this order:
//  split activations: 16-row tile t, group g is the 2 KiB block at
//    (t*G + g)*2048: 64 lanes x 16 bytes of hi parts, then 64 x 16 of lo
//    parts; lane 16q + li holds the 8 halves of fragment quarter q of row
//    16t + li (rows padded to 16, zero), so one 16-byte load per lane is a
//    whole MFMA operand and 1 KiB contiguous;
//  row exponents: one int32 per padded row and eighth of K, at row*8 + p;
//  weights in the matrix-core layout: u32x2 {bits[n][g], sh | sl << 16} at
//    g*N + n (16 bytes per output and group pair reserved);
//  output exponents: one int32 per output.
// The packed weights (q1_sign_pack) hold the table kernels' layout first:
// u32x4 at (g/2)*N + n = {bits[n][g], bits[n][g+1], scale[n][g],
// scale[n][g+1]} for even g (a missing group g+1 = G has scale 0), then the
// matrix-core layout and the output exponents. sign_wpack_kernel writes the
// first through LDS: a workgroup reads 64 rows x 32 groups with 16-byte
// loads along the rows and writes 16 pairs x 64 outputs, each pair a
// contiguous 1 KiB run.
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

// The matrix-core layout of the weights (see the header comment): output n
// gets the exponent c_n that puts its largest |scale| in [2^14, 2^15), and
// each group's scale s becomes v = s * 2^c_n split as h = fp16(v), l =
// fp16(v - h) (v - h is exact in f32). Group g of output n is the u32x2
// {bits, h | l << 16} at g*N + n. A workgroup packs 16 outputs. With at most
// kBpHeld * 128 groups per output (K <= 16384) every word it needs is loaded
// at once: half a wave per output, lane c holding groups 4c..4c+3 of each
// 128-group chunk, so the output's exponent comes from registers (a 32-lane
// reduction) with one memory latency in all; each chunk then turns around in
// LDS so that the 16 outputs' words of one group go out as one 128-byte
// write. Longer rows read the scales twice, 64 groups at a time.
constexpr int kBpCols = 16;   // outputs per workgroup
constexpr int kBpHeld = 4;    // 128-group chunks held in registers

__device__ __forceinline__ uint32_t split_scale(float s, int e) {
    const float v = __builtin_ldexpf(s, e);
    const _Float16 h = static_cast<_Float16>(v);
    const _Float16 l = static_cast<_Float16>(v - static_cast<float>(h));
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l)) << 16);
}

__device__ __forceinline__ int scale_exponent(float m) {
    return m > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(m) : 0;
}

__device__ __forceinline__ void bpack_held(const uint32_t *bits_g, const float *scales_g, int64_t N, int64_t G,
                                           u32x2 *__restrict__ wb, int32_t *__restrict__ cexp, int64_t blk,
                                           u32x2 (*tile)[129]) {
    static_assert(kBpCols * 32 == kPrepThreads, "half a wave per output");
    const int tid = threadIdx.x, r = tid / 32, c = tid % 32;
    const int64_t n0 = blk * kBpCols, n = n0 + r;
    const bool live = n < N;
    const int64_t H = (G + 127) / 128;   // chunks, <= kBpHeld
    uint32_t bw[kBpHeld][4];
    float sc[kBpHeld][4];
#pragma unroll
    for (int h = 0; h < kBpHeld; h++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int64_t g = 128 * h + 4 * c + j;
            const bool in = live && h < H && g < G;
            bw[h][j] = in ? bits_g[n * G + g] : 0u;
            sc[h][j] = in ? scales_g[n * G + g] : 0.0f;
        }
    float m = 0.0f;
#pragma unroll
    for (int h = 0; h < kBpHeld; h++)
#pragma unroll
        for (int j = 0; j < 4; j++) m = fmaxf(m, fabsf(sc[h][j]));
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 32));
    const int e = scale_exponent(m);
    if (c == 0 && live) cexp[n] = e;
#pragma unroll
    for (int h = 0; h < kBpHeld; h++) {
        if (h >= H) break;   // uniform
        if (h > 0) __syncthreads();   // the previous chunk's reads of the tile are done
#pragma unroll
        for (int j = 0; j < 4; j++) tile[r][4 * c + j] = u32x2{bw[h][j], split_scale(sc[h][j], e)};
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 128 * kBpCols / kPrepThreads; k++) {
            const int i = tid + kPrepThreads * k;
            const int gl = i / kBpCols, rr = i % kBpCols;
            const int64_t g = 128 * h + gl, nn = n0 + rr;
            if (g < G && nn < N) wb[g * N + nn] = tile[rr][gl];
        }
    }
}

__device__ __forceinline__ void bpack_cols(const uint32_t *bits_g, const float *scales_g, int64_t N, int64_t G,
                                           u32x2 *__restrict__ wb, int32_t *__restrict__ cexp, int64_t blk) {
    constexpr int kWaves = kPrepThreads / 64, kRows = kBpCols / kWaves;   // outputs per wave
    __shared__ u32x2 tile[kBpCols][129];
    __shared__ int ex[kBpCols];
    if (G <= 128 * kBpHeld) {   // uniform
        bpack_held(bits_g, scales_g, N, G, wb, cexp, blk, tile);
        return;
    }
    const int tid = threadIdx.x, w = tid / 64, l = tid % 64;
    const int64_t n0 = blk * kBpCols;
    // 1. each output's largest |scale| and exponent
#pragma unroll
    for (int k = 0; k < kRows; k++) {
        const int r = w + kWaves * k;
        const int64_t n = n0 + r;
        float m = 0.0f;
        if (n < N)
            for (int64_t g = l; g < G; g += 64) m = fmaxf(m, fabsf(scales_g[n * G + g]));
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
        if (l == 0) {
            const int e = scale_exponent(m);
            ex[r] = e;
            if (n < N) cexp[n] = e;
        }
    }
    __syncthreads();
    // 2. 64 groups at a time: rows in, turned around, groups out
    for (int64_t g0 = 0; g0 < G; g0 += 64) {
#pragma unroll
        for (int k = 0; k < kRows; k++) {
            const int r = w + kWaves * k;
            const int64_t n = n0 + r, g = g0 + l;
            u32x2 v = {0u, 0u};
            if (n < N && g < G) v = u32x2{bits_g[n * G + g], split_scale(scales_g[n * G + g], ex[r])};
            tile[r][l] = v;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 64 * kBpCols / kPrepThreads; k++) {
            const int i = tid + kPrepThreads * k;
            const int gl = i / kBpCols, r = i % kBpCols;
            const int64_t g = g0 + gl, n = n0 + r;
            if (g < G && n < N) wb[g * N + n] = tile[r][gl];
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(kPrepThreads) void sign_bpack_kernel(const uint32_t *bits_g, const float *scales_g,
                                                                  int64_t N, int64_t G, u32x2 *__restrict__ wb,
                                                                  int32_t *__restrict__ cexp) {
    bpack_cols(bits_g, scales_g, N, G, wb, cexp, blockIdx.x);
}

// The split: workgroup (t, p) takes rows 16t..16t+15 over K part p (groups
// p*Gp .. (p+1)*Gp - 1, Gp = ceil(G/8): the eighth of K one GEMM wave
// runs), finds each row's largest |x| in that part, so that (row, part) has
// its own exponent e (x * 2^e in [2^14, 2^15)), and writes the part's
// 2 KiB blocks whole. Lane 16q + r of wave w handles row 16t + r, quarter q
// of groups w, w + 8, ... of the part: the lane layout of the blocks.
constexpr int kParts = kKParts;

__device__ __forceinline__ void split_tile(const float *x_g, int64_t M, int64_t K, uint32_t *__restrict__ xs,
                                           int32_t *__restrict__ rexp, int64_t t, int p) {
    constexpr int kW = kPrepThreads / 64;   // waves; wave w takes groups w, w + kW, ... of the part
    const int64_t G = K / 32, Gp = (G + kParts - 1) / kParts;
    const int64_t g0 = p * Gp;
    int64_t gn = G - g0;
    gn = gn < 0 ? 0 : (gn > Gp ? Gp : gn);
    const int tid = threadIdx.x, w = tid / 64, l = tid % 64, r = l % 16, q = l / 16;
    const int64_t m = t * 16 + r;
    const bool live = m < M;
    const g_f4 row = (g_f4)(x_g + (live ? m : 0) * K);
    __shared__ float red[kW][16];
    // Up to kHeld groups per lane stay in registers between the two passes
    // (K <= 256 * kW * kHeld); longer parts are read again for the second.
    constexpr int kHeld = 2;
    const bool held = gn <= kW * kHeld;
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4 ha[kHeld], hb[kHeld];
    float amax = 0.0f;
    if (held) {
#pragma unroll
        for (int k = 0; k < kHeld; k++) {
            const int64_t i = w + kW * k;
            const bool in = live && i < gn;
            ha[k] = in ? row[8 * (g0 + i) + q] : zero;
            hb[k] = in ? row[8 * (g0 + i) + 4 + q] : zero;
#pragma unroll
            for (int e = 0; e < 4; e++) amax = fmaxf(amax, fmaxf(fabsf(ha[k][e]), fabsf(hb[k][e])));
        }
    } else if (live) {
        for (int64_t i = w; i < gn; i += kW) {
            const int64_t g = g0 + i;
            const f32x4 a = row[8 * g + q], b = row[8 * g + 4 + q];
#pragma unroll
            for (int e = 0; e < 4; e++) amax = fmaxf(amax, fmaxf(fabsf(a[e]), fabsf(b[e])));
        }
    }
    amax = fmaxf(amax, __shfl_xor(amax, 16));   // the four quarters of row r
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    if (q == 0) red[w][r] = amax;
    __syncthreads();
    float rm = red[0][r];
#pragma unroll
    for (int k = 1; k < kW; k++) rm = fmaxf(rm, red[k][r]);
    const int e = rm > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(rm) : 0;
    if (w == 0 && q == 0) rexp[m * kParts + p] = e;   // padded rows included (e = 0)

    // (16-row tile t, group g): 64 lanes x 16 bytes of hi parts, then of lo
    // parts; lane 16q + r holds the 8 halves of quarter q of row 16t + r.
    u32x4 *dst = reinterpret_cast<u32x4 *>(xs) + t * G * 128 + l;
    auto emit = [&](int64_t g, const f32x4 &a, const f32x4 &b) {
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
        dst[g * 128] = hv.u;
        dst[g * 128 + 64] = lv.u;
    };
    if (held) {
#pragma unroll
        for (int k = 0; k < kHeld; k++)
            if (w + kW * k < gn) emit(g0 + w + kW * k, ha[k], hb[k]);
    } else {
        for (int64_t i = w; i < gn; i += kW) {
            const int64_t g = g0 + i;
            emit(g, live ? row[8 * g + q] : zero, live ? row[8 * g + 4 + q] : zero);
        }
    }
}

__global__ __launch_bounds__(kPrepThreads) void sign_split_kernel(const float *x_g, int64_t M, int64_t K,
                                                                  uint32_t *__restrict__ xs,
                                                                  int32_t *__restrict__ rexp) {
    split_tile(x_g, M, K, xs, rexp, blockIdx.x / kParts, static_cast<int>(blockIdx.x % kParts));
}

// Both per-call preparations in one launch (they are independent): the first
// n_split workgroups split one (16-row tile, K part) of x each, the rest
// pack 16 outputs' weights each, so the two run side by side.
__global__ __launch_bounds__(kPrepThreads) void sign_prep_kernel(const float *x_g, int64_t M, int64_t K,
                                                                 uint32_t *__restrict__ xs, int32_t *__restrict__ rexp,
                                                                 int64_t n_split, const uint32_t *bits_g,
                                                                 const float *scales_g, int64_t N,
                                                                 u32x2 *__restrict__ wb, int32_t *__restrict__ cexp) {
    const int64_t b = blockIdx.x;
    if (b < n_split)
        split_tile(x_g, M, K, xs, rexp, b / kParts, static_cast<int>(b % kParts));
    else
        bpack_cols(bits_g, scales_g, N, K / 32, wb, cexp, b - n_split);
}

// ------------------------------------------------------------------- gemm
struct StepBuf {
    u32x4 a[4][2];             // [m tile][hi, lo] A operands of one group
    u32x4 w;                   // {bits, h|l} of the tile's outputs 2*lane and 2*lane + 1
};

// B fragments of one n tile for one group from its sign word and its h|l
// scale word: element 2j + i of the lane's quarter is weight 16i + 4q + 3 - j,
// whose sign bit the shift by sh + j moves to bit 15 (i = 0) or 31 (i = 1);
// each fp16 lane value is then +h (bit 1) or -h (bit 0), (~t & 0x80008000)
// ^ (h | h << 16), and the same for l.
__device__ __forceinline__ void b_frags(uint32_t bits, uint32_t hl, int sh, half8 &bh, half8 &bl) {
    const uint32_t hh = __builtin_amdgcn_perm(hl, hl, 0x01000100u);   // h | h << 16
    const uint32_t ll = __builtin_amdgcn_perm(hl, hl, 0x03020302u);   // l | l << 16
    u32x4 vh, vl;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint32_t t = bits << (sh + j);
        vh[j] = (~t & 0x80008000u) ^ hh;
        vl[j] = (~t & 0x80008000u) ^ ll;
    }
    bh = __builtin_bit_cast(half8, vh);
    bl = __builtin_bit_cast(half8, vl);
}

// Workgroup of eight waves over a 64 (tokens) x 128 (outputs) tile, one
// workgroup per CU: wave w runs all 4 x 8 MFMA tiles of the tile over eighth
// w of the groups, so each B fragment (14 VALU ops to build) feeds twelve
// MFMAs and each A fragment 24. Every group adds hi*h, lo*h and hi*l to each
// tile's accumulator on the matrix cores; the eighths meet at the end in
// LDS in a fixed order.
__global__ __launch_bounds__(kThreads) void sign_gemm_kernel(const uint32_t *xs_g, const int32_t *rexp,
                                                             const u32x2 *wb_g, const int32_t *cexp,
                                                             float *__restrict__ y, int64_t M, int64_t N, int64_t G,
                                                             int64_t tiles_n, int64_t tiles, int64_t per_xcd) {
    __shared__ floatx4 part[4][32][64];                 // four partial tiles: [slot][tile][lane], 128 KiB
    __shared__ u32x4 wst[kThreads / 64][64];            // per wave: one group's words of the tile's outputs
    __shared__ int ex_r[kTM][kKParts], ex_c[kTN];       // the tile's row (per K part) and output exponents
    const int64_t wg = blockIdx.x;
    const int64_t L = (wg % 8) * per_xcd + wg / 8;     // workgroup wg runs on XCD wg % 8
    if (L >= tiles) return;                             // uniform: the whole workgroup leaves
    const int64_t tm = L / tiles_n, tn = L % tiles_n;
    const int64_t m16 = (M + 15) / 16;
    // The tile's row (per K part) and output exponents, fetched now and
    // parked in LDS for the epilogue (a barrier before it orders them);
    // rows past the padded rows take the last padded tile's (never stored).
    static_assert(kTM * kKParts == kThreads && kTN <= kThreads, "one exponent per thread");
    int my_er, my_ec = 0;
    {
        const int lr = static_cast<int>(threadIdx.x) / kKParts, lp = static_cast<int>(threadIdx.x) % kKParts;
        int64_t t = tm * 4 + lr / 16;
        t = t < m16 ? t : m16 - 1;
        my_er = rexp[(t * 16 + lr % 16) * kKParts + lp];
        if (threadIdx.x < kTN) {
            const int64_t n = tn * kTN + threadIdx.x;
            my_ec = cexp[n < N ? n : N - 1];
        }
    }
    const int kw = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / 64);   // wave-uniform
    const int l = threadIdx.x % 64;
    const int li = l % 16, lq = l / 16;

    g_u4 xrow[4];              // this lane's A operands of m tile mt (row tile t clamped to the last one)
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
        int64_t t = tm * 4 + mt;
        t = t < m16 ? t : m16 - 1;
        xrow[mt] = (g_u4)xs_g + t * G * 128 + l;
    }
    // The tile's 128 outputs' group-g words are 1 KiB at (g*N + 128*tn)*8 of
    // the packed weights: one 16-byte load per lane (outputs 2*lane, 2*lane +
    // 1), through a buffer descriptor of their size, so that outputs past N
    // read zeros (last group) or another output's words (never stored). The
    // wave parks them in its LDS slot; column li of n tile nt (output 16*nt +
    // li of the tile) reads its 8 bytes back.
    const int64_t wbytes = G * N * 8;
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u32x2 *>(wb_g), 0, static_cast<int>(wbytes < INT32_MAX ? wbytes : INT32_MAX), kBufFlags);
    const uint32_t woff = static_cast<uint32_t>((tn * kTN + 2 * l) * 8);
    u32x2 *slot = reinterpret_cast<u32x2 *>(wst[kw]);

    const int64_t Ge = (G + 7) / 8;                     // groups per eighth (the last may have fewer)
    const int64_t first = kw * Ge;
    int64_t cnt = G - first;                            // this wave's groups
    cnt = cnt < 0 ? 0 : (cnt > Ge ? Ge : cnt);

    // Group i of this wave; i >= cnt reloads the last one (never computed).
    auto load = [&](int64_t i, StepBuf &r) {
        i = i < cnt ? i : (cnt > 0 ? cnt - 1 : 0);
        int64_t g = first + i;
        g = g < G ? g : G - 1;                 // a wave with no groups (cnt == 0) loads the last one
#pragma unroll
        for (int mt = 0; mt < 4; mt++) {
            r.a[mt][0] = xrow[mt][g * 128];
            r.a[mt][1] = xrow[mt][g * 128 + 64];
        }
        r.w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, woff, static_cast<int>(g * N * 8), 0));
    };

    floatx4 acc[4][8];
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int nt = 0; nt < 8; nt++) acc[mt][nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    const int sh = 12 - 4 * lq;
    // Hands a loaded group's words to the wave's LDS slot and reads n tile
    // 0's back, one group ahead of its arithmetic. Only this wave uses its
    // slot, and one wave's LDS accesses complete in program order: the
    // previous group's reads are done before this write, and this write
    // before the reads that follow.
    auto stage = [&](const StepBuf &r, u32x2 &v0) {
        wst[kw][l] = r.w;
        __builtin_amdgcn_wave_barrier();
        v0 = slot[li];
    };
    auto compute = [&](const StepBuf &r, const u32x2 v0) {
        half8 ah[4], al[4];
#pragma unroll
        for (int mt = 0; mt < 4; mt++) {
            ah[mt] = __builtin_bit_cast(half8, r.a[mt][0]);
            al[mt] = __builtin_bit_cast(half8, r.a[mt][1]);
        }
        // The group's words are in the slot (stage) and n tile 0's already
        // read. n tile nt's twelve MFMAs (hi*h, lo*h, hi*l for the four m
        // tiles, four apart on each accumulator) run while n tile nt+1's B
        // fragments are built.
        half8 bh[2], bl[2];
        {
            const uint32_t wbits = v0[0], whl = v0[1];
            b_frags(wbits, whl, sh, bh[0], bl[0]);
        }
#pragma unroll
        for (int nt = 0; nt < 8; nt++) {
            if (nt + 1 < 8) {
                const u32x2 v = slot[16 * (nt + 1) + li];
                // the elements go through scalars first: a bit_cast applied to an
                // ext-vector element directly reads the vector's first word
                const uint32_t wbits = v[0], whl = v[1];
                b_frags(wbits, whl, sh, bh[(nt + 1) & 1], bl[(nt + 1) & 1]);
            }
            const half8 h = bh[nt & 1], lo = bl[nt & 1];
#pragma unroll
            for (int mt = 0; mt < 4; mt++)
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[mt], h, acc[mt][nt], 0, 0, 0);
#pragma unroll
            for (int mt = 0; mt < 4; mt++)
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[mt], h, acc[mt][nt], 0, 0, 0);
#pragma unroll
            for (int mt = 0; mt < 4; mt++)
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[mt], lo, acc[mt][nt], 0, 0, 0);
        }
    };

    // Scheduling barriers keep each group's loads where they are written and
    // stop the compiler from pulling one group's arithmetic into another's
    // (which would wait for loads that are meant to still be in flight).
    // Two register sets rotate by name over an unconditional loop body; an
    // odd last group is peeled off after it.
    StepBuf r0, r1;
    u32x2 v0;
    load(0, r0);
    stage(r0, v0);
    __builtin_amdgcn_sched_barrier(0);
    int64_t i = 0;
    for (; i + 1 < cnt; i += 2) {
        load(i + 1, r1);
        __builtin_amdgcn_sched_barrier(0);
        compute(r0, v0);
        __builtin_amdgcn_sched_barrier(0);
        stage(r1, v0);
        __builtin_amdgcn_sched_barrier(0);
        load(i + 2, r0);
        __builtin_amdgcn_sched_barrier(0);
        compute(r1, v0);
        __builtin_amdgcn_sched_barrier(0);
        stage(r0, v0);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (i < cnt) compute(r0, v0);
    ex_r[threadIdx.x / kKParts][threadIdx.x % kKParts] = my_er;
    if (threadIdx.x < kTN) ex_c[threadIdx.x] = my_ec;
    __syncthreads();

    // Each wave first undoes its part's scalings on its own sums, exactly:
    // element (row, output) times 2^-(row's exponent in this part + the
    // output's exponent). The D layout of a 16x16 MFMA tile: lane l holds
    // rows 4*(l/16) + r, column l % 16. The eighths then meet in LDS in three
    // rounds, in a fixed order: waves 4-7 hand their tiles to waves 0-3 (w
    // += w + 4), then waves 2-3 to waves 0-1 (w += w + 2); waves 0-1 park
    // their sums, and every thread adds the two for four slots, ((e0 + e4)
    // + (e2 + e6)) + ((e1 + e5) + (e3 + e7)), and stores them. Slot (tile,
    // lane) is tile 8*mt + nt.
    {
        int ce[8];
#pragma unroll
        for (int nt = 0; nt < 8; nt++) ce[nt] = ex_c[nt * 16 + li];
#pragma unroll
        for (int mt = 0; mt < 4; mt++)
#pragma unroll
            for (int rr = 0; rr < 4; rr++) {
                const int re = ex_r[mt * 16 + 4 * lq + rr][kw];
#pragma unroll
                for (int nt = 0; nt < 8; nt++) acc[mt][nt][rr] = __builtin_ldexpf(acc[mt][nt][rr], -(re + ce[nt]));
            }
    }
    auto park = [&](int s) {
#pragma unroll
        for (int mt = 0; mt < 4; mt++)
#pragma unroll
            for (int nt = 0; nt < 8; nt++) part[s][mt * 8 + nt][l] = acc[mt][nt];
    };
    auto take = [&](int s) {
#pragma unroll
        for (int mt = 0; mt < 4; mt++)
#pragma unroll
            for (int nt = 0; nt < 8; nt++) {
                const floatx4 o = part[s][mt * 8 + nt][l];
#pragma unroll
                for (int rr = 0; rr < 4; rr++) acc[mt][nt][rr] = acc[mt][nt][rr] + o[rr];
            }
    };
    if (kw >= 4) park(kw - 4);
    __syncthreads();
    if (kw < 4) take(kw);
    __syncthreads();
    if (kw == 2 || kw == 3) park(kw - 2);
    __syncthreads();
    if (kw < 2) take(kw);
    __syncthreads();
    if (kw < 2) park(kw);
    __syncthreads();
    const floatx4 *pf = &part[0][0][0];
    constexpr int kSlots = 32 * 64;                     // accumulator slots per partial tile
#pragma unroll
    for (int k = 0; k < kSlots / kThreads; k++) {
        const int f = static_cast<int>(threadIdx.x) + k * kThreads;
        const floatx4 a0 = pf[f], a1 = pf[kSlots + f];
        floatx4 v;
#pragma unroll
        for (int rr = 0; rr < 4; rr++) v[rr] = a0[rr] + a1[rr];
        const int sl = f % 64, tile = f / 64;
        const int64_t n = tn * kTN + (tile % 8) * 16 + sl % 16;
        const int64_t m0 = tm * kTM + (tile / 8) * 16 + 4 * (sl / 16);
        if (n >= N) continue;
#pragma unroll
        for (int rr = 0; rr < 4; rr++) {
            const int64_t m = m0 + rr;
            if (m < M) y[m * N + n] = v[rr];
        }
    }
}

int workspace_size(int64_t M, int64_t N, int64_t K, int64_t *bytes) {
    const int64_t m16 = (M + 15) / 16, G2 = (K / 32 + 1) / 2;
    int64_t a, b, c, d;
    GD_REQUIRE(gd::mul_ok(m16 * 16, K, &a) && gd::mul_ok(a, 4, &b) && gd::mul_ok(G2, N, &c) &&
                   gd::mul_ok(c, 16, &d),
               GD_ERANGE, "workspace size overflows");
    int64_t e;
    GD_REQUIRE(gd::mul_ok(N, 4, &e), GD_ERANGE, "workspace size overflows");
    // split activations, row exponents, packed weights, output exponents
    *bytes = b + m16 * 16 * 4 * kKParts + d + e;
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

// Packed weights: the table kernels' section (16 bytes per output and group
// pair), the matrix-core section (as many), then one exponent per output.
int packed_size(int64_t N, int64_t K, int64_t *bytes, int64_t *section = nullptr) {
    int64_t c, sec;
    GD_REQUIRE(gd::mul_ok((K / 32 + 1) / 2, N, &c) && gd::mul_ok(c, 16, &sec) && sec <= INT64_MAX / 4, GD_ERANGE,
               "packed weight size overflows");
    if (section) *section = sec;
    *bytes = 2 * sec + 4 * N;
    return GD_OK;
}

// Launches split + GEMM against weights already in the matrix-core layout.
int split_and_gemm(const float *x, const u32x2 *wb, const int32_t *cexp, float *y, int64_t M, int64_t N, int64_t K,
                   void *workspace, hipStream_t s, const char *who, bool split_done = false) {
    const int64_t G = K / 32;
    const int64_t m16 = (M + 15) / 16;
    uint32_t *xs = static_cast<uint32_t *>(workspace);
    int32_t *rexp = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + m16 * 16 * K * 4);
    const int64_t tiles_m = (M + kTM - 1) / kTM, tiles_n = (N + kTN - 1) / kTN;
    const int64_t tiles = tiles_m * tiles_n;
    const int64_t per_xcd = (tiles + 7) / 8;
    GD_REQUIRE(per_xcd * 8 <= INT64_C(0xffffffff), GD_ERANGE, "%s: grid too large", who);
    GD_REQUIRE(m16 * kParts <= INT64_C(0xffffffff), GD_ERANGE, "%s: grid too large", who);
    if (!split_done)
        hipLaunchKernelGGL(sign_split_kernel, dim3(static_cast<uint32_t>(m16 * kParts)), dim3(kPrepThreads), 0, s, x,
                           M, K, xs, rexp);
    hipLaunchKernelGGL(sign_gemm_kernel, dim3(static_cast<uint32_t>(per_xcd * 8)), dim3(kThreads), 0, s, xs, rexp,
                       wb, cexp, y, M, N, G, tiles_n, tiles, per_xcd);
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
    int64_t total, sec;
    st = packed_size(N, K, &total, &sec);
    if (st) return st;
    const int64_t wpack_x = (N + kPackRows - 1) / kPackRows, wpack_y = (G + kPackGroups - 1) / kPackGroups;
    const int64_t bpack = (N + kBpCols - 1) / kBpCols;
    GD_REQUIRE(wpack_x <= INT64_C(0xffffffff) && wpack_y <= 65535 && bpack <= INT64_C(0xffffffff), GD_ERANGE,
               "q1_sign_pack: grid too large");
    char *base = static_cast<char *>(w_packed);
    hipLaunchKernelGGL(sign_wpack_kernel, dim3(static_cast<uint32_t>(wpack_x), static_cast<uint32_t>(wpack_y)),
                       dim3(kPrepThreads), 0, as_stream(stream), w_bits, w_scales, N, G, reinterpret_cast<u32x4 *>(base));
    hipLaunchKernelGGL(sign_bpack_kernel, dim3(static_cast<uint32_t>(bpack)), dim3(kPrepThreads), 0,
                       as_stream(stream), w_bits, w_scales, N, G, reinterpret_cast<u32x2 *>(base + sec),
                       reinterpret_cast<int32_t *>(base + 2 * sec));
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
    need += m16 * 16 * 4 * kKParts;   // split activations and row exponents; no weight part
    GD_REQUIRE(workspace_bytes >= static_cast<size_t>(need), GD_ERANGE,
               "q1_sign_gemm_packed: workspace of %zu bytes, %lld needed", workspace_bytes, (long long)need);
    int64_t total, sec;
    st = packed_size(N, K, &total, &sec);
    if (st) return st;
    const char *base = static_cast<const char *>(w_packed);
    return split_and_gemm(x, reinterpret_cast<const u32x2 *>(base + sec),
                          reinterpret_cast<const int32_t *>(base + 2 * sec), y, M, N, K, workspace,
                          as_stream(stream), "q1_sign_gemm_packed");
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
    const int64_t m16 = (M + 15) / 16;
    const int64_t G2 = (K / 32 + 1) / 2;
    char *base = static_cast<char *>(workspace);
    const int64_t xs_bytes = m16 * 16 * K * 4, rexp_bytes = m16 * 16 * 4 * kKParts;
    u32x2 *wb = reinterpret_cast<u32x2 *>(base + xs_bytes + rexp_bytes);
    int32_t *cexp = reinterpret_cast<int32_t *>(base + xs_bytes + rexp_bytes + 16 * G2 * N);
    const int64_t n_split = m16 * kParts;
    const int64_t n_prep = n_split + (N + kBpCols - 1) / kBpCols;
    GD_REQUIRE(n_prep <= INT64_C(0xffffffff), GD_ERANGE, "q1_sign_gemm: grid too large");
    hipStream_t s = as_stream(stream);
    uint32_t *xs = reinterpret_cast<uint32_t *>(base);
    int32_t *rexp = reinterpret_cast<int32_t *>(base + m16 * 16 * K * 4);
    hipLaunchKernelGGL(sign_prep_kernel, dim3(static_cast<uint32_t>(n_prep)), dim3(kPrepThreads), 0, s, x, M, K, xs,
                       rexp, n_split, w_bits, w_scales, N, wb, cexp);
    return split_and_gemm(x, wb, cexp, y, M, N, K, workspace, s, "q1_sign_gemm", true);
}
