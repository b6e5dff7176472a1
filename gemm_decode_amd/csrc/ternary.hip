// ternary.hip -- ternary bitplane GEMV on gfx950 (page "BonsaiのWebGPU
// カーネルを読み解く", section on Bonsai: P/N bitplanes and the popcount
// identity dot = 2(pc(P&X) - pc(N&X)) - pc(P) + pc(N) for a binary plane X).
//
// int8 activations enter as their eight two's-complement bit planes B_b
// (x = sum_{b<7} 2^b B_b - 128 B_7). Per plane the identity's difference
// pc(P&B) - pc(N&B) equals pc((P&B) | (N&~B)) - pc(N) when P&N = 0, and
// (P&B) | (N&~B) is one v_bfi_b32; summing c_b = 2^b (b<7), c_7 = -128 over
// planes (sum c_b = -1) gives
//     dot = sum_b c_b * pc(bfi(B_b, P, N)) + pc(N),
// i.e. one bit-select and one popcount-accumulate per plane per 32 weights.
// An element with P and N both set contributes 0 here, as in w = P - N.
//
// Mapping (general kernel; the held-row kernel below covers K % 128 == 0,
// K <= 8192 with all of a lane's loads issued at once). Eight lanes share a
// row and split its K range in 16-byte pieces
// (integer sums are associative, so the split is exact); a wave covers eight
// rows and reads 128 contiguous bytes of each. The activation planes are
// copied once per workgroup into LDS, where the eight lanes of a row read
// eight consecutive 16-byte pieces and the eight rows of a wave read the same
// addresses (broadcast).
#include "gd_device.h"
#include "gd_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerRow = 8;
constexpr int kRowsPerPass = kThreads / kLanesPerRow;   // 32
constexpr int kPasses = 4;                              // rows per WG = 128
constexpr int kRowsPerWG = kRowsPerPass * kPasses;

// ------------------------------------------------------------ bit planes
// One thread per (vector, 32-element word): plane b word m = bit b of the
// bytes x[32m .. 32m+31], element 32m+j at bit j.
// bit 8j + b of x -> bit 4b + j: nibble b of the result holds bit b of the
// word's four bytes, in byte order (four delta swaps of the 5-bit bit index).
__device__ __forceinline__ uint32_t bytes_to_nibbles(uint32_t x) {
    uint32_t t;
    t = (x ^ (x >> 12)) & 0x0000F0F0u;
    x ^= t ^ (t << 12);
    t = (x ^ (x >> 6)) & 0x00CC00CCu;
    x ^= t ^ (t << 6);
    t = (x ^ (x >> 3)) & 0x0A0A0A0Au;
    x ^= t ^ (t << 3);
    t = (x ^ (x >> 1)) & 0x22222222u;
    x ^= t ^ (t << 1);
    return x;
}

// One plane word per thread: its 32 codes are 8 words of 4 bytes; each word
// turns into 8 nibbles (bit b of its four codes in nibble b), then an 8 x 8
// transpose of those nibbles across the 8 registers (three swap stages)
// leaves plane b's word, bit j = bit b of code j, in register b.
__global__ void act_bitplanes_kernel(const int8_t *__restrict__ x, uint32_t *__restrict__ planes, int64_t count,
                                     int64_t W) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (gid >= count * W) return;
    const int64_t v = gid / W, m = gid % W;
    const uint4 *src = reinterpret_cast<const uint4 *>(x + (v * W + m) * 32);
    const uint4 lo = src[0], hi = src[1];
    uint32_t r[8] = {bytes_to_nibbles(lo.x), bytes_to_nibbles(lo.y), bytes_to_nibbles(lo.z), bytes_to_nibbles(lo.w),
                     bytes_to_nibbles(hi.x), bytes_to_nibbles(hi.y), bytes_to_nibbles(hi.z), bytes_to_nibbles(hi.w)};
    constexpr uint32_t kMask[3] = {0x0F0F0F0Fu, 0x00FF00FFu, 0x0000FFFFu};
#pragma unroll
    for (int st = 0; st < 3; st++) {
        const int d = 1 << st, sh = 4 << st;
#pragma unroll
        for (int q = 0; q < 8; q++) {
            if (q & d) continue;
            const uint32_t t = ((r[q] >> sh) ^ r[q + d]) & kMask[st];
            r[q + d] ^= t;
            r[q] ^= t << sh;
        }
    }
    uint32_t *dst = planes + v * 8 * W + m;
#pragma unroll
    for (int b = 0; b < 8; b++) dst[b * W] = r[b];
}

// --------------------------------------------------------------- GEMV
struct TernArgs {
    const uint32_t *P, *N, *X;
    float *y;
    int32_t *dot;
    float w_scale, x_scale;
    const float *xs_dev;  // device activation scale (read in place of x_scale), or null
};

// Per-lane partial counts over words [w0, w0+4): cnt[b] += pc(bfi(B_b, P, N)),
// cn += pc(N).
__device__ __forceinline__ void count4(const uint4 &p4, const uint4 &n4, const uint32_t *xl, int64_t W4,
                                       int64_t w0, uint32_t cnt[8], uint32_t &cn) {
    const uint32_t p[4] = {p4.x, p4.y, p4.z, p4.w};
    const uint32_t n[4] = {n4.x, n4.y, n4.z, n4.w};
#pragma unroll
    for (int b = 0; b < 8; b++) {
        const uint4 x4 = *reinterpret_cast<const uint4 *>(xl + b * W4 + w0);
        const uint32_t xb[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
        for (int q = 0; q < 4; q++) cnt[b] += __builtin_popcount((p[q] & xb[q]) | (n[q] & ~xb[q]));
    }
#pragma unroll
    for (int q = 0; q < 4; q++) cn += __builtin_popcount(n[q]);
}

__device__ __forceinline__ void ternary_body(const TernArgs &a, uint32_t *xl, int64_t rows, int64_t W) {
    const int64_t W4 = (W + 3) / 4 * 4;
    const float x_scale = a.xs_dev ? *a.xs_dev : a.x_scale;
    // stage the planes (zero-padded to a multiple of 4 words) into LDS
    for (int64_t i = threadIdx.x; i < 8 * W4; i += kThreads) {
        const int64_t b = i / W4, m = i % W4;
        xl[i] = (m < W) ? a.X[b * W + m] : 0u;
    }
    __syncthreads();
    const int lane = threadIdx.x % kLanesPerRow;
    const int rsub = threadIdx.x / kLanesPerRow;
    const bool vec = (W % 4) == 0;
    for (int pass = 0; pass < kPasses; pass++) {
        const int64_t r = static_cast<int64_t>(blockIdx.x) * kRowsPerWG + pass * kRowsPerPass + rsub;
        uint32_t cnt[8] = {0, 0, 0, 0, 0, 0, 0, 0}, cn = 0;
        if (r < rows) {
            const uint32_t *Pr = a.P + r * W, *Nr = a.N + r * W;
            if (vec) {
                for (int64_t w0 = 4 * lane; w0 < W; w0 += 4 * kLanesPerRow) {
                    const uint4 p4 = *reinterpret_cast<const uint4 *>(Pr + w0);
                    const uint4 n4 = *reinterpret_cast<const uint4 *>(Nr + w0);
                    count4(p4, n4, xl, W4, w0, cnt, cn);
                }
            } else {
                for (int64_t w0 = 4 * lane; w0 < W; w0 += 4 * kLanesPerRow) {
                    uint32_t pw[4], nw[4];
                    for (int q = 0; q < 4; q++) {
                        pw[q] = (w0 + q < W) ? Pr[w0 + q] : 0u;
                        nw[q] = (w0 + q < W) ? Nr[w0 + q] : 0u;
                    }
                    count4(make_uint4(pw[0], pw[1], pw[2], pw[3]), make_uint4(nw[0], nw[1], nw[2], nw[3]), xl, W4,
                           w0, cnt, cn);
                }
            }
        }
        int32_t part = static_cast<int32_t>(cn) - 128 * static_cast<int32_t>(cnt[7]);
#pragma unroll
        for (int b = 0; b < 7; b++) part += static_cast<int32_t>(cnt[b]) << b;
        // sum over the 8 lanes of the row (exact integer adds)
        part += __shfl_xor(part, 1, kLanesPerRow);
        part += __shfl_xor(part, 2, kLanesPerRow);
        part += __shfl_xor(part, 4, kLanesPerRow);
        if (lane == 0 && r < rows) {
            const float s = a.w_scale * x_scale;
            a.y[r] = static_cast<float>(part) * s;
            if (a.dot) a.dot[r] = part;
        }
    }
}

__global__ __launch_bounds__(kThreads) void ternary_gemv_kernel(TernArgs a, int64_t rows, int64_t W) {
    extern __shared__ __align__(16) uint32_t xl[];
    ternary_body(a, xl, rows, W);
}

__device__ __forceinline__ TernArgs problem_args(const gd_ternary_problem &pr) {
    return TernArgs{pr.w_pos, pr.w_neg, pr.x_planes, pr.y, pr.dot_out, pr.w_scale, pr.x_scale, pr.x_scale_dev};
}

__global__ __launch_bounds__(kThreads) void ternary_gemv_grouped_kernel(const gd_ternary_problem *probs,
                                                                        int64_t rows, int64_t W) {
    extern __shared__ __align__(16) uint32_t xl[];
    ternary_body(problem_args(probs[blockIdx.y]), xl, rows, W);
}

// ----------------------------------------------------- held-row GEMV
// For K % 128 == 0 and K <= 8192 (NIT = K/1024 rounded up <= 8 sixteen-byte
// pieces per lane): a workgroup of kHeldThreads covers kHeldRows rows in one
// pass, eight lanes per row, and every lane issues the loads of all its
// pieces of P and N before counting, so a wave keeps 2*NIT 1 KiB loads in
// flight. Pieces past the row end read a clamped (valid) address and count
// as zero words.
constexpr int kHeldThreads = 512;
constexpr int kHeldRows = kHeldThreads / kLanesPerRow;   // 64
constexpr int kHeldMaxIt = 8;
// The weight planes take streaming (non-temporal) loads up to this many
// pieces per lane: measured faster at K = 2560 (3 pieces), slower at
// K = 6912 (7 pieces).
constexpr int kHeldStreamMaxIt = 4;
constexpr size_t kHeldStage = kHeldThreads * 16;   // LDS: one 16-byte plane piece per thread (8W*4 <= this)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef const u32x4 __attribute__((address_space(1))) *g_u4;

// The planes (8W words = 2W sixteen-byte pieces, one per thread) are
// loaded first: loads complete in the order they are issued, so the LDS
// stage waits only for the plane load and runs while the weights are still
// in flight.
typedef const float __attribute__((address_space(1))) *g_f32;

template <int NIT>
__device__ __forceinline__ void ternary_held_body(const TernArgs &a, uint32_t *xl, int64_t rows, int64_t W) {
    const int lane = threadIdx.x % kLanesPerRow;
    const int rsub = threadIdx.x / kLanesPerRow;
    const int64_t r = static_cast<int64_t>(blockIdx.x) * kHeldRows + rsub;
    const int64_t rc = r < rows ? r : rows - 1;                 // clamped: loads valid, never stored
    const g_u4 Pr = (g_u4)(a.P + rc * W), Nr = (g_u4)(a.N + rc * W);
    const int64_t np = 2 * W;                                   // plane pieces, <= kHeldThreads
    const u32x4 xw = ((g_u4)a.X)[threadIdx.x < np ? threadIdx.x : np - 1];
    u32x4 pv[NIT], nv[NIT];
#pragma unroll
    for (int it = 0; it < NIT; it++) {                          // all weight loads next
        int64_t w4 = lane + kLanesPerRow * it;                  // 16-byte piece index in the row
        w4 = w4 < W / 4 ? w4 : W / 4 - 1;
        if constexpr (NIT <= kHeldStreamMaxIt) {
            pv[it] = gd::ld_stream(&Pr[w4]);
            nv[it] = gd::ld_stream(&Nr[w4]);
        } else {
            pv[it] = Pr[w4];
            nv[it] = Nr[w4];
        }
    }
    // the device scale, if any, is loaded last (it lands with the weights);
    // the address is always valid and the value used only when set
    const float xs = *(g_f32)(a.xs_dev ? a.xs_dev : reinterpret_cast<const float *>(a.X));
    // every thread stores its piece: those past the 2W planes land in the
    // stage's padding (kHeldStage bytes), so the load stays ahead of the weights'
    *reinterpret_cast<u32x4 *>(xl + 4 * threadIdx.x) = xw;
    const float x_scale = a.xs_dev ? xs : a.x_scale;
    __syncthreads();
    uint32_t cnt[8] = {0, 0, 0, 0, 0, 0, 0, 0}, cn = 0;
#pragma unroll
    for (int it = 0; it < NIT; it++) {
        const int64_t w0 = 4 * (lane + kLanesPerRow * it);
        const bool live = w0 < W;
        const u32x4 p4 = live ? pv[it] : u32x4{0u, 0u, 0u, 0u};
        const u32x4 n4 = live ? nv[it] : u32x4{0u, 0u, 0u, 0u};
        const int64_t wx = live ? w0 : 0;
#pragma unroll
        for (int b = 0; b < 8; b++) {
            const uint4 x4 = *reinterpret_cast<const uint4 *>(xl + b * W + wx);
            const uint32_t xb[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
            for (int q = 0; q < 4; q++) cnt[b] += __builtin_popcount((p4[q] & xb[q]) | (n4[q] & ~xb[q]));
        }
#pragma unroll
        for (int q = 0; q < 4; q++) cn += __builtin_popcount(n4[q]);
    }
    int32_t part = static_cast<int32_t>(cn) - 128 * static_cast<int32_t>(cnt[7]);
#pragma unroll
    for (int b = 0; b < 7; b++) part += static_cast<int32_t>(cnt[b]) << b;
    part += __shfl_xor(part, 1, kLanesPerRow);
    part += __shfl_xor(part, 2, kLanesPerRow);
    part += __shfl_xor(part, 4, kLanesPerRow);
    if (lane == 0 && r < rows) {
        const float s = a.w_scale * x_scale;
        a.y[r] = static_cast<float>(part) * s;
        if (a.dot) a.dot[r] = part;
    }
}

template <int NIT>
__global__ __launch_bounds__(kHeldThreads) void ternary_held_kernel(TernArgs a, int64_t rows, int64_t W) {
    extern __shared__ __align__(16) uint32_t xl[];
    ternary_held_body<NIT>(a, xl, rows, W);
}

template <int NIT>
__global__ __launch_bounds__(kHeldThreads) void ternary_held_grouped_kernel(const gd_ternary_problem *probs,
                                                                            int64_t rows, int64_t W) {
    extern __shared__ __align__(16) uint32_t xl[];
    ternary_held_body<NIT>(problem_args(probs[blockIdx.y]), xl, rows, W);
}

// Launch the held-row kernel for W = K/32 (W % 4 == 0, W <= 256); false if
// the shape does not qualify. `probs` null: the single-problem form with `a`;
// else the problem-array form.
template <int NIT>
void launch_held_n(const TernArgs &a, const gd_ternary_problem *probs, int64_t count, int64_t rows, int64_t W,
                   hipStream_t st) {
    const dim3 grid(static_cast<uint32_t>((rows + kHeldRows - 1) / kHeldRows), static_cast<uint32_t>(count));
    if (probs)
        hipLaunchKernelGGL(ternary_held_grouped_kernel<NIT>, grid, dim3(kHeldThreads), kHeldStage, st, probs, rows,
                           W);
    else
        hipLaunchKernelGGL(ternary_held_kernel<NIT>, grid, dim3(kHeldThreads), kHeldStage, st, a, rows, W);
}

bool launch_held(const TernArgs &a, const gd_ternary_problem *probs, int64_t count, int64_t rows, int64_t W,
                 hipStream_t st) {
    if (W % 4 != 0 || W > 32 * kHeldMaxIt) return false;
    switch ((W + 31) / 32) {
        case 1: launch_held_n<1>(a, probs, count, rows, W, st); return true;
        case 2: launch_held_n<2>(a, probs, count, rows, W, st); return true;
        case 3: launch_held_n<3>(a, probs, count, rows, W, st); return true;
        case 4: launch_held_n<4>(a, probs, count, rows, W, st); return true;
        case 5: launch_held_n<5>(a, probs, count, rows, W, st); return true;
        case 6: launch_held_n<6>(a, probs, count, rows, W, st); return true;
        case 7: launch_held_n<7>(a, probs, count, rows, W, st); return true;
        case 8: launch_held_n<8>(a, probs, count, rows, W, st); return true;
        default: return false;
    }
}

int check_shape(int64_t rows, int64_t K) {
    GD_REQUIRE(rows >= 1 && K >= 1, GD_EINVAL, "rows (%lld) and K (%lld) must be >= 1", (long long)rows,
               (long long)K);
    GD_REQUIRE(K % 32 == 0, GD_ESHAPE, "K (%lld) must be a multiple of 32", (long long)K);
    GD_REQUIRE(K <= (INT64_C(1) << 17), GD_ERANGE, "K (%lld) above 2^17 (|dot| must stay below 2^24)",
               (long long)K);
    GD_REQUIRE(rows <= INT64_C(1) << 31, GD_ERANGE, "rows (%lld) above 2^31", (long long)rows);
    return GD_OK;
}

size_t lds_bytes(int64_t K) { return static_cast<size_t>(8 * ((K / 32 + 3) / 4 * 4) * 4); }

}  // namespace

using namespace gd;

extern "C" int ternary_act_bitplanes(const int8_t *x_q, int64_t count, int64_t K, uint32_t *planes,
                                     void *stream) {
    GD_REQUIRE(x_q && planes, GD_EINVAL, "ternary_act_bitplanes: null pointer");
    GD_REQUIRE(count >= 1 && K >= 1, GD_EINVAL, "ternary_act_bitplanes: count and K must be >= 1");
    GD_REQUIRE(K % 32 == 0, GD_ESHAPE, "ternary_act_bitplanes: K (%lld) must be a multiple of 32", (long long)K);
    GD_REQUIRE(count <= 65535 && K <= (INT64_C(1) << 17), GD_ERANGE, "ternary_act_bitplanes: count or K too large");
    GD_REQUIRE(aligned(x_q, 16) && aligned(planes, 16), GD_EALIGN,
               "ternary_act_bitplanes: x_q and planes must be 16-byte aligned");
    const int64_t W = K / 32, n = count * W;
    hipLaunchKernelGGL(act_bitplanes_kernel, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0,
                       as_stream(stream), x_q, planes, count, W);
    return check_launch("ternary_act_bitplanes");
}

extern "C" int ternary_gemv(const uint32_t *w_pos, const uint32_t *w_neg, float w_scale, const uint32_t *x_planes,
                            float x_scale, float *y, int32_t *dot_out, int64_t rows, int64_t K, void *stream) {
    GD_REQUIRE(w_pos && w_neg && x_planes && y, GD_EINVAL, "ternary_gemv: null pointer");
    int st = check_shape(rows, K);
    if (st) return st;
    GD_REQUIRE(aligned(w_pos, 16) && aligned(w_neg, 16) && aligned(x_planes, 16), GD_EALIGN,
               "ternary_gemv: w_pos, w_neg and x_planes must be 16-byte aligned");
    GD_REQUIRE(aligned(y, 4) && aligned(dot_out, 4), GD_EALIGN, "ternary_gemv: y/dot_out must be 4-byte aligned");
    const int64_t W = K / 32;
    const size_t lds = lds_bytes(K);
    GD_REQUIRE(lds <= 64 * 1024, GD_ERANGE, "ternary_gemv: K too large for the LDS plane stage");
    TernArgs a{w_pos, w_neg, x_planes, y, dot_out, w_scale, x_scale, nullptr};
    if (launch_held(a, nullptr, 1, rows, W, as_stream(stream))) return check_launch("ternary_gemv");
    const int64_t gx = (rows + kRowsPerWG - 1) / kRowsPerWG;
    hipLaunchKernelGGL(ternary_gemv_kernel, dim3(static_cast<uint32_t>(gx)), dim3(kThreads), lds,
                       as_stream(stream), a, rows, W);
    return check_launch("ternary_gemv");
}

extern "C" int ternary_gemv_grouped(const gd_ternary_problem *problems, int64_t count, int64_t rows, int64_t K,
                                    void *stream) {
    GD_REQUIRE(problems, GD_EINVAL, "ternary_gemv_grouped: null problems array");
    int st = check_shape(rows, K);
    if (st) return st;
    GD_REQUIRE(count >= 1, GD_EINVAL, "ternary_gemv_grouped: count (%lld) must be >= 1", (long long)count);
    GD_REQUIRE(count <= 65535, GD_ERANGE, "ternary_gemv_grouped: count (%lld) above 65535", (long long)count);
    GD_REQUIRE(aligned(problems, 8), GD_EALIGN, "ternary_gemv_grouped: problems must be 8-byte aligned");
    const int64_t W = K / 32;
    const size_t lds = lds_bytes(K);
    GD_REQUIRE(lds <= 64 * 1024, GD_ERANGE, "ternary_gemv_grouped: K too large for the LDS plane stage");
    if (launch_held(TernArgs{}, problems, count, rows, W, as_stream(stream)))
        return check_launch("ternary_gemv_grouped");
    const int64_t gx = (rows + kRowsPerWG - 1) / kRowsPerWG;
    hipLaunchKernelGGL(ternary_gemv_grouped_kernel, dim3(static_cast<uint32_t>(gx), static_cast<uint32_t>(count)),
                       dim3(kThreads), lds, as_stream(stream), problems, rows, W);
    return check_launch("ternary_gemv_grouped");
}
