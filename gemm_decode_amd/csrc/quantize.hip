// quantize.hip -- on-device activation quantization, the step before each
// GEMV: f32 -> q8_0 blocks for the Q1 path, and f32 -> per-token int8
// codes, delivered as the eight bit planes the ternary GEMV reads, plus
// their scale.
//
// The rule is the page "web-xpu-ops" operator "quantize" (absmax to int8,
// symmetric in [-127, 127]) with the reciprocal and rounding its q4 format
// table states for the same convention: 127/absmax formed in f64, and
// Math.round (ties toward +infinity) of x * (127/absmax), evaluated as
// floor(v) + (v - floor(v) >= 0.5) in f64. The scale is absmax/127 (f64
// quotient rounded to f32). For q8_0 (page "browseml-gpu.js", packQ8: f16 d,
// then 32 int8 codes) the same rule is applied per block of 32, with d the
// f16 rounding (nearest even) of that f32 scale. Every decision is made in
// f64 exactly as written, so codes and scales are bit-exact with any IEEE
// evaluation of the same steps. Inputs must be finite.
#include "gd_internal.h"

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int32_t round_code(double v) {
    const double f = floor(v);
    double q = f + ((v - f) >= 0.5 ? 1.0 : 0.0);
    q = q > 127.0 ? 127.0 : q;
    q = q < -127.0 ? -127.0 : q;
    return static_cast<int32_t>(q);
}

__device__ __forceinline__ float absmax4(const float4 &v) {
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// ----------------------------------------------------------------- q8_0
// Eight lanes per 32-element block (one float4 each); the block's absmax
// meets over the eight lanes, each lane writes its four codes as two 16-bit
// stores (a 34-byte block is only 2-byte aligned) and lane 0 writes d.
__global__ __launch_bounds__(kThreads) void q8_0_quantize_kernel(const float4 *__restrict__ x,
                                                                 uint16_t *__restrict__ out, int64_t nblocks) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const int64_t blk = gid >> 3;
    const int part = static_cast<int>(threadIdx.x & 7);
    if (blk >= nblocks) return;   // all eight lanes of a block leave together
    const float4 v = x[blk * 8 + part];
    float m = absmax4(v);
    m = fmaxf(m, __shfl_xor(m, 1, 8));
    m = fmaxf(m, __shfl_xor(m, 2, 8));
    m = fmaxf(m, __shfl_xor(m, 4, 8));
    const double amax = static_cast<double>(m);
    uint32_t packed = 0;
    uint16_t d = 0;
    if (amax > 0.0) {
        const double inv = 127.0 / amax;
        const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; j++)
            packed |= (static_cast<uint32_t>(round_code(static_cast<double>(e[j]) * inv)) & 0xffu) << (8 * j);
        d = __builtin_bit_cast(uint16_t, static_cast<_Float16>(static_cast<float>(amax / 127.0)));
    }
    uint16_t *o = out + blk * 17;   // 34 bytes = 17 halves
    o[1 + 2 * part] = static_cast<uint16_t>(packed & 0xffffu);
    o[2 + 2 * part] = static_cast<uint16_t>(packed >> 16);
    if (part == 0) o[0] = d;
}

// ------------------------------------------------------- per-token int8
// One workgroup (four waves) per token. Stripe s holds elements 64s..64s+63;
// wave w owns stripes wR .. wR+R-1 (K <= 256 R). Each lane loads its
// element of each of its stripes at once, the token's absmax meets through
// the waves and LDS, and each stripe's codes give, by eight ballots, its two
// words of every plane (plane b, word m, bit j = bit b of the two's-
// complement code of element 32m + j). The words are gathered into one
// register per plane (lane 2i+h takes word h of stripe i) and each plane's
// run of 2R words is written by one coalesced store. Past K the lanes vote
// 0, and words past K/32 are not written.
__device__ __forceinline__ float token_absmax(float m, float *red, int wave, int lane) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (lane == 0) red[wave] = m;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

template <int R>
__global__ __launch_bounds__(kThreads) void act_quant_kernel(const float *__restrict__ x,
                                                             uint32_t *__restrict__ planes,
                                                             float *__restrict__ scale, int64_t K) {
    static_assert(2 * R <= 64, "a plane's words of one wave fit one register");
    __shared__ float red[kThreads / 64];
    const int64_t c = blockIdx.x;
    const float *xr = x + c * K;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int64_t s0 = static_cast<int64_t>(wave) * R;
    float v[R];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < R; i++) {
        const int64_t e = (s0 + i) * 64 + lane;
        v[i] = xr[e < K ? e : K - 1];   // clamped: every load issued, the extra ones unused
        if (e < K) m = fmaxf(m, fabsf(v[i]));
    }
    const double amax = static_cast<double>(token_absmax(m, red, wave, lane));
    const double inv = amax > 0.0 ? 127.0 / amax : 0.0;
    if (threadIdx.x == 0) scale[c] = amax > 0.0 ? static_cast<float>(amax / 127.0) : 0.0f;
    uint32_t pw[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < R; i++) {
        if ((s0 + i) * 64 < K) {   // uniform per wave
            const int64_t e = (s0 + i) * 64 + lane;
            const int32_t q = (e < K) ? round_code(static_cast<double>(v[i]) * inv) : 0;
            const uint32_t u = static_cast<uint32_t>(q) & 0xffu;
            const bool lo_here = lane == 2 * i, hi_here = lane == 2 * i + 1;
#pragma unroll
            for (int b = 0; b < 8; b++) {
                const uint64_t mb = __ballot((u >> b) & 1u);
                pw[b] = lo_here ? static_cast<uint32_t>(mb) : pw[b];
                pw[b] = hi_here ? static_cast<uint32_t>(mb >> 32) : pw[b];
            }
        }
    }
    const int64_t W = K / 32;
    const int64_t w0 = 2 * s0;   // this wave's first word of each plane
    if (lane < 2 * R && w0 + lane < W) {
        uint32_t *pl = planes + c * 8 * W + w0 + lane;
#pragma unroll
        for (int b = 0; b < 8; b++) pl[b * W] = pw[b];
    }
}

// One stripe's two words of every plane, written by the lanes b that hold
// plane b's ballot.
__device__ __forceinline__ void stripe_planes(uint32_t *pl, int64_t W, int64_t s, int lane, int32_t q) {
    const uint32_t u = static_cast<uint32_t>(q) & 0xffu;
#pragma unroll
    for (int b = 0; b < 8; b++) {
        const uint64_t mb = __ballot((u >> b) & 1u);
        if (lane == b) {
            pl[b * W + 2 * s] = static_cast<uint32_t>(mb);
            if (2 * s + 1 < W) pl[b * W + 2 * s + 1] = static_cast<uint32_t>(mb >> 32);
        }
    }
}

// Tokens longer than 256 * 32 elements: the same steps with a second read
// and one stripe of stores at a time.
__global__ __launch_bounds__(kThreads) void act_quant_long_kernel(const float *__restrict__ x,
                                                                  uint32_t *__restrict__ planes,
                                                                  float *__restrict__ scale, int64_t K) {
    __shared__ float red[kThreads / 64];
    const int64_t c = blockIdx.x;
    const float *xr = x + c * K;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    float m = 0.0f;
    const float4 *x4 = reinterpret_cast<const float4 *>(xr);
    for (int64_t i = threadIdx.x; i < K / 4; i += kThreads) m = fmaxf(m, absmax4(x4[i]));
    const double amax = static_cast<double>(token_absmax(m, red, wave, lane));
    const double inv = amax > 0.0 ? 127.0 / amax : 0.0;
    if (threadIdx.x == 0) scale[c] = amax > 0.0 ? static_cast<float>(amax / 127.0) : 0.0f;
    const int64_t W = K / 32;
    uint32_t *pl = planes + c * 8 * W;
    for (int64_t s = wave; s * 64 < K; s += kThreads / 64) {   // uniform per wave
        const int64_t e = s * 64 + lane;
        stripe_planes(pl, W, s, lane, (e < K) ? round_code(static_cast<double>(xr[e]) * inv) : 0);
    }
}

}  // namespace

using namespace gd;

extern "C" int q8_0_quantize(const float *x, void *a_q8, int64_t n, int64_t K, void *stream) {
    GD_REQUIRE(x && a_q8, GD_EINVAL, "q8_0_quantize: null pointer");
    GD_REQUIRE(n >= 1 && K >= 1, GD_EINVAL, "q8_0_quantize: n (%lld) and K (%lld) must be >= 1", (long long)n,
               (long long)K);
    GD_REQUIRE(K % 32 == 0, GD_ESHAPE, "q8_0_quantize: K (%lld) must be a multiple of 32", (long long)K);
    GD_REQUIRE(aligned(x, 16), GD_EALIGN, "q8_0_quantize: x must be 16-byte aligned");
    GD_REQUIRE(aligned(a_q8, 2), GD_EALIGN, "q8_0_quantize: a_q8 must be 2-byte aligned");
    int64_t nblocks;
    GD_REQUIRE(mul_ok(n, K / 32, &nblocks) && nblocks <= (INT64_C(1) << 34), GD_ERANGE,
               "q8_0_quantize: n * K too large");
    const int64_t grid = (nblocks * 8 + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(q8_0_quantize_kernel, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0, as_stream(stream),
                       reinterpret_cast<const float4 *>(x), static_cast<uint16_t *>(a_q8), nblocks);
    return check_launch("q8_0_quantize");
}

extern "C" int ternary_quantize_act(const float *x, int64_t count, int64_t K, uint32_t *planes, float *x_scale,
                                    void *stream) {
    GD_REQUIRE(x && planes && x_scale, GD_EINVAL, "ternary_quantize_act: null pointer");
    GD_REQUIRE(count >= 1 && K >= 1, GD_EINVAL, "ternary_quantize_act: count (%lld) and K (%lld) must be >= 1",
               (long long)count, (long long)K);
    GD_REQUIRE(K % 32 == 0, GD_ESHAPE, "ternary_quantize_act: K (%lld) must be a multiple of 32", (long long)K);
    GD_REQUIRE(count <= INT64_C(2147483647) && K <= (INT64_C(1) << 30), GD_ERANGE,
               "ternary_quantize_act: count or K too large");
    GD_REQUIRE(aligned(x, 16), GD_EALIGN, "ternary_quantize_act: x must be 16-byte aligned");
    GD_REQUIRE(aligned(planes, 4) && aligned(x_scale, 4), GD_EALIGN,
               "ternary_quantize_act: planes and x_scale must be 4-byte aligned");
    const dim3 grid(static_cast<uint32_t>(count)), block(kThreads);
    hipStream_t hs = as_stream(stream);
    const int64_t per_lane = (K + kThreads - 1) / kThreads;   // elements each lane holds
    if (per_lane <= 4)
        hipLaunchKernelGGL(act_quant_kernel<4>, grid, block, 0, hs, x, planes, x_scale, K);
    else if (per_lane <= 8)
        hipLaunchKernelGGL(act_quant_kernel<8>, grid, block, 0, hs, x, planes, x_scale, K);
    else if (per_lane <= 16)
        hipLaunchKernelGGL(act_quant_kernel<16>, grid, block, 0, hs, x, planes, x_scale, K);
    else if (per_lane <= 32)
        hipLaunchKernelGGL(act_quant_kernel<32>, grid, block, 0, hs, x, planes, x_scale, K);
    else
        hipLaunchKernelGGL(act_quant_long_kernel, grid, block, 0, hs, x, planes, x_scale, K);
    return check_launch("ternary_quantize_act");
}
