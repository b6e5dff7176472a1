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
// f16 rounding (nearest even) of that f32 scale. Codes are decided in f32
// where that provably gives the f64 rule's result, and in f64 exactly as
// written everywhere else (near a tie, or when 127/absmax leaves f32's
// range), so codes and scales are bit-exact with any IEEE evaluation of the
// rule's steps. Inputs must be finite.
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

// ------------------------------------------------------ f32 decisions
// Codes are decided in f32 first: with inv32 = f32(127/absmax) and v32 = x *
// inv32 (two roundings), |v32 - v| <= 127 * 2^-23 ~ 1.5e-5 for the f64
// product v the rule rounds, so Math.round(v32) = Math.round(v) unless v32
// lies within kTieGuard of a half-integer; only those elements are decided
// again in f64 exactly as the rule states.
constexpr float kTieGuard = 6.4e-5f;   // 4x the f32 error bound above

// f32(127 / a) and f32(a / 127) for a finite f32 a > 0, correctly rounded
// f32 divisions. They equal the f64 quotients rounded to f32 (the rule's
// order): an f32 midpoint is never within 2^-49 (relative) of either exact
// quotient, far beyond f64's rounding, so rounding twice cannot differ.
__device__ __forceinline__ float recip127(float a) { return 127.0f / a; }
__device__ __forceinline__ float scale_of(float a) { return a / 127.0f; }

// Four codes, byte j of the result the code of element j. A code is
// floor(v32 + 0.5) for v32 = x * inv32: outside kTieGuard of a half-integer
// that is Math.round of the f64 product (v32 + 0.5 rounds by at most 2^-17
// for |v32| < 128, and |v32| <= 127 + 2^-16 keeps it in [-127, 127] without
// a clamp). A lane with any of its codes near a tie, or whose reciprocal
// overflowed f32 (f64_only), decides its four codes again in f64 exactly as
// the rule states.
__device__ __forceinline__ uint32_t codes4(const float4 &v, float inv32, float absmax, bool f64_only) {
    const float e[4] = {v.x, v.y, v.z, v.w};
    int32_t q[4];
    bool exact = f64_only;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const float t = e[j] * inv32;
        q[j] = static_cast<int32_t>(floorf(t + 0.5f));
        exact |= fabsf(__builtin_amdgcn_fractf(t) - 0.5f) < kTieGuard;
    }
    if (exact) {   // rare
        const double inv = 127.0 / static_cast<double>(absmax);
#pragma unroll
        for (int j = 0; j < 4; j++) q[j] = round_code(static_cast<double>(e[j]) * inv);
    }
    uint32_t packed = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) packed |= (static_cast<uint32_t>(q[j]) & 0xffu) << (8 * j);
    return packed;
}

// ----------------------------------------------------------------- q8_0
// Eight lanes per 32-element block (one float4 each); the block's absmax
// meets over the eight lanes (three DPP steps), each lane writes its four
// codes (codes4) as two 16-bit stores (a 34-byte block is only 2-byte
// aligned) and lane 0 writes d.
__device__ __forceinline__ float max8(float v) {   // max over the 8 lanes of a half-row
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
    return v;
}

__global__ __launch_bounds__(kThreads) void q8_0_quantize_kernel(const float4 *__restrict__ x,
                                                                 uint16_t *__restrict__ out, int64_t nblocks) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const int64_t blk = gid >> 3;
    const int part = static_cast<int>(threadIdx.x & 7);
    if (blk >= nblocks) return;   // all eight lanes of a block leave together (blocks are 8-lane aligned)
    const float4 v = x[blk * 8 + part];
    const float m = max8(absmax4(v));
    uint32_t packed = 0;
    uint16_t d = 0;
    if (m > 0.0f) {
        const float inv32 = recip127(m);
        packed = codes4(v, inv32, m, !(inv32 <= 3.40282347e38f));   // f64 only if the reciprocal overflowed
        d = __builtin_bit_cast(uint16_t, static_cast<_Float16>(scale_of(m)));
    }
    uint16_t *o = out + blk * 17;   // 34 bytes = 17 halves
    o[1 + 2 * part] = static_cast<uint16_t>(packed & 0xffffu);
    o[2 + 2 * part] = static_cast<uint16_t>(packed >> 16);
    if (part == 0) o[0] = d;
}

// ------------------------------------------------------- per-token int8
// One workgroup (four waves) per token. Chunk c holds elements 256c..256c+255,
// lane l its four elements 256c + 4l .. +3 (one 16-byte load); wave w owns
// chunks wR .. wR+R-1 (K <= 1024 R), all loaded at once. The token's absmax
// meets through the waves and LDS; codes come from codes4. Planes: lanes
// 8g .. 8g+7 of a chunk hold the 32 elements of plane word 8c + g, lane 8g + k
// elements 4k .. 4k+3 of it, i.e. bits 4k .. 4k+3 of every plane's word. A
// lane first transposes its 4 x 8 code bits in place (four delta swaps), so
// that nibble b holds bit b of its four codes; the eight lanes then
// transpose their 8 x 8 nibbles (three exchange steps with the lanes k ^ 1,
// k ^ 2, k ^ 4), after which lane 8g + b holds plane b's word, and one
// store per chunk writes all 64 words (plane b, word 8c + g at lane 8g + b).
__device__ __forceinline__ uint32_t bits_to_nibbles(uint32_t x) {   // bit 8j + b -> bit 4b + j
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

// One exchange step of the 8 x 8 nibble transpose: keep the nibbles whose
// slot bit t equals this lane's bit t, take the partner's others, moved by
// 2^t slots (a rotate by sh bits, sh per lane).
__device__ __forceinline__ uint32_t nibble_step(uint32_t x, uint32_t partner, uint32_t sh, uint32_t keep) {
    const uint32_t rot = __builtin_amdgcn_alignbit(partner, partner, sh);
    return (x & keep) | (rot & ~keep);
}

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
    __shared__ float red[kThreads / 64];
    const int64_t c = blockIdx.x;
    const float *xr = x + c * K;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int64_t c0 = static_cast<int64_t>(wave) * R;   // this wave's first chunk
    const int64_t nq = K / 4;                            // float4s of the token
    float4 v[R];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < R; i++) {
        const int64_t e4 = (c0 + i) * 64 + lane;
        v[i] = reinterpret_cast<const float4 *>(xr)[e4 < nq ? e4 : nq - 1];   // clamped: issued, not used
        if (e4 < nq) m = fmaxf(m, absmax4(v[i]));
    }
    const float amax = token_absmax(m, red, wave, lane);
    const float inv32 = amax > 0.0f ? recip127(amax) : 0.0f;
    const bool f64_only = !(inv32 <= 3.40282347e38f);   // uniform: the reciprocal overflowed f32
    if (threadIdx.x == 0) scale[c] = amax > 0.0f ? scale_of(amax) : 0.0f;
    const int64_t W = K / 32;
    const int k8 = lane % 8, g = lane / 8;
    // the exchange steps' per-lane rotates and keep masks (kLow: slot bit t = 0)
    constexpr uint32_t kLow[3] = {0x0F0F0F0Fu, 0x00FF00FFu, 0x0000FFFFu};
    uint32_t sh[3], keep[3];
#pragma unroll
    for (int t = 0; t < 3; t++) {
        const bool hi = (k8 >> t) & 1;
        sh[t] = hi ? (4u << t) : 32u - (4u << t);
        keep[t] = hi ? ~kLow[t] : kLow[t];
    }
#pragma unroll
    for (int i = 0; i < R; i++) {
        if ((c0 + i) * 256 < K) {   // uniform per wave
            uint32_t w = bits_to_nibbles(codes4(v[i], inv32, amax, f64_only));
            int p = __builtin_amdgcn_update_dpp(0, static_cast<int>(w), 0xB1, 0xF, 0xF, false);   // lane k ^ 1
            w = nibble_step(w, static_cast<uint32_t>(p), sh[0], keep[0]);
            p = __builtin_amdgcn_update_dpp(0, static_cast<int>(w), 0x4E, 0xF, 0xF, false);       // lane k ^ 2
            w = nibble_step(w, static_cast<uint32_t>(p), sh[1], keep[1]);
            p = __builtin_amdgcn_ds_swizzle(static_cast<int>(w), 0x101F);   // lane k ^ 4: xor mask 4, 32-lane groups
            w = nibble_step(w, static_cast<uint32_t>(p), sh[2], keep[2]);
            const int64_t wi = (c0 + i) * 8 + g;   // plane word index of this lane's group
            if (wi < W) planes[c * 8 * W + k8 * W + wi] = w;
        }
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
    const int64_t chunks_per_wave = (K + 1023) / 1024;   // 256-element chunks, four waves
    if (chunks_per_wave <= 1)
        hipLaunchKernelGGL(act_quant_kernel<1>, grid, block, 0, hs, x, planes, x_scale, K);
    else if (chunks_per_wave <= 2)
        hipLaunchKernelGGL(act_quant_kernel<2>, grid, block, 0, hs, x, planes, x_scale, K);
    else if (chunks_per_wave <= 4)
        hipLaunchKernelGGL(act_quant_kernel<4>, grid, block, 0, hs, x, planes, x_scale, K);
    else if (chunks_per_wave <= 8)
        hipLaunchKernelGGL(act_quant_kernel<8>, grid, block, 0, hs, x, planes, x_scale, K);
    else
        hipLaunchKernelGGL(act_quant_long_kernel, grid, block, 0, hs, x, planes, x_scale, K);
    return check_launch("ternary_quantize_act");
}
