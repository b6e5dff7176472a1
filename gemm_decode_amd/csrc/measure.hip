// measure.hip -- bandwidth-ceiling kernels (page "roofline.html": a FILL
// pass writes a non-zero, incompressible pattern so that reads reach DRAM,
// then a read pass streams 16-byte words through an XOR into a sink).
//
// The read kernel gives each wave a contiguous span of the buffer and walks
// it with 16-byte non-temporal loads, eight in flight per lane: of the
// patterns tried on this chip (grid-stride or per-wave spans, four or eight
// loads in flight, with or without the hint, 1024 to 8192 workgroups) it
// read fastest, so the figure is the chip's streaming-read ceiling rather
// than a latency bound.
#include "gd_internal.h"

namespace {

__global__ void fill_kernel(uint4 *__restrict__ d, int64_t n, uint32_t seed) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        const uint32_t u = static_cast<uint32_t>(i) ^ seed;
        d[i] = make_uint4(u * 2654435761u + 1u, u * 40503u + 7u, u ^ 0x9e3779b9u, u * 2246822519u + 3u);
    }
}

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;                    // loads in flight per lane
constexpr int kReadStep = 64 * kReadUnroll;       // 16-byte words per wave step

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef const u32x4 __attribute__((address_space(1))) *gptr_u4;

// Wave w reads words [w*span, min((w+1)*span, n)); span is a multiple of
// kReadStep with waves*span >= n, so whole steps need no bounds check.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4 *__restrict__ dp, int64_t n,
                                                                   int64_t span, int32_t passes,
                                                                   uint32_t *__restrict__ sink,
                                                                   int64_t sink_words) {
    const gptr_u4 d = (gptr_u4)dp;
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t lane = threadIdx.x % 64;
    const int64_t b = (tid / 64) * span;
    const int64_t e = b + span < n ? b + span : n;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int32_t p = 0; p < passes; p++) {
        int64_t j = b;
        for (; j + kReadStep <= e; j += kReadStep) {
            u32x4 v[kReadUnroll];
#pragma unroll
            for (int u = 0; u < kReadUnroll; u++) v[u] = __builtin_nontemporal_load(&d[j + 64 * u + lane]);
#pragma unroll
            for (int u = 0; u < kReadUnroll; u++) acc ^= v[u];
        }
        for (int64_t i = j + lane; i < e; i += 64) acc ^= d[i];
    }
    sink[tid % sink_words] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

using namespace gd;

extern "C" int gemm_decode_fill(void *buf, size_t bytes, uint32_t seed, void *stream) {
    GD_REQUIRE(buf, GD_EINVAL, "gemm_decode_fill: null buffer");
    GD_REQUIRE(bytes > 0, GD_EINVAL, "gemm_decode_fill: zero bytes");
    GD_REQUIRE(bytes % 16 == 0, GD_ESHAPE, "gemm_decode_fill: bytes must be a multiple of 16");
    GD_REQUIRE(aligned(buf, 16), GD_EALIGN, "gemm_decode_fill: buffer must be 16-byte aligned");
    const int64_t n = static_cast<int64_t>(bytes / 16);
    const int64_t blocks = (n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536;
    hipLaunchKernelGGL(fill_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, as_stream(stream),
                       static_cast<uint4 *>(buf), n, seed);
    return check_launch("gemm_decode_fill");
}

extern "C" int gemm_decode_stream_read(const void *buf, size_t bytes, int32_t passes, uint32_t *sink,
                                       int64_t sink_words, void *stream) {
    GD_REQUIRE(buf && sink, GD_EINVAL, "gemm_decode_stream_read: null pointer");
    GD_REQUIRE(bytes > 0 && passes >= 1 && sink_words >= 1, GD_EINVAL,
               "gemm_decode_stream_read: bytes, passes and sink_words must be positive");
    GD_REQUIRE(bytes % 16 == 0, GD_ESHAPE, "gemm_decode_stream_read: bytes must be a multiple of 16");
    GD_REQUIRE(aligned(buf, 16) && aligned(sink, 4), GD_EALIGN, "gemm_decode_stream_read: misaligned pointer");
    const int64_t n = static_cast<int64_t>(bytes / 16);
    // four workgroups of 256 per CU on 256 CUs
    const int64_t blocks = 1024, waves = blocks * (kReadThreads / 64);
    int64_t span = (n + waves - 1) / waves;
    span = (span + kReadStep - 1) / kReadStep * kReadStep;
    hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kReadThreads), 0,
                       as_stream(stream), static_cast<const uint4 *>(buf), n, span, passes, sink, sink_words);
    return check_launch("gemm_decode_stream_read");
}
