// measure.hip -- bandwidth-ceiling kernels (page "roofline.html": a FILL
// pass writes a non-zero, incompressible pattern so that reads reach DRAM,
// then a read pass streams 16-byte words through an XOR into a sink).
//
// The read kernel gives each wave a contiguous span of the buffer and walks
// it with 16-byte loads, four in flight per lane, so the measured figure is
// the chip's streaming-read ceiling rather than a latency bound.
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

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4 *__restrict__ d, int64_t n,
                                                                   int32_t passes, uint32_t *__restrict__ sink,
                                                                   int64_t sink_words) {
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t nthreads = static_cast<int64_t>(gridDim.x) * blockDim.x;
    uint4 acc = make_uint4(0, 0, 0, 0);
    for (int32_t p = 0; p < passes; p++) {
        int64_t i = tid;
        for (; i + 3 * nthreads < n; i += 4 * nthreads) {
            const uint4 a = d[i], b = d[i + nthreads], c = d[i + 2 * nthreads], e = d[i + 3 * nthreads];
            acc.x ^= a.x ^ b.x ^ c.x ^ e.x;
            acc.y ^= a.y ^ b.y ^ c.y ^ e.y;
            acc.z ^= a.z ^ b.z ^ c.z ^ e.z;
            acc.w ^= a.w ^ b.w ^ c.w ^ e.w;
        }
        for (; i < n; i += nthreads) {
            const uint4 a = d[i];
            acc.x ^= a.x;
            acc.y ^= a.y;
            acc.z ^= a.z;
            acc.w ^= a.w;
        }
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
    // 8 workgroups of 256 per CU on 256 CUs keeps every SIMD busy.
    int64_t blocks = 2048;
    if (blocks * kReadThreads > n) blocks = (n + kReadThreads - 1) / kReadThreads;
    hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kReadThreads), 0,
                       as_stream(stream), static_cast<const uint4 *>(buf), n, passes, sink, sink_words);
    return check_launch("gemm_decode_stream_read");
}
