// q1.hip -- Q1_0 . q8_0 on gfx950: the one-time plane repack and the
// bit-exact batch-1 GEMV (page "browseml-gpu.js": header comment "The
// arithmetic, as the reference does it", Q1_DOT_WGSL, Q1_MM_WGSL, packQ1).
//
// Mapping. One thread owns one weight row and all eight accumulation lanes
// of that row, so every lane's chain (ab over the four sub-blocks, then the
// fused acc step per block) and the final tree run in registers in exactly
// the stated order. A wave is 64 consecutive rows; the Q1 planes store a
// 64-row tile block-major so one 16-byte load per lane per block is a fully
// coalesced 1 KiB wave load.
//
// Activation staging. The q8_0 vector is shared by every row, so each
// workgroup turns it into product tables in LDS: for block i, sub-block k
// and lane l, T[i][k][l][n] = d1_k * s(n), where n is a 4-bit sign group and
// s(n) the wrapped integer sum of its four quants. |s| <= 512 and d1 has 11
// significant bits, so every entry is the exact f32 product the stated
// arithmetic forms; a row then needs one table read per 4-bit group instead
// of four selects, three integer adds, a conversion and a multiply. All 64
// lanes of a wave read the same 16-entry table at a time, so a read touches
// at most 16 distinct LDS words in 16 distinct banks.
#include "gd_internal.h"

namespace {

constexpr int kRowsPerWG = 256;           // one row per thread
constexpr int kChunkBlocks = 32;          // blocks whose tables fit in LDS
constexpr int kTableFloats = kChunkBlocks * 32 * 16;   // 64 KiB

// Exact f16 -> f32 (the hardware conversion is exact for every f16 value,
// subnormals included, with the default denormal mode).
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Bit position of element 32k + 4l + j inside word k of the bits plane.
__host__ __device__ constexpr int plane_bit(int l, int j) {
    return (8 * (l % 4) + 2 + 4 * (l / 4) + j) % 32;
}

// ------------------------------------------------------------------ repack
// One thread per (padded row, block slot). Reads the 18-byte AoS block (nine
// 16-bit loads), writes its four permuted bit words and its scale; padding
// rows and padding blocks are written as zero.
__global__ void q1_repack_kernel(const uint16_t *__restrict__ w_aos, uint32_t *__restrict__ bits,
                                 uint16_t *__restrict__ scales, int64_t rows, int64_t nb,
                                 int64_t nb8, int64_t r64) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (gid >= r64 * nb8) return;
    const int64_t r = gid / nb8;
    const int64_t i = gid % nb8;
    const int64_t t = r / 64, lane = r % 64;
    const bool live = r < rows && i < nb;
    uint16_t d0 = 0;
    uint32_t in[4] = {0u, 0u, 0u, 0u};
    if (live) {
        const uint16_t *o = w_aos + (r * nb + i) * 9;   // 18 bytes = 9 halves
        d0 = o[0];
        for (int k = 0; k < 4; k++)
            in[k] = static_cast<uint32_t>(o[1 + 2 * k]) | (static_cast<uint32_t>(o[2 + 2 * k]) << 16);
    }
    scales[((t * (nb8 / 8) + i / 8) * 64 + lane) * 8 + i % 8] = d0;
    if (i < nb) {
        uint4 out;
        uint32_t *ow = reinterpret_cast<uint32_t *>(&out);
        for (int k = 0; k < 4; k++) {
            uint32_t word = 0;
            for (int l = 0; l < 8; l++) {
                const uint32_t nib = (in[k] >> (4 * l)) & 0xfu;
                word |= __builtin_amdgcn_alignbit(nib, nib, (32 - plane_bit(l, 0)) % 32);
            }
            ow[k] = word;
        }
        *reinterpret_cast<uint4 *>(bits + ((t * nb + i) * 64 + lane) * 4) = out;
    }
}

// -------------------------------------------------------------------- GEMV
struct Q1Args {
    const uint4 *bits;        // bits plane
    const uint4 *scales;      // scale plane, 8 f16 per 16 bytes
    const uint16_t *a;        // q8_0 AoS activation (one column)
    float *y;                 // output column
};

// Builds the product tables of blocks [c0, c0 + cb) into `tab`: group
// g = (i_local*4 + k)*8 + l holds 16 floats. One thread per group per pass.
__device__ __forceinline__ void build_tables(float *tab, const uint16_t *__restrict__ a,
                                             int64_t c0, int cb) {
    for (int g = threadIdx.x; g < cb * 32; g += kRowsPerWG) {
        const int il = g >> 5, k = (g >> 3) & 3, l = g & 7;
        const uint16_t *blk = a + ((c0 + il) * 4 + k) * 17;   // 34 bytes = 17 halves
        const float d1 = f16_to_f32(blk[0]);
        const uint32_t q01 = blk[1 + 2 * l], q23 = blk[2 + 2 * l];
        int32_t q[4] = {static_cast<int8_t>(q01 & 0xff), static_cast<int8_t>(q01 >> 8),
                        static_cast<int8_t>(q23 & 0xff), static_cast<int8_t>(q23 >> 8)};
        int32_t base = 0, delta[4];
        for (int j = 0; j < 4; j++) {
            const int32_t neg = (q[j] == -128) ? -128 : -q[j];   // int8 wrapping negation
            base += neg;
            delta[j] = q[j] - neg;
        }
        float v[16];
        for (int n = 0; n < 16; n++) {
            int32_t s = base;
            for (int j = 0; j < 4; j++)
                if ((n >> j) & 1) s += delta[j];
            v[n] = d1 * static_cast<float>(s);    // exact: |s| <= 512
        }
        float4 *dst = reinterpret_cast<float4 *>(tab + g * 16);
        for (int m = 0; m < 4; m++) dst[m] = make_float4(v[4 * m], v[4 * m + 1], v[4 * m + 2], v[4 * m + 3]);
    }
}

// Table entry for the 4-bit group of lane l held in word w (see plane_bit):
// lanes 0-3 sit at bits 8l+2.., lanes 4-7 at bits 8(l-4)+6.. (mod 32), so the
// group pre-shifted by 2 is ((w or w rotated right by 4) >> 8(l%4)) & 0x3c.
template <int L>
__device__ __forceinline__ float lookup(const char *tabg, uint32_t w, uint32_t w_r4) {
    const uint32_t src = (L < 4) ? w : w_r4;
    const uint32_t off = (src >> (8 * (L % 4))) & 0x3cu;
    return *reinterpret_cast<const float *>(tabg + L * 64 + off);
}

__device__ __forceinline__ float d0_of(const uint4 &s8, int idx) {
    const uint32_t word = (idx < 2) ? s8.x : (idx < 4) ? s8.y : (idx < 6) ? s8.z : s8.w;
    const uint16_t h = (idx & 1) ? static_cast<uint16_t>(word >> 16) : static_cast<uint16_t>(word & 0xffff);
    return f16_to_f32(h);
}

__device__ __forceinline__ void q1_gemv_body(const Q1Args &p, float *tab, int64_t rows, int64_t nb,
                                             int64_t nb8) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * kRowsPerWG + threadIdx.x;
    const int64_t r64 = (rows + 63) / 64 * 64;
    const bool live = r < r64;
    const int64_t t = r / 64, lane = r % 64;
    const uint4 *bits_row = p.bits + t * nb * 64 + lane;           // + i*64 per block
    const uint4 *sc_row = p.scales + t * (nb8 / 8) * 64 + lane;     // + (i/8)*64

    float acc[8];
#pragma unroll
    for (int l = 0; l < 8; l++) acc[l] = 0.0f;

    for (int64_t c0 = 0; c0 < nb; c0 += kChunkBlocks) {
        const int cb = static_cast<int>((nb - c0) < kChunkBlocks ? (nb - c0) : kChunkBlocks);
        if (c0 > 0) __syncthreads();
        build_tables(tab, p.a, c0, cb);
        __syncthreads();
        if (live) {
            uint4 s8 = make_uint4(0, 0, 0, 0);
            for (int il = 0; il < cb; il++) {
                const int64_t i = c0 + il;
                if ((i & 7) == 0 || il == 0) s8 = sc_row[(i >> 3) * 64];
                const float d0 = d0_of(s8, static_cast<int>(i & 7));
                const uint4 wb = bits_row[i * 64];
                const uint32_t wk[4] = {wb.x, wb.y, wb.z, wb.w};
                float ab[8];
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    const char *tabg = reinterpret_cast<const char *>(tab) + ((il * 4 + k) * 8) * 64;
                    const uint32_t w = wk[k];
                    const uint32_t w_r4 = __builtin_amdgcn_alignbit(w, w, 4);
                    float v[8];
                    v[0] = lookup<0>(tabg, w, w_r4);
                    v[1] = lookup<1>(tabg, w, w_r4);
                    v[2] = lookup<2>(tabg, w, w_r4);
                    v[3] = lookup<3>(tabg, w, w_r4);
                    v[4] = lookup<4>(tabg, w, w_r4);
                    v[5] = lookup<5>(tabg, w, w_r4);
                    v[6] = lookup<6>(tabg, w, w_r4);
                    v[7] = lookup<7>(tabg, w, w_r4);
#pragma unroll
                    for (int l = 0; l < 8; l++) ab[l] = (k == 0) ? v[l] : ab[l] + v[l];
                }
#pragma unroll
                for (int l = 0; l < 8; l++) acc[l] = __builtin_fmaf(d0, ab[l], acc[l]);
            }
        }
    }
    if (r < rows)
        p.y[r] = ((acc[0] + acc[4]) + (acc[2] + acc[6])) + ((acc[1] + acc[5]) + (acc[3] + acc[7]));
}

__global__ __launch_bounds__(kRowsPerWG) void q1_gemv_kernel(const uint4 *bits, const uint4 *scales,
                                                             const uint16_t *a, float *y, int64_t rows,
                                                             int64_t nb, int64_t nb8) {
    __shared__ float tab[kTableFloats];
    const int64_t c = blockIdx.y;   // activation column
    Q1Args p{bits, scales, a + c * (nb * 4) * 17, y + c * rows};
    q1_gemv_body(p, tab, rows, nb, nb8);
}

__global__ __launch_bounds__(kRowsPerWG) void q1_gemv_grouped_kernel(const gd_q1_problem *probs,
                                                                     int64_t rows, int64_t nb,
                                                                     int64_t nb8) {
    __shared__ float tab[kTableFloats];
    const gd_q1_problem pr = probs[blockIdx.y];
    Q1Args p{static_cast<const uint4 *>(pr.bits_plane), static_cast<const uint4 *>(pr.scale_plane),
             static_cast<const uint16_t *>(pr.a_q8), pr.y};
    q1_gemv_body(p, tab, rows, nb, nb8);
}

// ------------------------------------------------------------ validation
int plane_sizes(int64_t rows, int64_t K, int64_t *bits_bytes, int64_t *scale_bytes) {
    GD_REQUIRE(rows >= 1 && K >= 1, GD_EINVAL, "rows (%lld) and K (%lld) must be >= 1",
               (long long)rows, (long long)K);
    GD_REQUIRE(K % 128 == 0, GD_ESHAPE, "K (%lld) must be a multiple of 128", (long long)K);
    GD_REQUIRE(rows <= INT64_C(2147483584), GD_ERANGE, "rows (%lld) above 2^31 - 64", (long long)rows);
    const int64_t nb = K / 128, nb8 = (nb + 7) / 8 * 8, r64 = (rows + 63) / 64 * 64;
    int64_t t1, t2;
    GD_REQUIRE(gd::mul_ok(r64, nb, &t1) && gd::mul_ok(t1, 16, bits_bytes), GD_EINVAL, "bits plane size overflows");
    GD_REQUIRE(gd::mul_ok(r64, nb8, &t2) && gd::mul_ok(t2, 2, scale_bytes), GD_EINVAL, "scale plane size overflows");
    return GD_OK;
}

}  // namespace

using namespace gd;

extern "C" int q1_planes_bytes(int64_t rows, int64_t K, size_t *bits_bytes, size_t *scale_bytes) {
    GD_REQUIRE(bits_bytes && scale_bytes, GD_EINVAL, "q1_planes_bytes: null output pointer");
    int64_t b, s;
    int st = plane_sizes(rows, K, &b, &s);
    if (st) return st;
    *bits_bytes = static_cast<size_t>(b);
    *scale_bytes = static_cast<size_t>(s);
    clear_error();
    return GD_OK;
}

extern "C" int q1_repack(const void *w_aos, int64_t rows, int64_t K, void *bits_plane, void *scale_plane,
                         void *stream) {
    GD_REQUIRE(w_aos && bits_plane && scale_plane, GD_EINVAL, "q1_repack: null pointer");
    int64_t b, s;
    int st = plane_sizes(rows, K, &b, &s);
    if (st) return st;
    GD_REQUIRE(aligned(w_aos, 2), GD_EALIGN, "q1_repack: w_aos must be 2-byte aligned");
    GD_REQUIRE(aligned(bits_plane, 16) && aligned(scale_plane, 16), GD_EALIGN,
               "q1_repack: planes must be 16-byte aligned");
    const int64_t nb = K / 128, nb8 = (nb + 7) / 8 * 8, r64 = (rows + 63) / 64 * 64;
    const int64_t n = r64 * nb8;
    const int tpb = 256;
    const int64_t grid = (n + tpb - 1) / tpb;
    GD_REQUIRE(grid <= INT64_C(2147483647), GD_ERANGE, "q1_repack: weight too large for one launch");
    hipLaunchKernelGGL(q1_repack_kernel, dim3(static_cast<uint32_t>(grid)), dim3(tpb), 0, as_stream(stream),
                       static_cast<const uint16_t *>(w_aos), static_cast<uint32_t *>(bits_plane),
                       static_cast<uint16_t *>(scale_plane), rows, nb, nb8, r64);
    return check_launch("q1_repack");
}

extern "C" int q1_q8_gemv(const void *bits_plane, const void *scale_plane, const void *a_q8, float *y,
                          int64_t rows, int64_t K, int64_t n_act, void *stream) {
    GD_REQUIRE(bits_plane && scale_plane && a_q8 && y, GD_EINVAL, "q1_q8_gemv: null pointer");
    int64_t b, s;
    int st = plane_sizes(rows, K, &b, &s);
    if (st) return st;
    GD_REQUIRE(n_act >= 1, GD_EINVAL, "q1_q8_gemv: n_act (%lld) must be >= 1", (long long)n_act);
    GD_REQUIRE(n_act <= 65535, GD_ERANGE, "q1_q8_gemv: n_act (%lld) above 65535", (long long)n_act);
    GD_REQUIRE(aligned(bits_plane, 16) && aligned(scale_plane, 16), GD_EALIGN,
               "q1_q8_gemv: planes must be 16-byte aligned");
    GD_REQUIRE(aligned(a_q8, 2), GD_EALIGN, "q1_q8_gemv: a_q8 must be 2-byte aligned");
    GD_REQUIRE(aligned(y, 4), GD_EALIGN, "q1_q8_gemv: y must be 4-byte aligned");
    const int64_t nb = K / 128, nb8 = (nb + 7) / 8 * 8;
    const int64_t gx = (rows + kRowsPerWG - 1) / kRowsPerWG;
    hipLaunchKernelGGL(q1_gemv_kernel, dim3(static_cast<uint32_t>(gx), static_cast<uint32_t>(n_act)),
                       dim3(kRowsPerWG), 0, as_stream(stream), static_cast<const uint4 *>(bits_plane),
                       static_cast<const uint4 *>(scale_plane), static_cast<const uint16_t *>(a_q8), y, rows,
                       nb, nb8);
    return check_launch("q1_q8_gemv");
}

extern "C" int q1_q8_gemv_grouped(const gd_q1_problem *problems, int64_t count, int64_t rows, int64_t K,
                                  void *stream) {
    GD_REQUIRE(problems, GD_EINVAL, "q1_q8_gemv_grouped: null problems array");
    int64_t b, s;
    int st = plane_sizes(rows, K, &b, &s);
    if (st) return st;
    GD_REQUIRE(count >= 1, GD_EINVAL, "q1_q8_gemv_grouped: count (%lld) must be >= 1", (long long)count);
    GD_REQUIRE(count <= 65535, GD_ERANGE, "q1_q8_gemv_grouped: count (%lld) above 65535", (long long)count);
    GD_REQUIRE(aligned(problems, 8), GD_EALIGN, "q1_q8_gemv_grouped: problems must be 8-byte aligned");
    const int64_t nb = K / 128, nb8 = (nb + 7) / 8 * 8;
    const int64_t gx = (rows + kRowsPerWG - 1) / kRowsPerWG;
    hipLaunchKernelGGL(q1_gemv_grouped_kernel, dim3(static_cast<uint32_t>(gx), static_cast<uint32_t>(count)),
                       dim3(kRowsPerWG), 0, as_stream(stream), problems, rows, nb, nb8);
    return check_launch("q1_q8_gemv_grouped");
}
