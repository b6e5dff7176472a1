// attention.hip -- split-K decode attention on gfx950 (page
// "BonsaiのWebGPUカーネルを読み解く", section on split-K flash decode
// attention: one query token has nothing to parallelise along the queries,
// so the KV sequence is cut into splits that run in parallel, each keeping
// a running maximum, a running denominator and a running output rescaled by
// exp(old max - new max) whenever the maximum grows; a merge pass brings
// every split's partials to the global maximum and combines them).
//
// Split kernel. A workgroup (four waves) owns one KV head and one split:
// the G = Hq/Hkv query heads that read that KV head are served together, so
// each key and value row is read from HBM once for all of them. Keys come in
// tiles of 64: the K and V tile are loaded with 16-byte coalesced loads into
// registers one tile ahead, stored to LDS, and then wave w serves query head
// 4i + w: lane t scores key t (scale * (q . k) over 128 dims, q read with
// scalar loads since it is the same for the whole wave, K rows padded to 132
// floats in LDS so the lanes' 16-byte reads hit distinct banks), the wave's
// maximum and sum of exp
// update the running state, and lane l accumulates output dims 2l, 2l+1
// over the tile's keys, each key's weight taken from its lane with
// v_readlane. The split writes its running output, maximum and denominator.
//
// Merge kernel. One workgroup per query head: the global maximum over the
// splits, then sum_s exp(m_s - max) o_s[d] / sum_s exp(m_s - max) l_s, the
// weights computed once per split into LDS.
// A split with no keys writes max -inf, denominator 0 and output 0, and
// contributes nothing.
#include "gd_device.h"
#include "gd_internal.h"

namespace {

constexpr int kD = 128;          // head dim
constexpr int kT = 64;           // keys per tile
constexpr int kKPad = kD + 4;    // padded K row in LDS (floats)
constexpr int kThreads = 256;
constexpr int kTileF4 = kT * kD / 4;                  // float4s per K (or V) tile
constexpr int kLoadsPerThread = kTileF4 / kThreads;   // 8

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef const f32x4 __attribute__((address_space(1))) *g_f4;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Loads of one K and one V tile (rows t0.. of this KV head; rows past the
// split end read as zero and are masked out of the scores).
__device__ __forceinline__ void load_tile(const float *kb, const float *vb, int64_t t0, int64_t t_end,
                                          f32x4 (&rk)[kLoadsPerThread], f32x4 (&rv)[kLoadsPerThread]) {
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; i++) {
        const int e = threadIdx.x + kThreads * i;
        const int row = e / (kD / 4), c4 = e % (kD / 4);
        const int64_t t = t0 + row;
        if (t < t_end) {
            rk[i] = gd::ld_stream(&((g_f4)(kb + t * kD))[c4]);   // each K/V row is read once
            rv[i] = gd::ld_stream(&((g_f4)(vb + t * kD))[c4]);
        } else {
            rk[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            rv[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }
}

template <int G>
__global__ __launch_bounds__(kThreads) void attn_split_kernel(const float *__restrict__ q,
                                                              const float *__restrict__ kc,
                                                              const float *__restrict__ vc,
                                                              float *__restrict__ part_o, float *__restrict__ part_ml,
                                                              int64_t Hq, int64_t kv_len, int64_t kv_stride,
                                                              int64_t keys_per_split, float scale) {
    constexpr int P = (G + 3) / 4;   // query heads per wave
    __shared__ f32x4 ks[kT * kKPad / 4];
    __shared__ f32x2 vs[kT * kD / 2];
    const int64_t kvh = blockIdx.x, split = blockIdx.y;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / 64);   // wave-uniform
    const int lane = threadIdx.x % 64;
    const int64_t j0 = split * keys_per_split;
    const int64_t j1 = (j0 + keys_per_split) < kv_len ? (j0 + keys_per_split) : kv_len;
    const float *kb = kc + kvh * kv_stride * kD;
    const float *vb = vc + kvh * kv_stride * kD;
    float m[P], l[P], acc[P][2];
#pragma unroll
    for (int p = 0; p < P; p++) {
        m[p] = -__builtin_inff();
        l[p] = 0.0f;
        acc[p][0] = acc[p][1] = 0.0f;
    }
    f32x4 rk[kLoadsPerThread], rv[kLoadsPerThread];
    if (j0 < j1) load_tile(kb, vb, j0, j1, rk, rv);
    for (int64_t t0 = j0; t0 < j1; t0 += kT) {
        __syncthreads();   // the previous tile's LDS reads are done (and q is stored)
#pragma unroll
        for (int i = 0; i < kLoadsPerThread; i++) {
            const int e = threadIdx.x + kThreads * i;
            const int row = e / (kD / 4), c4 = e % (kD / 4);
            ks[row * (kKPad / 4) + c4] = rk[i];
            vs[row * (kD / 2) + 2 * c4] = f32x2{rv[i][0], rv[i][1]};
            vs[row * (kD / 2) + 2 * c4 + 1] = f32x2{rv[i][2], rv[i][3]};
        }
        __syncthreads();
        if (t0 + kT < j1) load_tile(kb, vb, t0 + kT, j1, rk, rv);   // next tile, in flight during this one
        const int nvalid = static_cast<int>((j1 - t0) < kT ? (j1 - t0) : kT);
#pragma unroll
        for (int p = 0; p < P; p++) {
            const int h = 4 * p + wave;   // uniform per wave
            if (h < G) {
                // q[h] is the same for every lane: a uniform address, read
                // with scalar loads and used as scalar operands
                const g_f4 qh = (g_f4)(q + (kvh * G + h) * kD);
                float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
                for (int c = 0; c < kD / 4; c += 2) {
                    const f32x4 k0 = ks[lane * (kKPad / 4) + c], k1 = ks[lane * (kKPad / 4) + c + 1];
                    const f32x4 q0 = qh[c], q1 = qh[c + 1];
                    s0 = __builtin_fmaf(q0[0], k0[0], s0);
                    s0 = __builtin_fmaf(q0[1], k0[1], s0);
                    s0 = __builtin_fmaf(q0[2], k0[2], s0);
                    s0 = __builtin_fmaf(q0[3], k0[3], s0);
                    s1 = __builtin_fmaf(q1[0], k1[0], s1);
                    s1 = __builtin_fmaf(q1[1], k1[1], s1);
                    s1 = __builtin_fmaf(q1[2], k1[2], s1);
                    s1 = __builtin_fmaf(q1[3], k1[3], s1);
                }
                const float s = lane < nvalid ? scale * (s0 + s1) : -__builtin_inff();
                const float mnew = fmaxf(m[p], wave_max(s));   // finite: nvalid >= 1
                const float pr = lane < nvalid ? expf(s - mnew) : 0.0f;
                const float corr = expf(m[p] - mnew);         // 0 on the first tile
                l[p] = l[p] * corr + wave_sum(pr);
                m[p] = mnew;
                float a0 = acc[p][0] * corr, a1 = acc[p][1] * corr;
#pragma unroll
                for (int t = 0; t < kT; t++) {
                    const float pt = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pr), t));
                    const f32x2 v2 = vs[t * (kD / 2) + lane];
                    a0 = __builtin_fmaf(pt, v2[0], a0);
                    a1 = __builtin_fmaf(pt, v2[1], a1);
                }
                acc[p][0] = a0;
                acc[p][1] = a1;
            }
        }
    }
#pragma unroll
    for (int p = 0; p < P; p++) {
        const int h = 4 * p + wave;
        if (h < G) {
            const int64_t hq = kvh * G + h;
            float *o = part_o + (split * Hq + hq) * kD;
            reinterpret_cast<f32x2 *>(o)[lane] = f32x2{acc[p][0], acc[p][1]};
            if (lane == 0) {
                part_ml[(split * Hq + hq) * 2] = m[p];
                part_ml[(split * Hq + hq) * 2 + 1] = l[p];
            }
        }
    }
}

constexpr int kMergeChunk = 1024;   // split weights staged in LDS at a time

__device__ __forceinline__ float block_reduce(float v, bool is_max, float *red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float u = __shfl_xor(v, o);
        v = is_max ? fmaxf(v, u) : v + u;
    }
    __syncthreads();   // red is free (a previous reduction's reads are done)
    if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = v;
    __syncthreads();
    return is_max ? fmaxf(red[0], red[1]) : red[0] + red[1];
}

// One workgroup (two waves, one output dim per thread) per query head: the
// splits' maxima are reduced to the global maximum, each split's weight
// exp(m_s - max) is computed once into LDS, and every dim's weighted sum
// runs over the splits with eight loads in flight.
__global__ __launch_bounds__(kD) void attn_merge_kernel(const float *__restrict__ part_o,
                                                        const float *__restrict__ part_ml, float *__restrict__ out,
                                                        int64_t Hq, int64_t S) {
    static_assert(kD == 128, "two waves");
    __shared__ float w[kMergeChunk];
    __shared__ float red[kD / 64];
    const int64_t h = blockIdx.x;
    const int d = threadIdx.x;
    float mx = -__builtin_inff();
    for (int64_t s = d; s < S; s += kD) mx = fmaxf(mx, part_ml[(s * Hq + h) * 2]);
    mx = block_reduce(mx, true, red);   // finite: some split has keys
    float den = 0.0f, num = 0.0f;
    for (int64_t c0 = 0; c0 < S; c0 += kMergeChunk) {
        const int cn = static_cast<int>((S - c0) < kMergeChunk ? (S - c0) : kMergeChunk);
        __syncthreads();   // the previous chunk's weights are read
        for (int i = d; i < cn; i += kD) {
            const float ms = part_ml[((c0 + i) * Hq + h) * 2];
            const float wi = ms == -__builtin_inff() ? 0.0f : expf(ms - mx);   // an empty split weighs 0
            w[i] = wi;
            den = __builtin_fmaf(part_ml[((c0 + i) * Hq + h) * 2 + 1], wi, den);
        }
        __syncthreads();
        const float *po = part_o + (c0 * Hq + h) * kD + d;
#pragma unroll 8
        for (int i = 0; i < cn; i++) num = __builtin_fmaf(po[static_cast<int64_t>(i) * Hq * kD], w[i], num);
    }
    den = block_reduce(den, false, red);
    out[h * kD + d] = num / den;
}

int plan(int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, int64_t kv_len, int64_t num_splits,
         int64_t *splits, int64_t *keys_per_split) {
    GD_REQUIRE(n_heads >= 1 && n_kv_heads >= 1 && kv_len >= 1, GD_EINVAL,
               "attention: n_heads (%lld), n_kv_heads (%lld) and kv_len (%lld) must be >= 1", (long long)n_heads,
               (long long)n_kv_heads, (long long)kv_len);
    GD_REQUIRE(head_dim == kD, GD_ESHAPE, "attention: head_dim (%lld) must be %d", (long long)head_dim, kD);
    GD_REQUIRE(n_heads % n_kv_heads == 0, GD_ESHAPE, "attention: n_heads (%lld) not a multiple of n_kv_heads (%lld)",
               (long long)n_heads, (long long)n_kv_heads);
    const int64_t G = n_heads / n_kv_heads;
    GD_REQUIRE(G == 1 || G == 2 || G == 4 || G == 8, GD_ESHAPE,
               "attention: n_heads / n_kv_heads (%lld) must be 1, 2, 4 or 8", (long long)G);
    GD_REQUIRE(n_kv_heads <= 65535 && kv_len <= (INT64_C(1) << 40), GD_ERANGE, "attention: sizes too large");
    GD_REQUIRE(num_splits >= 0 && num_splits <= 65535, GD_ERANGE, "attention: num_splits (%lld) outside [0, 65535]",
               (long long)num_splits);
    int64_t s = num_splits;
    if (s == 0) {   // about 512 workgroups, at least one tile of keys each
        const int64_t tiles = (kv_len + kT - 1) / kT;
        s = (512 + n_kv_heads - 1) / n_kv_heads;
        s = s < tiles ? s : tiles;
        s = s < 1 ? 1 : s;
    }
    *splits = s;
    *keys_per_split = (kv_len + s - 1) / s;
    return GD_OK;
}

}  // namespace

using namespace gd;

extern "C" int attn_decode_workspace_bytes(int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, int64_t kv_len,
                                           int64_t num_splits, size_t *bytes) {
    GD_REQUIRE(bytes, GD_EINVAL, "attn_decode_workspace_bytes: null output pointer");
    int64_t s, kps;
    int st = plan(n_heads, n_kv_heads, head_dim, kv_len, num_splits, &s, &kps);
    if (st) return st;
    *bytes = static_cast<size_t>(s * n_heads * (kD + 2) * 4);
    clear_error();
    return GD_OK;
}

extern "C" int attn_decode_splitk(const float *q, const float *k_cache, const float *v_cache, float *out,
                                  int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, int64_t kv_len,
                                  int64_t kv_stride, float scale, int64_t num_splits, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    GD_REQUIRE(q && k_cache && v_cache && out && workspace, GD_EINVAL, "attn_decode_splitk: null pointer");
    int64_t s, kps;
    int st = plan(n_heads, n_kv_heads, head_dim, kv_len, num_splits, &s, &kps);
    if (st) return st;
    GD_REQUIRE(kv_stride >= kv_len, GD_EINVAL, "attn_decode_splitk: kv_stride (%lld) below kv_len (%lld)",
               (long long)kv_stride, (long long)kv_len);
    GD_REQUIRE(aligned(q, 16) && aligned(k_cache, 16) && aligned(v_cache, 16) && aligned(workspace, 16) &&
                   aligned(out, 4),
               GD_EALIGN, "attn_decode_splitk: q, caches and workspace must be 16-byte aligned, out 4-byte");
    const size_t need = static_cast<size_t>(s * n_heads * (kD + 2) * 4);
    GD_REQUIRE(workspace_bytes >= need, GD_ERANGE, "attn_decode_splitk: workspace of %zu bytes, %zu needed",
               workspace_bytes, need);
    float *part_o = static_cast<float *>(workspace);
    float *part_ml = part_o + s * n_heads * kD;
    const int64_t G = n_heads / n_kv_heads;
    hipStream_t hs = as_stream(stream);
    const dim3 grid(static_cast<uint32_t>(n_kv_heads), static_cast<uint32_t>(s));
#define GD_ATTN(GG)                                                                                              \
    hipLaunchKernelGGL(attn_split_kernel<GG>, grid, dim3(kThreads), 0, hs, q, k_cache, v_cache, part_o, part_ml, \
                       n_heads, kv_len, kv_stride, kps, scale)
    if (G == 1)
        GD_ATTN(1);
    else if (G == 2)
        GD_ATTN(2);
    else if (G == 4)
        GD_ATTN(4);
    else
        GD_ATTN(8);
#undef GD_ATTN
    hipLaunchKernelGGL(attn_merge_kernel, dim3(static_cast<uint32_t>(n_heads)), dim3(kD), 0, hs, part_o, part_ml,
                       out, n_heads, s);
    return check_launch("attn_decode_splitk");
}
