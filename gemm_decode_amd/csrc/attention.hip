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
// tiles of 64: the K tile and then the V tile are loaded with 16-byte
// coalesced loads into registers, K is stored to LDS and scored while V is
// still arriving, then V is stored; wave w serves query head 4i + w: lane t
// scores key t (scale * (q . k) over 128 dims, q read with scalar loads since
// it is the same for the whole wave, K rows padded to 132 floats in LDS so
// the lanes' 16-byte reads hit distinct banks), the wave's maximum and sum
// of exp update the running state, and lane l accumulates output dims 2l,
// 2l+1 over the tile's keys, each key's weight taken from its lane with
// v_readlane. The next tile's K and V loads go out as soon as this tile's
// registers are in LDS. The split writes its running output, maximum and
// denominator.
//
// Merge kernel. One workgroup per query head computes
// sum_s exp(m_s - max) o_s[d] / sum_s exp(m_s - max) l_s over the splits,
// 64 splits at a time under a running maximum.
// A split with no keys writes max -inf, denominator 0 and output 0, and
// contributes nothing.
#include <mutex>

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

// Loads of one K (or V) tile: rows t0.. of this KV head, each read once.
// Rows past the split end are clamped to its last row, so every load is
// issued unconditionally (no branch between the loads, so the wait for the
// K tile need not include the V tile behind it); such keys are masked out of
// the scores and get weight 0, and the row they repeat is finite.
__device__ __forceinline__ void load_rows(const float *base, int64_t t0, int64_t t_end,
                                          f32x4 (&r)[kLoadsPerThread]) {
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; i++) {
        const int e = threadIdx.x + kThreads * i;
        const int row = e / (kD / 4), c4 = e % (kD / 4);
        const int64_t t = (t0 + row) < t_end ? (t0 + row) : t_end - 1;
        r[i] = gd::ld_stream(&((g_f4)(base + t * kD))[c4]);
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
    // The K tile is loaded before the V tile, so the scores can start as soon
    // as K is in (loads complete in order) while V is still arriving; the next
    // tile's K goes out once this K is in LDS, its V once this V is.
    f32x4 rk[kLoadsPerThread], rv[kLoadsPerThread];
    if (j0 < j1) {
        load_rows(kb, j0, j1, rk);
        load_rows(vb, j0, j1, rv);
    }
    for (int64_t t0 = j0; t0 < j1; t0 += kT) {
        const bool more = t0 + kT < j1;
        __syncthreads();   // the previous tile's LDS reads are done
#pragma unroll
        for (int i = 0; i < kLoadsPerThread; i++) {
            const int e = threadIdx.x + kThreads * i;
            ks[(e / (kD / 4)) * (kKPad / 4) + e % (kD / 4)] = rk[i];
        }
        __syncthreads();
        if (more) load_rows(kb, t0 + kT, j1, rk);
        const int nvalid = static_cast<int>((j1 - t0) < kT ? (j1 - t0) : kT);
        float pr[P];
#pragma unroll
        for (int p = 0; p < P; p++) {
            const int h = 4 * p + wave;   // uniform per wave
            pr[p] = 0.0f;
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
                const float sc = lane < nvalid ? scale * (s0 + s1) : -__builtin_inff();
                const float mnew = fmaxf(m[p], wave_max(sc));   // finite: nvalid >= 1
                pr[p] = lane < nvalid ? expf(sc - mnew) : 0.0f;
                const float corr = expf(m[p] - mnew);          // 0 on the first tile
                l[p] = l[p] * corr + wave_sum(pr[p]);
                m[p] = mnew;
                acc[p][0] *= corr;
                acc[p][1] *= corr;
            }
        }
#pragma unroll
        for (int i = 0; i < kLoadsPerThread; i++) {
            const int e = threadIdx.x + kThreads * i;
            const int row = e / (kD / 4), c4 = e % (kD / 4);
            vs[row * (kD / 2) + 2 * c4] = f32x2{rv[i][0], rv[i][1]};
            vs[row * (kD / 2) + 2 * c4 + 1] = f32x2{rv[i][2], rv[i][3]};
        }
        __syncthreads();
        if (more) load_rows(vb, t0 + kT, j1, rv);
#pragma unroll
        for (int p = 0; p < P; p++) {
            const int h = 4 * p + wave;
            if (h < G) {
                float a0 = acc[p][0], a1 = acc[p][1];
#pragma unroll
                for (int t = 0; t < kT; t++) {
                    const float pt = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pr[p]), t));
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

constexpr int kMergeChunk = 64;                          // splits per step: one per lane of a wave
constexpr int kMergeGroups = 4;                          // thread groups of kD, each a quarter of a step
constexpr int kMergeThreads = kD * kMergeGroups;
constexpr int kMergePerGroup = kMergeChunk / kMergeGroups;

// One workgroup per query head: kMergeGroups groups of kD threads, one
// output dim per thread. The splits are taken 64 at a time: lane i of every
// wave loads split c0 + i's maximum and denominator (one vector load), and
// group g loads its dim of the partial outputs of splits c0 + 16g .. +15,
// all issued before any is used (one memory latency per step). Every wave
// sees all 64 maxima, so all groups follow the same running maximum: the
// step's maximum raises it, the running sums are rescaled by exp(old - new),
// and split i adds w_i = exp(m_i - max) times its denominator and output,
// w_i computed once by lane i and read with v_readlane. The groups' sums
// meet in LDS at the end. Splits past S and splits without keys (max -inf)
// weigh 0.
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(const float *__restrict__ part_o,
                                                                   const float *__restrict__ part_ml,
                                                                   float *__restrict__ out, int64_t Hq, int64_t S) {
    static_assert(kD == 128 && kMergeChunk == 64, "lanes of a wave index the splits of a step");
    __shared__ float part[kMergeGroups][kD];
    const int64_t h = blockIdx.x;
    const int d = threadIdx.x % kD;
    const int grp = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kD);   // wave-uniform
    const int lane = threadIdx.x % 64;
    float mx = -__builtin_inff(), den = 0.0f, num = 0.0f;
    for (int64_t c0 = 0; c0 < S; c0 += kMergeChunk) {
        const int64_t mine = (c0 + lane) < S ? (c0 + lane) : S - 1;   // clamped: weighed 0 below
        const f32x2 ml = *(const f32x2 *)(part_ml + (mine * Hq + h) * 2);
        const int64_t g0 = c0 + kMergePerGroup * grp;
        float o[kMergePerGroup];
#pragma unroll
        for (int i = 0; i < kMergePerGroup; i++) {
            const int64_t sp = (g0 + i) < S ? (g0 + i) : S - 1;
            o[i] = part_o[(sp * Hq + h) * kD + d];
        }
        __builtin_amdgcn_sched_barrier(0);   // every load of the step is issued before any is used
        // cm is finite: split 0 (in the first step) always has keys
        const float mi = (c0 + lane) < S ? ml[0] : -__builtin_inff();
        const float cm = fmaxf(mx, wave_max(mi));
        const float corr = mx == -__builtin_inff() ? 0.0f : expf(mx - cm);
        const float wi = mi == -__builtin_inff() ? 0.0f : expf(mi - cm);
        den = den * corr + wave_sum(wi * ((c0 + lane) < S ? ml[1] : 0.0f));
        num *= corr;
#pragma unroll
        for (int i = 0; i < kMergePerGroup; i++) {
            const float w = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wi), kMergePerGroup * grp + i));
            num = __builtin_fmaf(o[i], w, num);
        }
        mx = cm;
    }
    part[grp][d] = num;
    __syncthreads();
    if (grp == 0) {
        const float t = (part[0][d] + part[1][d]) + (part[2][d] + part[3][d]);
        out[h * kD + d] = t / den;   // den > 0: split 0 always has keys
    }
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

namespace {

// Enqueues the split and merge launches on a validated call; `workspace`
// holds the partials of `s` splits (caller-owned, or the file-scope scratch
// below).
int launch_attention(const float *q, const float *k_cache, const float *v_cache, float *out, int64_t n_heads,
                     int64_t n_kv_heads, int64_t kv_len, int64_t kv_stride, float scale, int64_t s, int64_t kps,
                     void *workspace, hipStream_t hs) {
    float *part_o = static_cast<float *>(workspace);
    float *part_ml = part_o + s * n_heads * kD;
    const int64_t G = n_heads / n_kv_heads;
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
    hipLaunchKernelGGL(attn_merge_kernel, dim3(static_cast<uint32_t>(n_heads)), dim3(kMergeThreads), 0, hs, part_o,
                       part_ml, out, n_heads, s);
    return GD_OK;
}

// The checks every attention entry point makes before its launches.
int validate(const float *q, const float *k_cache, const float *v_cache, float *out, int64_t n_heads,
             int64_t n_kv_heads, int64_t head_dim, int64_t kv_len, int64_t kv_stride, int64_t num_splits,
             int64_t *s, int64_t *kps, const char *name) {
    GD_REQUIRE(q && k_cache && v_cache && out, GD_EINVAL, "%s: null pointer", name);
    int st = plan(n_heads, n_kv_heads, head_dim, kv_len, num_splits, s, kps);
    if (st) return st;
    GD_REQUIRE(kv_stride >= kv_len, GD_EINVAL, "%s: kv_stride (%lld) below kv_len (%lld)", name,
               (long long)kv_stride, (long long)kv_len);
    GD_REQUIRE(aligned(q, 16) && aligned(k_cache, 16) && aligned(v_cache, 16) && aligned(out, 4), GD_EALIGN,
               "%s: q and caches must be 16-byte aligned, out 4-byte", name);
    return GD_OK;
}

}  // namespace

extern "C" int attn_decode_splitk(const float *q, const float *k_cache, const float *v_cache, float *out,
                                  int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, int64_t kv_len,
                                  int64_t kv_stride, float scale, int64_t num_splits, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    int64_t s, kps;
    int st = validate(q, k_cache, v_cache, out, n_heads, n_kv_heads, head_dim, kv_len, kv_stride, num_splits, &s,
                      &kps, "attn_decode_splitk");
    if (st) return st;
    GD_REQUIRE(workspace, GD_EINVAL, "attn_decode_splitk: null workspace");
    GD_REQUIRE(aligned(workspace, 16), GD_EALIGN, "attn_decode_splitk: workspace must be 16-byte aligned");
    const size_t need = static_cast<size_t>(s * n_heads * (kD + 2) * 4);
    GD_REQUIRE(workspace_bytes >= need, GD_ERANGE, "attn_decode_splitk: workspace of %zu bytes, %zu needed",
               workspace_bytes, need);
    launch_attention(q, k_cache, v_cache, out, n_heads, n_kv_heads, kv_len, kv_stride, scale, s, kps, workspace,
                     as_stream(stream));
    return check_launch("attn_decode_splitk");
}

// ---------------------------------------------------- no-allocation variant
// For callers that cannot allocate device memory (code under graph capture,
// serving loops that forbid it): the split partials live in this file-scope
// array instead of a caller workspace. Each device the library runs on holds
// its own copy until the process ends. Host code never uses the array's name
// as an address: its device address is resolved once per device with
// hipGetSymbolAddress (with that device current) and kept per device.
// Nothing in it needs to start at zero: the split launch writes every
// partial the merge launch reads. Calls that overlap on one device share the
// array and race.
static __device__ __align__(256) unsigned char scratch[GD_ATTN_NOALLOC_MAX_BYTES];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices];   // device address of `scratch` per device; null until resolved

int scratch_address(void **addr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GD_EHIP, "attn_decode_splitk_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    GD_REQUIRE(dev >= 0 && dev < kMaxDevices, GD_ERANGE, "attn_decode_splitk_noalloc: device %d", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(GD_EHIP, "attn_decode_splitk_noalloc: hipGetSymbolAddress on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_addr[dev] = p;
    }
    *addr = g_scratch_addr[dev];
    return GD_OK;
}

}  // namespace

extern "C" int attn_decode_splitk_noalloc(const float *q, const float *k_cache, const float *v_cache, float *out,
                                          int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, int64_t kv_len,
                                          int64_t kv_stride, float scale, int64_t num_splits, void *stream) {
    int64_t s, kps;
    int st = validate(q, k_cache, v_cache, out, n_heads, n_kv_heads, head_dim, kv_len, kv_stride, num_splits, &s,
                      &kps, "attn_decode_splitk_noalloc");
    if (st) return st;
    const size_t need = static_cast<size_t>(s * n_heads * (kD + 2) * 4);
    GD_REQUIRE(need <= GD_ATTN_NOALLOC_MAX_BYTES, GD_ERANGE,
               "attn_decode_splitk_noalloc: %zu bytes of split partials needed, above the %d-byte scratch; "
               "use attn_decode_splitk with a workspace", need, GD_ATTN_NOALLOC_MAX_BYTES);
    void *ws = nullptr;
    st = scratch_address(&ws);
    if (st) return st;
    launch_attention(q, k_cache, v_cache, out, n_heads, n_kv_heads, kv_len, kv_stride, scale, s, kps, ws,
                     as_stream(stream));
    return check_launch("attn_decode_splitk_noalloc");
}
