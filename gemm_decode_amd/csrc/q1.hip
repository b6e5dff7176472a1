// q1.hip -- Q1_0 . q8_0 on gfx950: the one-time plane repack and the
// bit-exact batch-1 GEMV (page "browseml-gpu.js": header comment "The
// arithmetic, as the reference does it", Q1_DOT_WGSL, Q1_MM_WGSL, packQ1).
//
// Arithmetic. For each row the eight accumulation lanes l = 0..7 run in the
// stated order: ab_l = T0 + T1 + T2 + T3 over the sub-blocks (T_k the exact
// product d1_k * s_{k,l}), then acc_l = fma(d0, ab_l, acc_l) per block, and
// finally ((a0+a4)+(a2+a6)) + ((a1+a5)+(a3+a7)). Every step is one IEEE
// operation in that order, so the result is bit-exact.
//
// Activation staging. The q8_0 vector is shared by every row, so each
// workgroup turns it into product tables in LDS: for block i, sub-block k
// and lane l, T[i][k][l][n] = d1_k * s(n), n a 4-bit sign group and s(n) the
// wrapped integer sum of its four quants. |s| <= 512 and d1 has 11
// significant bits, so every entry is the exact f32 product the stated
// arithmetic forms, and a row needs one table read per 4-bit group.
//
// Mapping. A 64-row tile is served by two waves: the "low" wave runs lanes
// 0-3 of all 64 rows, the "high" wave lanes 4-7. Each wave reads its own
// 8 bytes per row and block (the planes store the two halves apart, so a
// wave load is 512 contiguous bytes), pulls 16 table offsets out of them
// with one v_and_b32 (SDWA byte select) each, and reads the tables at
// immediate LDS offsets. All 64 lanes of a wave read the same 16-entry table
// per instruction: at most 16 distinct dwords in 16 distinct banks. The two
// halves meet once per row, through LDS, for the final tree.
#include "gd_device.h"
#include "gd_internal.h"

namespace {

constexpr int kThreads = 512;             // 8 waves: 4 tiles x 2 halves
constexpr int kRowsPerWG = 256;
constexpr int kChunkBlocks = 32;          // blocks whose tables fit in LDS
constexpr int kTableFloats = kChunkBlocks * 32 * 16;   // 64 KiB
// A single GEMV of up to this many 256-row blocks takes the one-chain-per-
// thread kernel (latency); larger ones take the four-chain kernel.
constexpr int64_t kLatMaxRowBlocks = 64;
constexpr int64_t kLatWideRows = 8192;
// While n_act * rows stays within this (about two waves per SIMD in all), a
// few-row product runs as independent one-chain-per-thread GEMVs, one per
// column; above it each column runs the four-chain kernel (both re-read the
// weights per column, mostly from cache).
// Up to this many workgroups (half the CUs), a launch takes workgroups of
// half the rows: 128 instead of 256 on the four-chain kernel, 16 instead of
// 32 on the one-chain kernel (there only while K is one table chunk).
constexpr int64_t kLatMaxColumnRows = 16384;
constexpr int64_t kNarrowMaxWGs = 128;
// Threads per workgroup of the grouped launch (two per row of a 64-row tile).
constexpr int kGroupedThreads = 512;
// 256-row units per workgroup of the grouped launch when K is 16, 24 or 32
// whole blocks (one table chunk): the units share the table build. On the
// decode step (weights streamed from HBM) two units per workgroup measured
// 3 % faster than one and three another 1.5 %; four need 132 VGPRs (three
// waves per SIMD) and were much slower.
constexpr int kUnitsPerWG = 3;

// Pointers into device global memory (address space 1), so weight loads are
// global_load (counted by vmcnt only), not flat loads that also hold lgkmcnt.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef const u32x2 __attribute__((address_space(1))) *gptr_u2;
typedef const u32x4 __attribute__((address_space(1))) *gptr_u4;

using gd::ld_stream;


// Exact f16 -> f32 (the conversion is exact for every f16 value, subnormals
// included, under the default denormal mode).
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// ------------------------------------------------------------------ repack
// Nibble of lane l in sub-block k of a block, from the page's LSB-first
// words (element 32k + e at bit e of word k).
__device__ __forceinline__ uint32_t nib_of(const uint32_t (&in)[4], int k, int l) {
    return (in[k] >> (4 * l)) & 0xfu;
}

// One thread per (padded row, block slot): reads the 18-byte AoS block (nine
// 16-bit loads), writes its two 8-byte halves and its scale; padding rows and
// blocks are written as zero.
__global__ void q1_repack_kernel(const uint16_t *__restrict__ w_aos, uint32_t *__restrict__ bits,
                                 uint16_t *__restrict__ scales, int64_t rows, int64_t nb, int64_t nb8,
                                 int64_t r64) {
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
        for (int h = 0; h < 2; h++) {
            uint32_t out[2];
            for (int m = 0; m < 2; m++) {
                uint32_t word = 0;
                for (int jj = 0; jj < 4; jj++)
                    for (int kk = 0; kk < 2; kk++) {
                        const uint32_t nib = nib_of(in, 2 * m + kk, 4 * h + jj);
                        const int pos = (8 * jj + 2 + 4 * kk) % 32;
                        word |= __builtin_amdgcn_alignbit(nib, nib, (32 - pos) % 32);   // rotate left by pos
                    }
                out[m] = word;
            }
            *reinterpret_cast<uint2 *>(bits + (((t * nb + i) * 2 + h) * 64 + lane) * 2) = make_uint2(out[0], out[1]);
        }
    }
}

// ------------------------------------------------------------ tables (a2)
// Group g = (i_local*4 + k)*8 + l of a chunk holds 16 floats. With NT
// threads, thread tid owns groups g = tid + NT*j. The build is split so its activation
// loads can be issued ahead of the weight prefetch (the load counter is in
// order: waiting for loads issued after the prefetch would drain it).
// NT threads build a chunk, 1024 / NT groups each.
template <int NT>
struct TableRawN {
    static constexpr int NG = kChunkBlocks * 32 / NT;
    uint32_t d[NG], q01[NG], q23[NG];
};
typedef TableRawN<kThreads> TableRaw;

template <int NT = kThreads>
__device__ __forceinline__ void table_loads(TableRawN<NT> &raw, const uint16_t *a_generic, int64_t c0, int cb) {
    // C-style cast: an address-space cast from the generic pointer
    const auto a = (const uint16_t __attribute__((address_space(1))) *)a_generic;
    const int ng = cb * 32;
#pragma unroll
    for (int j = 0; j < TableRawN<NT>::NG; j++) {
        int g = threadIdx.x + NT * j;
        g = g < ng ? g : ng - 1;                  // clamped: computed, never stored
        const int il = g >> 5, k = (g >> 3) & 3, l = g & 7;
        const auto blk = a + ((c0 + il) * 4 + k) * 17;   // 34 bytes = 17 halves
        raw.d[j] = blk[0];
        raw.q01[j] = blk[1 + 2 * l];
        raw.q23[j] = blk[2 + 2 * l];
    }
}

// Entries: T[0] = d1*s(0) and T[n] = T[n without its lowest set bit] +
// d1*delta(lowest bit). Every partial value is d1 times an integer of
// magnitude <= 512, so each add is exact and T[n] = d1*s(n) bit for bit.
// One group's 16 entries from its raw halves (d1, quants 0-1, quants 2-3).
__device__ __forceinline__ void table_group(float *dst_g, uint32_t rd, uint32_t rq01, uint32_t rq23) {
    const float d1 = f16_to_f32(static_cast<uint16_t>(rd));
    const int32_t q[4] = {static_cast<int8_t>(rq01 & 0xff), static_cast<int8_t>(rq01 >> 8),
                          static_cast<int8_t>(rq23 & 0xff), static_cast<int8_t>(rq23 >> 8)};
    int32_t base = 0;
    float dlt[4];
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
        const int32_t neg = (q[jj] == -128) ? -128 : -q[jj];   // int8 wrapping negation
        base += neg;
        dlt[jj] = d1 * static_cast<float>(q[jj] - neg);         // exact: |q - neg| <= 255
    }
    float v[16];
    v[0] = d1 * static_cast<float>(base);                        // exact: |base| <= 512
#pragma unroll
    for (int n = 1; n < 16; n++) {
        const int low = __builtin_ctz(n);
        v[n] = v[n & (n - 1)] + dlt[low];
    }
    float4 *dst = reinterpret_cast<float4 *>(dst_g);
#pragma unroll
    for (int m = 0; m < 4; m++) dst[m] = make_float4(v[4 * m], v[4 * m + 1], v[4 * m + 2], v[4 * m + 3]);
}

template <int NT = kThreads>
__device__ __forceinline__ void table_store(float *tab, const TableRawN<NT> &raw, int cb) {
    const int ng = cb * 32;
#pragma unroll
    for (int j = 0; j < TableRawN<NT>::NG; j++) {
        const int g = threadIdx.x + NT * j;
        if (g < ng) table_group(tab + g * 16, raw.d[j], raw.q01[j], raw.q23[j]);
    }
}

// ------------------------------------------------------------------ GEMV
struct Q1Args {
    const uint32_t *bits;     // bits plane
    const uint4 *scales;      // scale plane, 8 f16 per 16 bytes
    const uint16_t *a;        // q8_0 AoS activation (one column)
    float *y;                 // output column
};

// Table offsets: gd::grp<B>(w) is the 4-bit group held in byte B of w,
// pre-shifted by 2 (one SDWA v_and_b32).
using gd::grp;

template <int U>
__device__ __forceinline__ float d0_half(const u32x4 &s8) {
    const uint32_t word = (U < 2) ? s8.x : (U < 4) ? s8.y : (U < 6) ? s8.z : s8.w;
    return f16_to_f32(static_cast<uint16_t>((U & 1) ? (word >> 16) : (word & 0xffffu)));
}

// The 16 table reads of half H of block U of the chunk: word m covers
// sub-blocks 2m (bytes' bits 2..5) and 2m+1 (the word rotated by 4); byte jj
// is lane 4H + jj. Table (U, k, l) starts at byte U*2048 + k*512 + l*64.
template <int H, int U>
__device__ __forceinline__ void half_reads(const char *tab, const u32x2 &wb, float (&v)[16]) {
    const uint32_t wm[2] = {wb.x, wb.y};
#pragma unroll
    for (int m = 0; m < 2; m++) {
        const uint32_t w = wm[m];
        const uint32_t wr = __builtin_amdgcn_alignbit(w, w, 4);
        const char *t0 = tab + U * 2048 + (2 * m) * 512 + (4 * H) * 64;
        const char *t1 = t0 + 512;
        v[8 * m + 0] = *reinterpret_cast<const float *>(t0 + 0 * 64 + grp<0>(w));
        v[8 * m + 1] = *reinterpret_cast<const float *>(t0 + 1 * 64 + grp<1>(w));
        v[8 * m + 2] = *reinterpret_cast<const float *>(t0 + 2 * 64 + grp<2>(w));
        v[8 * m + 3] = *reinterpret_cast<const float *>(t0 + 3 * 64 + grp<3>(w));
        v[8 * m + 4] = *reinterpret_cast<const float *>(t1 + 0 * 64 + grp<0>(wr));
        v[8 * m + 5] = *reinterpret_cast<const float *>(t1 + 1 * 64 + grp<1>(wr));
        v[8 * m + 6] = *reinterpret_cast<const float *>(t1 + 2 * 64 + grp<2>(wr));
        v[8 * m + 7] = *reinterpret_cast<const float *>(t1 + 3 * 64 + grp<3>(wr));
    }
}

// ab_jj = T_{k=0} + T_{k=1} + T_{k=2} + T_{k=3} in order, then the fused step.
// v[8m + jj] is sub-block 2m, v[8m + 4 + jj] sub-block 2m+1.
__device__ __forceinline__ void half_math(const float (&v)[16], float d0, float (&acc)[4]) {
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
        float ab = v[jj];
        ab = ab + v[4 + jj];
        ab = ab + v[8 + jj];
        ab = ab + v[12 + jj];
        acc[jj] = __builtin_fmaf(d0, ab, acc[jj]);
    }
}

struct RowPtrs {
    gptr_u2 bits;          // this wave's half of block 0 of this row; + i*128 per block
    gptr_u4 sc;            // scales of blocks 0..7 of this row; + (i/8)*64
};

// Streaming loads when every group is read once; plain loads when a chunk's
// clamped prefetch will read the same group again (rows shorter than four
// groups, a partial last chunk), so that the repeats find it in L2 instead
// of fetching it from HBM again. `stream` is uniform.
__device__ __forceinline__ void load_group(const RowPtrs &rp, int64_t g, u32x2 (&wb)[8], u32x4 &s8, bool stream) {
    if (stream) {
#pragma unroll
        for (int u = 0; u < 8; u++) wb[u] = ld_stream(&rp.bits[(8 * g + u) * 128]);
        s8 = ld_stream(&rp.sc[g * 64]);
    } else {
#pragma unroll
        for (int u = 0; u < 8; u++) wb[u] = rp.bits[(8 * g + u) * 128];
        s8 = rp.sc[g * 64];
    }
}

// Eight blocks U0..U0+7 of the chunk: table reads run two blocks ahead of the
// arithmetic (three register sets of 16 values), which hides more LDS latency
// than one block ahead at the same register budget as a third set of weight
// registers would cost. With REFILL, block u's register is reloaded with
// block u of group gn as soon as its table offsets have been extracted, and
// the scales once the last d0 has been read, so the next loads leave one
// block at a time instead of after the whole group.
template <int H, int U0, bool REFILL>
__device__ __forceinline__ void group8(const char *tab, u32x2 (&wb)[8], u32x4 &s8, float (&acc)[4],
                                       const RowPtrs &rp, int64_t gn) {
    float va[16], vb[16], vc[16];
    auto refill = [&](int u) {
        if constexpr (REFILL) wb[u] = ld_stream(&rp.bits[(8 * gn + u) * 128]);
    };
    half_reads<H, U0 + 0>(tab, wb[0], va);
    refill(0);
    half_reads<H, U0 + 1>(tab, wb[1], vb);
    refill(1);
    half_reads<H, U0 + 2>(tab, wb[2], vc);
    refill(2);
    half_math(va, d0_half<0>(s8), acc);
    half_reads<H, U0 + 3>(tab, wb[3], va);
    refill(3);
    half_math(vb, d0_half<1>(s8), acc);
    half_reads<H, U0 + 4>(tab, wb[4], vb);
    refill(4);
    half_math(vc, d0_half<2>(s8), acc);
    half_reads<H, U0 + 5>(tab, wb[5], vc);
    refill(5);
    half_math(va, d0_half<3>(s8), acc);
    half_reads<H, U0 + 6>(tab, wb[6], va);
    refill(6);
    half_math(vb, d0_half<4>(s8), acc);
    half_reads<H, U0 + 7>(tab, wb[7], vb);
    refill(7);
    half_math(vc, d0_half<5>(s8), acc);
    half_math(va, d0_half<6>(s8), acc);
    half_math(vb, d0_half<7>(s8), acc);
    if constexpr (REFILL) s8 = ld_stream(&rp.sc[gn * 64]);
}


// One chunk of up to 32 blocks starting at group g0 (n4 full groups), with
// the chunk's tables built in LDS. Straight-line code: two register
// buffers; the first two groups refill them with groups g0+2 and g0+3 as
// they are consumed (group indices clamped to the last full group, so every
// load is issued).
template <int H, int NT>
__device__ __forceinline__ void chunk(float *tab, const Q1Args &p, const RowPtrs &rp, int64_t g0, int64_t n4,
                                      int64_t ng, int64_t nb, float (&acc)[4]) {
    const char *tabc = reinterpret_cast<const char *>(tab);
    const int64_t gl = ng - 1;
    const int64_t i0 = 8 * g0;
    const int cb = static_cast<int>((nb - i0) < kChunkBlocks ? (nb - i0) : kChunkBlocks);
    TableRawN<NT> raw;
    table_loads<NT>(raw, p.a, i0, cb);
    asm volatile("" ::: "memory");   // keep the table loads ahead of the prefetch
    u32x2 w0[8], w1[8];
    u32x4 s0, s1;
    // Prefetch indices past the last group are redirected to this chunk's
    // second group, which such a chunk loads with plain loads: the repeats
    // then hit L2.
    const bool stream = g0 + 3 <= gl;   // no prefetch index below is clamped
    const int64_t g1 = (g0 + 1 < gl) ? g0 + 1 : gl;
    load_group(rp, g0, w0, s0, stream);
    load_group(rp, g1, w1, s1, stream);
    if (g0 > 0) __syncthreads();
    table_store<NT>(tab, raw, cb);
    __syncthreads();
    group8<H, 0, true>(tabc, w0, s0, acc, rp, (g0 + 2 <= gl) ? g0 + 2 : g1);
    if (n4 > 1) group8<H, 8, true>(tabc, w1, s1, acc, rp, (g0 + 3 <= gl) ? g0 + 3 : g1);
    if (n4 > 2) group8<H, 16, false>(tabc, w0, s0, acc, rp, 0);
    if (n4 > 3) group8<H, 24, false>(tabc, w1, s1, acc, rp, 0);
}

// One block of half H at a run-time position (tail blocks past the last full
// group of eight): same reads, same arithmetic, run-time table offsets.
template <int H>
__device__ __forceinline__ void tail_block(const char *tabb, const u32x2 &wb, float d0, float (&acc)[4]) {
    const uint32_t wm[2] = {wb.x, wb.y};
    float v[16];
#pragma unroll
    for (int m = 0; m < 2; m++) {
        const uint32_t w = wm[m];
        const uint32_t wr = __builtin_amdgcn_alignbit(w, w, 4);
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
            const char *t0 = tabb + (2 * m) * 512 + (4 * H + jj) * 64;
            v[8 * m + jj] = *reinterpret_cast<const float *>(t0 + ((w >> (8 * jj)) & 0x3cu));
            v[8 * m + 4 + jj] = *reinterpret_cast<const float *>(t0 + 512 + ((wr >> (8 * jj)) & 0x3cu));
        }
    }
    half_math(v, d0, acc);
}

__device__ __forceinline__ float d0_of(const u32x4 &s8, int idx) {
    const uint32_t word = (idx < 2) ? s8.x : (idx < 4) ? s8.y : (idx < 6) ? s8.z : s8.w;
    return f16_to_f32(static_cast<uint16_t>((idx & 1) ? (word >> 16) : (word & 0xffffu)));
}

template <int H, int NT>
__device__ __forceinline__ void half_row(float *tab, const Q1Args &p, const RowPtrs &rp, int64_t nb, float (&acc)[4]) {
    const int64_t ng = nb / 8;
    constexpr int kGroupsPerChunk = kChunkBlocks / 8;
    for (int64_t g0 = 0; g0 < ng; g0 += kGroupsPerChunk) {
        const int64_t n4 = (ng - g0) < kGroupsPerChunk ? (ng - g0) : kGroupsPerChunk;
        chunk<H, NT>(tab, p, rp, g0, n4, ng, nb, acc);
    }
    const int64_t it0 = ng * 8;
    if (it0 < nb) {   // tail: the last nb % 8 blocks
        const int64_t c0 = it0 / kChunkBlocks * kChunkBlocks;
        if (it0 % kChunkBlocks == 0) {
            if (ng > 0) __syncthreads();
            TableRawN<NT> raw;
            table_loads<NT>(raw, p.a, it0, static_cast<int>(nb - it0));
            table_store<NT>(tab, raw, static_cast<int>(nb - it0));
            __syncthreads();
        }
        const u32x4 s8 = ld_stream(&rp.sc[(it0 >> 3) * 64]);
        const char *tabc = reinterpret_cast<const char *>(tab);
        for (int64_t i = it0; i < nb; i++) {
            const u32x2 wbv = ld_stream(&rp.bits[i * 128]);
            tail_block<H>(tabc + (i - c0) * 2048, wbv, d0_of(s8, static_cast<int>(i & 7)), acc);
        }
    }
}

// NT threads: NT/128 tiles of 64 rows, two waves (halves) each.
template <int NT>
__device__ __forceinline__ void q1_gemv_body(const Q1Args &p, float *tab, int64_t rows, int64_t nb, int64_t nb8) {
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int tl = wave >> 1, h = wave & 1;
    const int64_t r = static_cast<int64_t>(blockIdx.x) * (NT / 2) + tl * 64 + lane;
    const int64_t r64 = (rows + 63) / 64 * 64;
    // Rows past the padded rows read the last padded row (never stored), so
    // every thread runs the same loads and barriers.
    const int64_t rl = r < r64 ? r : r64 - 1;
    const int64_t t = rl / 64, ln = rl % 64;
    RowPtrs rp{(gptr_u2)p.bits + ((t * nb) * 2 + h) * 64 + ln, (gptr_u4)p.scales + t * (nb8 / 8) * 64 + ln};
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (h == 0)
        half_row<0, NT>(tab, p, rp, nb, acc);
    else
        half_row<1, NT>(tab, p, rp, nb, acc);
    // The high half hands lanes 4..7 to the low half through LDS.
    __syncthreads();
    float4 *xch = reinterpret_cast<float4 *>(tab) + tl * 64 + lane;
    if (h == 1) *xch = make_float4(acc[0], acc[1], acc[2], acc[3]);
    __syncthreads();
    if (h == 0 && r < rows) {
        const float4 hi = *xch;
        p.y[r] = ((acc[0] + hi.x) + (acc[2] + hi.z)) + ((acc[1] + hi.y) + (acc[3] + hi.w));
    }
}

// NT threads: NT/2 rows per workgroup (256, or 128 when the 256-row grid
// would leave at least half the CUs without a workgroup).
template <int NT>
__global__ __launch_bounds__(NT) void q1_gemv_kernel(const uint32_t *bits, const uint4 *scales, const uint16_t *a,
                                                     float *y, int64_t rows, int64_t nb, int64_t nb8) {
    __shared__ float tab[kTableFloats];
    const int64_t c = blockIdx.y;   // activation column
    Q1Args p{bits, scales, a + c * (nb * 4) * 17, y + c * rows};
    q1_gemv_body<NT>(p, tab, rows, nb, nb8);
}

template <int NT>
__global__ __launch_bounds__(NT) void q1_gemv_grouped_kernel(const gd_q1_problem *probs, int64_t rows, int64_t nb,
                                                             int64_t nb8) {
    __shared__ float tab[kTableFloats];
    const gd_q1_problem pr = probs[blockIdx.y];
    const int64_t prow = (pr.rows >= 1 && pr.rows <= rows) ? pr.rows : rows;
    if (static_cast<int64_t>(blockIdx.x) * (NT / 2) >= prow) return;   // uniform: before any barrier
    Q1Args p{static_cast<const uint32_t *>(pr.bits_plane), static_cast<const uint4 *>(pr.scale_plane),
             static_cast<const uint16_t *>(pr.a_q8), pr.y};
    q1_gemv_body<NT>(p, tab, prow, nb, nb8);
}

// Grouped problems with K = 8*NG blocks (NG = 2..4 full groups, one table
// chunk): a workgroup runs UN consecutive 256-row units of one problem. They
// all use the activation's one table, built once; each unit's first two
// groups are loaded while the previous unit's last two are computed (the
// refills of the flat group sequence simply run on into the next unit); and
// the workgroup's start (the problem's descriptor, the first loads, the
// table build) is paid once per UN units. Each unit's outputs meet through
// LDS slots of their own, so the table stays intact. Same reads and
// arithmetic as above, so the same bits.
template <int H>
__device__ __forceinline__ void unit_tree(float4 *slot, const float (&acc)[4], float *y, int64_t r, int64_t prow,
                                          bool first) {
    // The sums are needed only after the barrier on the low half, which would
    // let the compiler sink the whole unit's arithmetic past it and hold every
    // table read until then: pin them here.
    asm volatile("" ::"v"(acc[0]), "v"(acc[1]), "v"(acc[2]), "v"(acc[3]));
    if (!first) __syncthreads();   // the previous unit's values have been read
    if (H == 1) *slot = make_float4(acc[0], acc[1], acc[2], acc[3]);
    __syncthreads();
    if (H == 0 && r < prow) {
        const float4 hi = *slot;
        y[r] = ((acc[0] + hi.x) + (acc[2] + hi.z)) + ((acc[1] + hi.y) + (acc[3] + hi.w));
    }
}

// Group F of the flat sequence (unit F / NG, group F % NG), refilling its
// register set with group F + 2 of the sequence.
template <int H, int NG, int UN, int F>
__device__ __forceinline__ void unit_seq(const char *tabc, u32x2 (&w0)[8], u32x2 (&w1)[8], u32x4 &s0, u32x4 &s1,
                                         float (&acc)[4], const RowPtrs (&rp)[UN], float4 *slot, float *y,
                                         const int64_t (&r)[UN], int64_t prow, int live) {
    if constexpr (F < UN * NG) {
        constexpr int FT = F + 2;
        constexpr bool REF = FT < UN * NG;
        constexpr int TU = REF ? FT / NG : 0, TG = REF ? FT % NG : 0;
        if constexpr (F % 2 == 0)
            group8<H, 8 * (F % NG), REF>(tabc, w0, s0, acc, rp[TU], TG);
        else
            group8<H, 8 * (F % NG), REF>(tabc, w1, s1, acc, rp[TU], TG);
        if constexpr (F % NG == NG - 1) {
            constexpr int U = F / NG;
            unit_tree<H>(slot, acc, y, r[U], prow, U == 0);
            if constexpr (U + 1 < UN) {
                if (live <= U + 1) return;   // uniform: no further unit in this problem
#pragma unroll
                for (int i = 0; i < 4; i++) acc[i] = 0.0f;
            }
        }
        unit_seq<H, NG, UN, F + 1>(tabc, w0, w1, s0, s1, acc, rp, slot, y, r, prow, live);
    }
}

template <int NG, int UN>
__global__ __launch_bounds__(kGroupedThreads) void q1_gemv_grouped2_kernel(const gd_q1_problem *probs, int64_t rows) {
    constexpr int NT = kGroupedThreads;
    constexpr int64_t nb = 8 * NG, nb8 = nb;
    __shared__ float tab[kTableFloats];
    __shared__ float4 xch[NT / 128][64];
    const gd_q1_problem pr = probs[blockIdx.y];
    const int64_t prow = (pr.rows >= 1 && pr.rows <= rows) ? pr.rows : rows;
    const int64_t u0 = static_cast<int64_t>(blockIdx.x) * UN;    // first unit of 256 rows
    if (u0 * (NT / 2) >= prow) return;                           // uniform: before any barrier
    const int64_t units_left = (prow + NT / 2 - 1) / (NT / 2) - u0;
    const int live = static_cast<int>(units_left < UN ? units_left : UN);
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int tl = wave >> 1, h = wave & 1;
    const int64_t r64 = (prow + 63) / 64 * 64;
    int64_t r[UN];
    RowPtrs rp[UN];
#pragma unroll
    for (int u = 0; u < UN; u++) {
        r[u] = (u0 + u) * (NT / 2) + tl * 64 + lane;
        // rows past the padded rows (and missing units) read the last
        // padded row: never stored
        const int64_t rl = r[u] < r64 ? r[u] : r64 - 1;
        const int64_t t = rl / 64, ln = rl % 64;
        rp[u] = RowPtrs{(gptr_u2)pr.bits_plane + ((t * nb) * 2 + h) * 64 + ln,
                        (gptr_u4)pr.scale_plane + t * (nb8 / 8) * 64 + ln};
    }
    TableRaw raw;
    table_loads<NT>(raw, static_cast<const uint16_t *>(pr.a_q8), 0, static_cast<int>(nb));
    asm volatile("" ::: "memory");   // the table's loads go first
    u32x2 w0[8], w1[8];
    u32x4 s0, s1;
    load_group(rp[0], 0, w0, s0, true);
    load_group(rp[1 / NG], 1 % NG, w1, s1, true);
    table_store<NT>(tab, raw, static_cast<int>(nb));
    __syncthreads();
    const char *tabc = reinterpret_cast<const char *>(tab);
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float4 *slot = &xch[tl][lane];
    if (h == 0)
        unit_seq<0, NG, UN, 0>(tabc, w0, w1, s0, s1, acc, rp, slot, pr.y, r, prow, live);
    else
        unit_seq<1, NG, UN, 0>(tabc, w0, w1, s0, s1, acc, rp, slot, pr.y, r, prow, live);
}

// Grouped problems with K <= 1024: one group of at most eight blocks per
// row, so one table build per workgroup and no chunk loop. Each workgroup
// (NT threads: NT/2 rows, two waves per 64-row tile as above) stages its
// problem's activation into a 16 KiB table, loads its rows' blocks once and
// runs the same table reads and arithmetic (group8 for eight blocks, the
// tail steps for fewer), so the bits are those of the general kernel; the
// smaller table and register set let more workgroups share a CU, which
// hides the latency that a workgroup's single short pass otherwise exposes.
constexpr int kSmallBlocks = 8;
constexpr int kSmallThreads = 256;   // 128 rows per workgroup
// 128-row units per workgroup at K = 1024: two measured 1.5 % faster than one
// on 7,646 problems of 256 rows; three and four slower (the second register
// set and the row pointers cost occupancy: 94 to 116 VGPRs against 65).
constexpr int kSmallUnitsPerWG = 2;

template <int NT>
__global__ __launch_bounds__(NT) void q1_gemv_grouped_small_kernel(const gd_q1_problem *probs, int64_t rows,
                                                                   int64_t nb) {
    static_assert(NT >= 256, "one table group per thread at most");
    __shared__ __attribute__((aligned(16))) float tab[kSmallBlocks * 512];
    const gd_q1_problem pr = probs[blockIdx.y];
    const int64_t prow = (pr.rows >= 1 && pr.rows <= rows) ? pr.rows : rows;
    if (static_cast<int64_t>(blockIdx.x) * (NT / 2) >= prow) return;   // uniform: before any barrier
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int tl = wave >> 1, h = wave & 1;
    const int64_t r = static_cast<int64_t>(blockIdx.x) * (NT / 2) + tl * 64 + lane;
    const int64_t r64 = (prow + 63) / 64 * 64;
    const int64_t rl = r < r64 ? r : r64 - 1;   // padded rows: same work, never stored
    const int64_t t = rl / 64, ln = rl % 64;
    // nb <= 8: the scale plane holds one 8-block group per row
    const RowPtrs rp{(gptr_u2)pr.bits_plane + ((t * nb) * 2 + h) * 64 + ln,
                     (gptr_u4)pr.scale_plane + t * 64 + ln};
    // 1. the activation's table groups first (one per thread), so the table
    //    build waits for them only
    const int ng = static_cast<int>(nb) * 32;
    const auto a = (const uint16_t __attribute__((address_space(1))) *)pr.a_q8;
    const int g = static_cast<int>(threadIdx.x) < ng ? static_cast<int>(threadIdx.x) : ng - 1;
    const auto blk = a + ((g >> 5) * 4 + ((g >> 3) & 3)) * 17;   // 34 bytes = 17 halves
    const uint32_t rd = blk[0], rq01 = blk[1 + 2 * (g & 7)], rq23 = blk[2 + 2 * (g & 7)];
    asm volatile("" ::: "memory");
    // 2. this row half's blocks (each read once when there are eight; fewer
    //    repeat the last one, which plain loads then find in cache)
    u32x2 wb[kSmallBlocks];
    u32x4 s8;
    if (nb == kSmallBlocks) {
        load_group(rp, 0, wb, s8, true);
    } else {
#pragma unroll
        for (int u = 0; u < kSmallBlocks; u++) wb[u] = rp.bits[(u < nb ? u : nb - 1) * 128];
        s8 = rp.sc[0];
    }
    // 3. the table
    if (static_cast<int>(threadIdx.x) < ng) table_group(tab + threadIdx.x * 16, rd, rq01, rq23);
    __syncthreads();
    // 4. the blocks, in order
    const char *tabc = reinterpret_cast<const char *>(tab);
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (nb == kSmallBlocks) {
        if (h == 0)
            group8<0, 0, false>(tabc, wb, s8, acc, rp, 0);
        else
            group8<1, 0, false>(tabc, wb, s8, acc, rp, 0);
    } else {
#pragma unroll
        for (int u = 0; u < kSmallBlocks; u++) {
            if (u < nb) {   // uniform
                if (h == 0)
                    tail_block<0>(tabc + u * 2048, wb[u], d0_of(s8, u), acc);
                else
                    tail_block<1>(tabc + u * 2048, wb[u], d0_of(s8, u), acc);
            }
        }
    }
    // 5. the high half hands lanes 4..7 to the low half through LDS
    __syncthreads();
    float4 *xch = reinterpret_cast<float4 *>(tab) + tl * 64 + lane;
    if (h == 1) *xch = make_float4(acc[0], acc[1], acc[2], acc[3]);
    __syncthreads();
    if (h == 0 && r < prow) {
        const float4 hi = *xch;
        pr.y[r] = ((acc[0] + hi.x) + (acc[2] + hi.z)) + ((acc[1] + hi.y) + (acc[3] + hi.w));
    }
}

// K = 1024 (one group of eight blocks per row) with UN consecutive 128-row
// units per workgroup: one 16 KiB table for all of them, each unit's blocks
// loaded two units ahead (two register sets), the start paid once per UN
// units. Same reads and arithmetic as above, so the same bits.
template <int UN>
__global__ __launch_bounds__(kSmallThreads) void q1_gemv_grouped_small2_kernel(const gd_q1_problem *probs,
                                                                              int64_t rows) {
    constexpr int NT = kSmallThreads;
    constexpr int64_t nb = kSmallBlocks;
    __shared__ __attribute__((aligned(16))) float tab[kSmallBlocks * 512];
    __shared__ float4 xch[NT / 128][64];
    const gd_q1_problem pr = probs[blockIdx.y];
    const int64_t prow = (pr.rows >= 1 && pr.rows <= rows) ? pr.rows : rows;
    const int64_t u0 = static_cast<int64_t>(blockIdx.x) * UN;    // first unit of 128 rows
    if (u0 * (NT / 2) >= prow) return;                           // uniform: before any barrier
    const int64_t units_left = (prow + NT / 2 - 1) / (NT / 2) - u0;
    const int live = static_cast<int>(units_left < UN ? units_left : UN);
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int tl = wave >> 1, h = wave & 1;
    const int64_t r64 = (prow + 63) / 64 * 64;
    int64_t r[UN];
    RowPtrs rp[UN];
#pragma unroll
    for (int u = 0; u < UN; u++) {
        r[u] = (u0 + u) * (NT / 2) + tl * 64 + lane;
        const int64_t rl = r[u] < r64 ? r[u] : r64 - 1;
        const int64_t t = rl / 64, ln = rl % 64;
        rp[u] = RowPtrs{(gptr_u2)pr.bits_plane + ((t * nb) * 2 + h) * 64 + ln, (gptr_u4)pr.scale_plane + t * 64 + ln};
    }
    // the activation's table groups first (one per thread)
    const auto a = (const uint16_t __attribute__((address_space(1))) *)pr.a_q8;
    const int g = threadIdx.x;   // 256 groups, 256 threads
    const auto blk = a + ((g >> 5) * 4 + ((g >> 3) & 3)) * 17;
    const uint32_t rd = blk[0], rq01 = blk[1 + 2 * (g & 7)], rq23 = blk[2 + 2 * (g & 7)];
    asm volatile("" ::: "memory");
    u32x2 w0[8], w1[8];
    u32x4 s0, s1;
    load_group(rp[0], 0, w0, s0, true);
    load_group(rp[UN > 1 ? 1 : 0], 0, w1, s1, true);
    table_group(tab + threadIdx.x * 16, rd, rq01, rq23);
    __syncthreads();
    const char *tabc = reinterpret_cast<const char *>(tab);
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float4 *slot = &xch[tl][lane];
    if (h == 0)
        unit_seq<0, 1, UN, 0>(tabc, w0, w1, s0, s1, acc, rp, slot, pr.y, r, prow, live);
    else
        unit_seq<1, 1, UN, 0>(tabc, w0, w1, s0, s1, acc, rp, slot, pr.y, r, prow, live);
}

// -------------------------------------------------- one GEMV, few rows
// A lone GEMV with few row tiles (a decode step's projection) leaves most
// CUs idle under the 256-row mapping, and each of its threads walks four
// chains through every block. Here a thread runs ONE chain l of one row: a
// wave covers 16 rows and the four chains of half H (lanes 16j..16j+15 run
// chain 4H + j), and a workgroup of WAVES waves covers 8*WAVES rows, so the
// same GEMV occupies 4-16 times more waves with a quarter of the arithmetic
// each. The chain order, and so every bit, is that of the kernels above.
// A chain's byte of each weight word is lane-dependent, so its offsets come
// from a rotate by a per-lane amount and one and-or that also adds the
// chain's table base; the block and sub-block parts stay immediate offsets.
// Every load of a 32-block chunk is issued at once: weights, their scales
// and the next chunk's activations, the weights of the next chunk refilled
// into each block's registers as soon as that block's offsets are taken.
struct LatLane {
    uint32_t sh0, sh1;   // rotate amounts: sub-blocks 2m and 2m+1 of word m
    uint32_t lbase;      // byte offset of this chain's tables within a sub-block
};

// (w rotated right by sh) & 0x3c, or-ed with the table base: the nibble's
// byte offset, pre-shifted by 2. One v_and_or_b32 (the compiler would turn
// the or into an add and split it in two).
__device__ __forceinline__ uint32_t lat_off(uint32_t w, uint32_t sh, uint32_t lbase) {
    const uint32_t rot = __builtin_amdgcn_alignbit(w, w, sh);
    uint32_t r;
    asm("v_and_or_b32 %0, %1, 60, %2" : "=v"(r) : "v"(rot), "v"(lbase));
    return r;
}

// The four table reads of chunk block u for this lane's chain (u is a
// constant in every unrolled use, so its part of the offset is immediate).
__device__ __forceinline__ void lat_reads(const char *tab, int u, const u32x2 &wb, const LatLane &ln,
                                          float (&v)[4]) {
    const char *t = tab + u * 2048;
    v[0] = *reinterpret_cast<const float *>(t + 0 * 512 + lat_off(wb.x, ln.sh0, ln.lbase));
    v[1] = *reinterpret_cast<const float *>(t + 1 * 512 + lat_off(wb.x, ln.sh1, ln.lbase));
    v[2] = *reinterpret_cast<const float *>(t + 2 * 512 + lat_off(wb.y, ln.sh0, ln.lbase));
    v[3] = *reinterpret_cast<const float *>(t + 3 * 512 + lat_off(wb.y, ln.sh1, ln.lbase));
}

__device__ __forceinline__ void lat_math(const float (&v)[4], float d0, float &acc) {
    float ab = v[0];
    ab = ab + v[1];
    ab = ab + v[2];
    ab = ab + v[3];
    acc = __builtin_fmaf(d0, ab, acc);
}

struct LatBuf {
    u32x2 w[kChunkBlocks];
    u32x4 s[kChunkBlocks / 8];
};

// Block i of chunk c (clamped to the last block; scale groups to the last
// padded group) into the register of slot u.
__device__ __forceinline__ u32x2 lat_wload(const RowPtrs &rp, int64_t c, int u, int64_t nb) {
    int64_t i = c * kChunkBlocks + u;
    i = i < nb ? i : nb - 1;
    return rp.bits[i * 128];
}

__device__ __forceinline__ u32x4 lat_sload(const RowPtrs &rp, int64_t c, int g, int64_t ng8) {
    int64_t gi = c * (kChunkBlocks / 8) + g;
    gi = gi < ng8 ? gi : ng8 - 1;
    return rp.sc[gi * 64];
}

__device__ __forceinline__ void lat_load(const RowPtrs &rp, int64_t c, int64_t nb, int64_t ng8, LatBuf &b) {
#pragma unroll
    for (int u = 0; u < kChunkBlocks; u++) b.w[u] = lat_wload(rp, c, u, nb);
#pragma unroll
    for (int g = 0; g < kChunkBlocks / 8; g++) b.s[g] = lat_sload(rp, c, g, ng8);
}

// A full chunk in straight-line code: the reads of block u+2 are issued
// before block u's arithmetic (the scheduler would otherwise batch each
// block's reads with its own arithmetic and wait for them); with REFILL,
// block u's register then takes block u of chunk cn, and a scale group's
// register its successor once its last d0 has been read.
template <bool REFILL>
__device__ __forceinline__ void lat_chunk(const char *tab, LatBuf &b, const LatLane &ln, float &acc,
                                          const RowPtrs &rp, int64_t cn, int64_t nb, int64_t ng8) {
    constexpr int D = 2;   // blocks of read lookahead
    float v[D + 1][4];
#pragma unroll
    for (int u = 0; u < D; u++) lat_reads(tab, u, b.w[u], ln, v[u]);
#pragma unroll
    for (int u = 0; u < kChunkBlocks; u++) {
        if (u + D < kChunkBlocks) lat_reads(tab, u + D, b.w[u + D], ln, v[(u + D) % (D + 1)]);
        if constexpr (REFILL) b.w[u] = lat_wload(rp, cn, u, nb);
        __builtin_amdgcn_sched_barrier(0);
        lat_math(v[u % (D + 1)], d0_of(b.s[u / 8], u % 8), acc);
        if constexpr (REFILL) {
            if (u % 8 == 7) b.s[u / 8] = lat_sload(rp, cn, u / 8, ng8);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The last chunk when it holds fewer than 32 blocks: the same steps, block
// by block, guarded by the (uniform) block count.
__device__ __forceinline__ void lat_chunk_short(const char *tab, const LatBuf &b, const LatLane &ln, float &acc,
                                                int cb) {
#pragma unroll
    for (int u = 0; u < kChunkBlocks; u++) {
        if (u < cb) {
            float v[4];
            lat_reads(tab, u, b.w[u], ln, v);
            lat_math(v, d0_of(b.s[u / 8], u % 8), acc);
        }
    }
}

// blockIdx.y is the activation column: each column is its own batch-1 GEMV.
template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void q1_gemv_lat_kernel(const uint32_t *bits, const uint4 *scales,
                                                                 const uint16_t *a_all, float *y_all, int64_t rows,
                                                                 int64_t nb, int64_t nb8) {
    constexpr int NT = WAVES * 64;
    constexpr int R = 8 * WAVES;   // rows per workgroup
    __shared__ float tab[kTableFloats];
    __shared__ float xch[R * 8];
    const uint16_t *a = a_all + static_cast<int64_t>(blockIdx.y) * (nb * 4) * 17;
    float *y = y_all + static_cast<int64_t>(blockIdx.y) * rows;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int h = wave & 1, j = lane >> 4;
    const int rloc = (wave >> 1) * 16 + (lane & 15);
    const int64_t r = static_cast<int64_t>(blockIdx.x) * R + rloc;
    const int64_t r64 = (rows + 63) / 64 * 64;
    const int64_t rl = r < r64 ? r : r64 - 1;   // padded rows: same work, never stored
    const int64_t t = rl / 64, lnr = rl % 64;
    const RowPtrs rp{(gptr_u2)bits + ((t * nb) * 2 + h) * 64 + lnr, (gptr_u4)scales + t * (nb8 / 8) * 64 + lnr};
    const LatLane ln{static_cast<uint32_t>(8 * j), static_cast<uint32_t>(8 * j + 4),
                     static_cast<uint32_t>((4 * h + j) * 64)};
    const char *tabc = reinterpret_cast<const char *>(tab);
    const int64_t nch = (nb + kChunkBlocks - 1) / kChunkBlocks, ng8 = nb8 / 8;
    auto blocks_in = [&](int64_t c) {
        const int64_t left = nb - c * kChunkBlocks;
        return static_cast<int>(left < kChunkBlocks ? left : kChunkBlocks);
    };

    TableRawN<NT> raw;
    table_loads<NT>(raw, a, 0, blocks_in(0));
    asm volatile("" ::: "memory");   // activations first: the table build waits for them only
    LatBuf b;
    lat_load(rp, 0, nb, ng8, b);
    table_store<NT>(tab, raw, blocks_in(0));
    __syncthreads();
    float acc = 0.0f;
    for (int64_t c = 0; c < nch; c++) {
        const int64_t cn = (c + 1 < nch) ? c + 1 : c;   // the next chunk, clamped
        table_loads<NT>(raw, a, cn * kChunkBlocks, blocks_in(cn));
        asm volatile("" ::: "memory");
        const int cb = blocks_in(c);
        if (cb < kChunkBlocks)
            lat_chunk_short(tabc, b, ln, acc, cb);   // only ever the last chunk
        else if (c + 1 < nch)
            lat_chunk<true>(tabc, b, ln, acc, rp, cn, nb, ng8);
        else
            lat_chunk<false>(tabc, b, ln, acc, rp, cn, nb, ng8);
        if (c + 1 < nch) {
            __syncthreads();
            table_store<NT>(tab, raw, blocks_in(cn));
            __syncthreads();
        }
    }
    // The eight chains of a row meet in LDS for the fixed final tree.
    xch[rloc * 8 + 4 * h + j] = acc;
    __syncthreads();
    if (threadIdx.x < R) {
        const int64_t ro = static_cast<int64_t>(blockIdx.x) * R + threadIdx.x;
        const float *x = xch + threadIdx.x * 8;
        if (ro < rows) y[ro] = ((x[0] + x[4]) + (x[2] + x[6])) + ((x[1] + x[5]) + (x[3] + x[7]));
    }
}

// ------------------------------------------------------------ validation
int plane_sizes(int64_t rows, int64_t K, int64_t *bits_bytes, int64_t *scale_bytes) {
    GD_REQUIRE(rows >= 1 && K >= 1, GD_EINVAL, "rows (%lld) and K (%lld) must be >= 1", (long long)rows,
               (long long)K);
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

extern "C" int q1_q8_gemv(const void *bits_plane, const void *scale_plane, const void *a_q8, float *y, int64_t rows,
                          int64_t K, int64_t n_act, void *stream) {
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
    hipStream_t hs = as_stream(stream);
    const uint32_t *bp = static_cast<const uint32_t *>(bits_plane);
    const uint4 *sp = static_cast<const uint4 *>(scale_plane);
    const uint16_t *ap = static_cast<const uint16_t *>(a_q8);
    if (gx <= kLatMaxRowBlocks && (n_act == 1 || n_act * rows <= kLatMaxColumnRows)) {
        // One chain per thread, each column its own GEMV (blockIdx.y). A
        // wave is 16 rows whatever the workgroup, so 16-row workgroups (two
        // waves) while 32-row ones would fill at most half the CUs, 32-row
        // workgroups (one wave per SIMD) until they would stack on the CUs,
        // then 64-row ones, which build half as many tables.
        const uint32_t cols = static_cast<uint32_t>(n_act);
        if (rows >= kLatWideRows) {
            hipLaunchKernelGGL(q1_gemv_lat_kernel<8>, dim3(static_cast<uint32_t>((rows + 63) / 64), cols), dim3(512),
                               0, hs, bp, sp, ap, y, rows, nb, nb8);
        } else if ((rows + 31) / 32 * n_act <= kNarrowMaxWGs && nb <= kChunkBlocks) {
            // 32-row workgroups would leave at least half the CUs idle: 16-row
            // ones (two waves) use all of them. Each builds the whole table
            // with half the threads, which pays for one table (K <= 4096) and
            // not for several rebuilt along K (4096 x 11008: 13.5 -> 14.2 us);
            // 2560 x 2560 5.92 -> 5.56 us, 4096 x 4096 6.05 -> 5.92 us.
            hipLaunchKernelGGL(q1_gemv_lat_kernel<2>, dim3(static_cast<uint32_t>((rows + 15) / 16), cols), dim3(128),
                               0, hs, bp, sp, ap, y, rows, nb, nb8);
        } else {
            hipLaunchKernelGGL(q1_gemv_lat_kernel<4>, dim3(static_cast<uint32_t>((rows + 31) / 32), cols), dim3(256),
                               0, hs, bp, sp, ap, y, rows, nb, nb8);
        }
        return check_launch("q1_q8_gemv");
    }
    // Each column its own four-chain GEMV (blockIdx.y). Groups of columns that
    // share one read of the weights through LDS tables of several columns
    // (P1's Q1_MM4) measured slower at every n_act from 2 to 32: they halve
    // the independent chains per column group, and these launches are bound
    // by VALU latency, not by the weight stream (the re-reads hit L2 / MALL).
    // While the 256-row grid would give at most half the CUs a workgroup,
    // 128-row workgroups put twice as many CUs to work (each builds the
    // whole table for half the rows).
    if (gx * n_act <= kNarrowMaxWGs) {
        const int64_t gx2 = (rows + kRowsPerWG / 2 - 1) / (kRowsPerWG / 2);
        hipLaunchKernelGGL(q1_gemv_kernel<kThreads / 2>, dim3(static_cast<uint32_t>(gx2), static_cast<uint32_t>(n_act)),
                           dim3(kThreads / 2), 0, hs, bp, sp, ap, y, rows, nb, nb8);
        return check_launch("q1_q8_gemv");
    }
    hipLaunchKernelGGL(q1_gemv_kernel<kThreads>, dim3(static_cast<uint32_t>(gx), static_cast<uint32_t>(n_act)),
                       dim3(kThreads), 0, hs, bp, sp, ap, y, rows, nb, nb8);
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
    if (nb == kSmallBlocks) {   // one whole group per row: kSmallUnitsPerWG units per workgroup
        constexpr int NT = kSmallThreads;
        constexpr int UN = kSmallUnitsPerWG;
        const int64_t gx = (rows + UN * (NT / 2) - 1) / (UN * (NT / 2));
        hipLaunchKernelGGL(q1_gemv_grouped_small2_kernel<UN>,
                           dim3(static_cast<uint32_t>(gx), static_cast<uint32_t>(count)), dim3(NT), 0,
                           as_stream(stream), problems, rows);
        return check_launch("q1_q8_gemv_grouped");
    }
    if (nb <= kSmallBlocks) {   // one group of blocks per row
        constexpr int NT = kSmallThreads;
        const int64_t gx = (rows + NT / 2 - 1) / (NT / 2);
        hipLaunchKernelGGL(q1_gemv_grouped_small_kernel<NT>,
                           dim3(static_cast<uint32_t>(gx), static_cast<uint32_t>(count)), dim3(NT), 0,
                           as_stream(stream), problems, rows, nb);
        return check_launch("q1_q8_gemv_grouped");
    }
    constexpr int NT = kGroupedThreads;
    if (nb == 16 || nb == 24 || nb == 32) {   // full groups, one table chunk: kUnitsPerWG units per workgroup
        constexpr int UN = kUnitsPerWG;
        const dim3 grid(static_cast<uint32_t>((rows + UN * (NT / 2) - 1) / (UN * (NT / 2))),
                        static_cast<uint32_t>(count));
        if (nb == 16)
            hipLaunchKernelGGL((q1_gemv_grouped2_kernel<2, UN>), grid, dim3(NT), 0, as_stream(stream), problems, rows);
        else if (nb == 24)
            hipLaunchKernelGGL((q1_gemv_grouped2_kernel<3, UN>), grid, dim3(NT), 0, as_stream(stream), problems, rows);
        else
            hipLaunchKernelGGL((q1_gemv_grouped2_kernel<4, UN>), grid, dim3(NT), 0, as_stream(stream), problems, rows);
        return check_launch("q1_q8_gemv_grouped");
    }
    const int64_t gx = (rows + NT / 2 - 1) / (NT / 2);
    hipLaunchKernelGGL(q1_gemv_grouped_kernel<NT>, dim3(static_cast<uint32_t>(gx), static_cast<uint32_t>(count)),
                       dim3(NT), 0, as_stream(stream), problems, rows, nb, nb8);
    return check_launch("q1_q8_gemv_grouped");
}
