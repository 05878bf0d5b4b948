// common.h -- device building blocks shared by the HIP kernels of the
// speculative-sampling verification library (gfx950): launch geometry,
// logit storage types, 16-byte spans, online softmax and argmax merges,
// wave reductions, Philox4x32-10, input checks, and the row-statistics
// chunk pass that every verification streams its logit rows through.
//
// Internal header: included by every source of the library. Its names live
// in namespace spv, so that the kernels of one source can be instantiated
// on these types and launched from another.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include "spec_verify.h"

namespace spv {

constexpr int kThreads = 256;       // 4 waves of 64 lanes
constexpr int kWave = 64;
constexpr int kWaves = kThreads / kWave;
constexpr int kChunkBytes = 32768;  // one row-statistics item
constexpr int kTiles = 8;           // 16-byte vectors per thread per chunk
// A chunk is exactly kTiles tiles of one 16-byte vector per lane: the draw
// sums and the locate walk it tile by tile without a loop.
static_assert(kChunkBytes == kTiles * 256 * 16, "chunk geometry");
constexpr int kMaxLdsChunks = 256;  // chunk masses staged in LDS by the locate
// Draw-weight segments of a chunk, in element order: the scalar head, then
// one segment per (tile, wave) -- the 512 consecutive elements one wave
// reads in one tile -- tile-major, then the scalar tail.
constexpr int kSegs = kTiles * kWaves + 2;
constexpr int kTrStride = 68;       // LDS row of 64 lanes, skewed across banks
constexpr int kMaxNgram = SPEC_MAX_NGRAM;
constexpr int kFoldBatch = 8;       // partial loads in flight per lane when folding
constexpr int kDeviceVersion = 300;  // 0.3.0
// Early exit: positions below this one get a launch each; the rest share one.
constexpr int kEarlyExitSingle = 4;
// Draw grids up to this many workgroups (about 16 per CU) take their
// decisions inside k_draw; larger ones get a k_decide launch first.
constexpr int64_t kFoldDecisionItems = 4096;
// Row passes over at least this many chunks take two chunks per workgroup
// (chunk_pair_stats); smaller ones (a few rounds of the chip or less) keep
// one per workgroup, since fewer, longer workgroups there lengthen the tail.
constexpr int64_t kRowPairChunks = 16384;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte load

__host__ __device__ inline int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

// A 16-byte load of logits that are read once: the non-temporal hint keeps
// them from displacing reusable lines (measured: the row statistics stream
// 5% faster with it).
__device__ inline u32x4 stream_load(const u32x4 *p) { return __builtin_nontemporal_load(p); }

// ---------------------------------------------------------------------------
// Storage types: 16 bytes hold 4 fp32 or 8 bf16 logits.
// ---------------------------------------------------------------------------
struct F32 {
    using Elem = float;
    static constexpr int kVec = 4;
    static constexpr int kKeyBits = 32;  // order-preserving key of a logit (top-p)
    static constexpr uint32_t kNegInfWord = 0xff800000u;  // -inf
    __device__ static inline void unpack(const u32x4 v, float (&f)[kVec])
    {
        f[0] = __uint_as_float(v.x);
        f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z);
        f[3] = __uint_as_float(v.w);
    }
    __device__ static inline float at(const Elem *p, int64_t i) { return p[i]; }
};

struct BF16 {
    using Elem = uint16_t;  // raw bf16 bits; widening to fp32 is exact
    static constexpr int kVec = 8;
    static constexpr int kKeyBits = 16;
    static constexpr uint32_t kNegInfWord = 0xff80ff80u;  // two bf16 -inf
    __device__ static inline void unpack(const u32x4 v, float (&f)[kVec])
    {
        f[0] = __uint_as_float(v.x << 16);
        f[1] = __uint_as_float(v.x & 0xffff0000u);
        f[2] = __uint_as_float(v.y << 16);
        f[3] = __uint_as_float(v.y & 0xffff0000u);
        f[4] = __uint_as_float(v.z << 16);
        f[5] = __uint_as_float(v.z & 0xffff0000u);
        f[6] = __uint_as_float(v.w << 16);
        f[7] = __uint_as_float(v.w & 0xffff0000u);
    }
    __device__ static inline float at(const Elem *p, int64_t i)
    {
        return __uint_as_float((uint32_t)p[i] << 16);
    }
};

template <class D>
constexpr int64_t chunk_elems()
{
    return kChunkBytes / (int64_t)sizeof(typename D::Elem);
}

// Element range [s, e) of a row chunk split into a scalar head [s, a),
// groups of kVec elements [a, z) and a scalar tail [z, e). With `vec` the
// groups are 16-byte aligned and loaded as vectors.
struct Span {
    int64_t s, a, z, e, ngroups;
    bool vec;
};

template <class D>
__device__ inline Span make_span(const typename D::Elem *row, int64_t s, int64_t e)
{
    using E = typename D::Elem;
    const uintptr_t addr = (uintptr_t)(row + s);
    const int64_t head = (int64_t)(((16u - (addr & 15u)) & 15u) / sizeof(E));
    Span sp;
    sp.s = s;
    sp.e = e;
    sp.a = min64(e, s + head);
    sp.ngroups = (e - sp.a) / D::kVec;
    sp.z = sp.a + sp.ngroups * D::kVec;
    sp.vec = true;
    return sp;
}

// Span for reading two rows at once: vectors only if both share alignment.
template <class D>
__device__ inline Span make_span2(const typename D::Elem *r1, const typename D::Elem *r2,
                                  int64_t s, int64_t e)
{
    Span sp = make_span<D>(r1, s, e);
    if (((uintptr_t)(r1 + s) & 15u) != ((uintptr_t)(r2 + s) & 15u)) {
        sp.a = s;
        sp.ngroups = (e - s) / D::kVec;
        sp.z = s + sp.ngroups * D::kVec;
        sp.vec = false;
    }
    return sp;
}

template <class D>
__device__ inline void load_group(const typename D::Elem *row, const Span &sp, int64_t gi,
                                  float (&f)[D::kVec])
{
    if (sp.vec) {
        D::unpack(reinterpret_cast<const u32x4 *>(row + sp.a)[gi], f);
    } else {
#pragma unroll
        for (int j = 0; j < D::kVec; ++j)
            f[j] = D::at(row, sp.a + gi * D::kVec + j);
    }
}

// ---------------------------------------------------------------------------
// Online softmax statistics (Milakov & Gimelshein, "Online normalizer
// calculation for softmax", 2018): running max m of the raw logits and
// z = sum 2^((x - m) * scale), scale = log2(e) / tau.
// ---------------------------------------------------------------------------
struct Soft {
    float m, z;
};

__device__ inline float exp2_fast(float x)
{
    return __builtin_amdgcn_exp2f(x);  // v_exp_f32; exp2(-inf) = 0
}

// The row-statistics arithmetic is kept free of fused multiply-adds, so that
// every kernel that inlines it rounds the same way: the same chunk gives the
// same partial whichever kernel computes it.
__device__ inline Soft soft_merge(Soft a, Soft b, float scale)
{
#pragma clang fp contract(off)
    const float m = fmaxf(a.m, b.m);
    if (m == -INFINITY)
        return {m, 0.f};
    return {m, a.z * exp2_fast((a.m - m) * scale) + b.z * exp2_fast((b.m - m) * scale)};
}

template <int N>
__device__ inline void soft_update(Soft &st, const float (&x)[N], float scale)
{
#pragma clang fp contract(off)
    float bm = x[0];
#pragma unroll
    for (int j = 1; j < N; ++j)
        bm = fmaxf(bm, x[j]);
    const float m = fmaxf(st.m, bm);
    const float base = m == -INFINITY ? 0.f : m;  // a thread that saw only padding
    float z = st.z * exp2_fast((st.m - base) * scale);
#pragma unroll
    for (int j = 0; j < N; ++j)
        z += exp2_fast((x[j] - base) * scale);
    st.m = m;
    st.z = z;
}

struct ArgMax {
    float v;
    int32_t i;
};

__device__ inline ArgMax argmax_merge(ArgMax a, ArgMax b)
{
    return (b.v > a.v || (b.v == a.v && b.i < a.i)) ? b : a;
}

// ---------------------------------------------------------------------------
// Wave and block reductions (fixed order, independent of timing).
// ---------------------------------------------------------------------------
__device__ inline Soft wave_soft(Soft s, float scale)
{
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        Soft o{__shfl_xor(s.m, off, kWave), __shfl_xor(s.z, off, kWave)};
        s = soft_merge(s, o, scale);
    }
    return s;
}

__device__ inline ArgMax wave_argmax(ArgMax a)
{
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        ArgMax o{__shfl_xor(a.v, off, kWave), __shfl_xor(a.i, off, kWave)};
        a = argmax_merge(a, o);
    }
    return a;
}

__device__ inline double wave_sum(double v)
{
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    return v;
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds; each round
// multiplies counter words 0 and 2 by the Philox multipliers, keeps both
// halves of the products and mixes the high halves with words 1 and 3 and
// the round key; the key advances by the Weyl constants between rounds.
// ---------------------------------------------------------------------------
__device__ inline uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
        const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
        c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

__device__ inline float uniform24(uint32_t w)
{
    return (float)(w >> 8) * 0x1p-24f;  // exact: 24-bit integer times 2^-24
}

__host__ __device__ inline bool valid_len(int L, int k) { return L >= 0 && L <= k; }

__host__ __device__ inline bool valid_temp(float tau)
{
    return tau == 0.f || (tau >= FLT_MIN && tau <= FLT_MAX);  // NaN fails both
}

__device__ inline float temp_scale(float tau)
{
    return (float)(1.4426950408889634 / (double)tau);  // log2(e) / tau, rounded once
}

// Host helpers.
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

// LDS of the kernels.
struct RowShared {
    float a[kWaves], b[kWaves];
};
// ===========================================================================
// Row statistics of one chunk: returns the block's partial in thread 0.
// ===========================================================================
// Pieces shared by the general chunk pass and the full-chunk pass from
// preloaded registers, so that both give bit-identical partials.

// The softmax update of one block of kTiles 16-byte vectors per lane.
template <class D>
__device__ __forceinline__ void block_soft(Soft &st, const u32x4 (&r)[kTiles], float scale)
{
    constexpr int NX = kTiles * D::kVec;
    float x[NX];
#pragma unroll
    for (int u = 0; u < kTiles; ++u) {
        float f[D::kVec];
        D::unpack(r[u], f);
#pragma unroll
        for (int j = 0; j < D::kVec; ++j)
            x[u * D::kVec + j] = f[j];
    }
    soft_update(st, x, scale);
}

// The argmax update of one block; i0 is the id of the lane's first element
// of tile 0 (tile u starts u * kThreads vectors later).
template <class D>
__device__ __forceinline__ void block_argmax(ArgMax &am, const u32x4 (&r)[kTiles], int32_t i0)
{
#pragma unroll
    for (int u = 0; u < kTiles; ++u) {
        float f[D::kVec];
        D::unpack(r[u], f);
        const int32_t iu = i0 + u * kThreads * D::kVec;
#pragma unroll
        for (int j = 0; j < D::kVec; ++j)
            if (f[j] > am.v) am = ArgMax{f[j], iu + j};
    }
}

// Workgroup combines (waves through LDS), result in thread 0.
__device__ __forceinline__ float2 reduce_soft(Soft st, float scale, RowShared &sh, int tid)
{
    float2 out = make_float2(0.f, 0.f);
    st = wave_soft(st, scale);
    if ((tid & (kWave - 1)) == 0) {
        sh.a[tid / kWave] = st.m;
        sh.b[tid / kWave] = st.z;
    }
    __syncthreads();
    if (tid == 0) {
        Soft acc{sh.a[0], sh.b[0]};
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            acc = soft_merge(acc, Soft{sh.a[w], sh.b[w]}, scale);
        out = make_float2(acc.m, acc.z);
    }
    __syncthreads();  // sh is reused by the caller
    return out;
}

__device__ __forceinline__ float2 reduce_argmax(ArgMax am, RowShared &sh, int tid)
{
    float2 out = make_float2(0.f, 0.f);
    am = wave_argmax(am);
    if ((tid & (kWave - 1)) == 0) {
        sh.a[tid / kWave] = am.v;
        sh.b[tid / kWave] = __int_as_float(am.i);
    }
    __syncthreads();
    if (tid == 0) {
        ArgMax acc{sh.a[0], __float_as_int(sh.b[0])};
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            acc = argmax_merge(acc, ArgMax{sh.a[w], __float_as_int(sh.b[w])});
        out = make_float2(acc.v, __int_as_float(acc.i));
    }
    __syncthreads();  // sh is reused by the caller
    return out;
}

// `tid` in [0, kThreads): the lane's index among the kThreads lanes that
// share `sh` (two such groups may share a workgroup, calling in step: the
// function's barriers are workgroup-wide).
template <class D>
__device__ __forceinline__ float2 chunk_stats(const typename D::Elem *row, int64_t s, int64_t e,
                                              bool greedy, float scale, RowShared &sh,
                                              int tid = (int)threadIdx.x)
{
    const Span sp = make_span<D>(row, s, e);
    const u32x4 *vrow = reinterpret_cast<const u32x4 *>(row + sp.a);
    const u32x4 pad = {D::kNegInfWord, D::kNegInfWord, D::kNegInfWord, D::kNegInfWord};

    // A full block of kThreads * kTiles groups (every chunk but a row's last)
    // loads without per-load masking; a partial one pads with -inf, which
    // adds exact zeros to the sums and leaves the maxima alone.
    auto load_block = [&](int64_t base, u32x4 (&r)[kTiles]) {
        if (base + (int64_t)kThreads * kTiles <= sp.ngroups) {
            const u32x4 *blk = vrow + base;  // uniform; 32-bit lane offsets below
#pragma unroll
            for (int u = 0; u < kTiles; ++u)
                r[u] = stream_load(blk + (uint32_t)(u * kThreads + tid));
        } else {
#pragma unroll
            for (int u = 0; u < kTiles; ++u) {
                const int64_t vi = base + u * kThreads + tid;
                r[u] = vi < sp.ngroups ? stream_load(vrow + vi) : pad;
            }
        }
    };
    if (!greedy) {
        Soft st{-INFINITY, 0.f};
        for (int64_t base = 0; base < sp.ngroups; base += (int64_t)kThreads * kTiles) {
            u32x4 r[kTiles];
            load_block(base, r);
            block_soft<D>(st, r, scale);
        }
        {
            float x[2];
            const int64_t hi = sp.s + tid, ti = sp.z + tid;
            x[0] = hi < sp.a ? D::at(row, hi) : -INFINITY;
            x[1] = ti < sp.e ? D::at(row, ti) : -INFINITY;
            if (x[0] != -INFINITY || x[1] != -INFINITY)
                soft_update(st, x, scale);
        }
        return reduce_soft(st, scale, sh, tid);
    }
    ArgMax am{-INFINITY, INT32_MAX};
    // head, vectors, tail: each thread sees ascending ids
    if (sp.s + tid < sp.a) {
        const float x = D::at(row, sp.s + tid);
        if (x > am.v) am = ArgMax{x, (int32_t)(sp.s + tid)};
    }
    for (int64_t base = 0; base < sp.ngroups; base += (int64_t)kThreads * kTiles) {
        u32x4 r[kTiles];
        load_block(base, r);
        block_argmax<D>(am, r, (int32_t)(sp.a + (base + tid) * D::kVec));
    }
    if (sp.z + tid < sp.e) {
        const float x = D::at(row, sp.z + tid);
        if (x > am.v) am = ArgMax{x, (int32_t)(sp.z + tid)};
    }
    return reduce_argmax(am, sh, tid);
}

// Whether [s, e) of `row` is read by chunk_stats as one block and nothing
// else: 16-byte aligned at s, a whole number of vectors, at most one block
// (every chunk of a row with 16-byte aligned rows and V a multiple of kVec,
// its last chunk included).
template <class D>
__device__ inline bool single_block(const typename D::Elem *row, int64_t s, int64_t e)
{
    return ((uintptr_t)(row + s) & 15u) == 0 && (e - s) % D::kVec == 0 &&
           e - s <= (int64_t)kThreads * kTiles * D::kVec;
}

// The loads of such a chunk, padded with -inf past its end as chunk_stats
// pads a partial block.
template <class D>
__device__ __forceinline__ void load_single_block(const typename D::Elem *row, int64_t s,
                                                  int64_t e, int tid, u32x4 (&r)[kTiles])
{
    const u32x4 *blk = reinterpret_cast<const u32x4 *>(row + s);
    const int ngroups = (int)((e - s) / D::kVec);
    if (ngroups == kThreads * kTiles) {
#pragma unroll
        for (int u = 0; u < kTiles; ++u)
            r[u] = stream_load(blk + (uint32_t)(u * kThreads + tid));
    } else {
        const u32x4 pad = {D::kNegInfWord, D::kNegInfWord, D::kNegInfWord, D::kNegInfWord};
#pragma unroll
        for (int u = 0; u < kTiles; ++u) {
            const int vi = u * kThreads + tid;
            r[u] = vi < ngroups ? stream_load(blk + vi) : pad;
        }
    }
}

// chunk_stats of a single-block chunk whose block is already loaded: the
// same arithmetic (such a chunk has no head or tail elements).
template <class D>
__device__ __forceinline__ float2 chunk_stats_loaded(int64_t s, bool greedy, float scale,
                                                     RowShared &sh, int tid,
                                                     const u32x4 (&r)[kTiles])
{
    if (!greedy) {
        Soft st{-INFINITY, 0.f};
        block_soft<D>(st, r, scale);
        return reduce_soft(st, scale, sh, tid);
    }
    ArgMax am{-INFINITY, INT32_MAX};
    block_argmax<D>(am, r, (int32_t)(s + tid * D::kVec));
    return reduce_argmax(am, sh, tid);
}

// Whether chunks [c0, cend) of a row of V elements (nc chunks) are all
// single blocks: the row 16-byte aligned, and V a whole number of vectors if
// the range holds the row's last chunk.
template <class D>
__device__ inline bool chunks_single_blocks(const typename D::Elem *row, int64_t V, int nc,
                                            int cend)
{
    return ((uintptr_t)row & 15u) == 0 && (cend < nc || V % D::kVec == 0);
}

// Partials of chunk c0 of a row and, when c0 + 1 < cend, of chunk c0 + 1,
// both single blocks (chunks_single_blocks). Chunk c0's values fold into the
// lane's (max, sum) or argmax, then chunk c0 + 1's loads go out and stay in
// flight through chunk c0's reduction and its barriers. Each partial is the
// one chunk_stats gives. emit(c, partial) runs in thread 0, in chunk order.
template <class D, class Emit>
__device__ __forceinline__ void chunk_pair_stats(const typename D::Elem *row, int64_t V, int c0,
                                                 int cend, bool greedy, float scale,
                                                 RowShared &sh, int tid, Emit emit)
{
    constexpr int64_t CH = chunk_elems<D>();
    auto s_of = [&](int c) { return (int64_t)c * CH; };
    auto e_of = [&](int c) { return min64(V, (int64_t)(c + 1) * CH); };
    const int c1 = c0 + 1;
    const bool two = c1 < cend;
    u32x4 r[kTiles];
    load_single_block<D>(row, s_of(c0), e_of(c0), tid, r);
    Soft st{-INFINITY, 0.f};
    ArgMax am{-INFINITY, INT32_MAX};
    if (greedy)
        block_argmax<D>(am, r, (int32_t)(s_of(c0) + tid * D::kVec));
    else
        block_soft<D>(st, r, scale);
    if (two)
        load_single_block<D>(row, s_of(c1), e_of(c1), tid, r);
    const float2 v0 = greedy ? reduce_argmax(am, sh, tid) : reduce_soft(st, scale, sh, tid);
    if (tid == 0)
        emit(c0, v0);
    if (two) {
        const float2 v1 = chunk_stats_loaded<D>(s_of(c1), greedy, scale, sh, tid, r);
        if (tid == 0)
            emit(c1, v1);
    }
}

}  // namespace spv
