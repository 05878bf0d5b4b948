// spec_verify.hip -- HIP kernels and C ABI for the speculative-sampling
// verification step on MI355X (gfx950).
//
// The step, per sequence b with draft length L and temperature tau
// ("Speculative Decoding and the Art of Fast LLM Inference", "The Algorithm,
// Step by Step"; thelatentsource.com "speculative-decoding-llm-speed", "The
// correction that keeps the target in charge"; techaiinterview.com
// speculative-decoding question, "Core explanation" and "Deep dive"):
//
//   sampling: p_i = softmax(target_i / tau), q_i = softmax(draft_i / tau);
//             accept g_i while u_i < min(1, p_i(g_i) / q_i(g_i)); at the first
//             rejection j draw from norm(max(0, p_j - q_j)); if all L are
//             accepted draw a bonus token from p_L.
//   greedy:   accept g_i while it equals argmax(target_i); emit that argmax.
//
// Launches per call, all stream-ordered, no host synchronisation:
//
//   k_reset          zeroes the per-sequence counters and chunk claims.
//   k_verify         one workgroup per 32 KiB chunk of every logit row the
//                    step needs (b-major). Each streams its chunk once with
//                    16-byte loads and publishes an 8-byte partial: (max
//                    logit, sum 2^((x - max) * log2(e)/tau)) for sampling
//                    rows, (max logit, lowest index of it) for greedy rows.
//                    These items carry ~all of the HBM traffic. The item that
//                    completes a sequence only marks it ready. The items of
//                    target row 0 then, by a fixed rule, take the decision
//                    of an earlier sequence (fold the partials in chunk
//                    order, gather p_i(g_i) and q_i(g_i), draw Philox, run
//                    the left-to-right test, write the accepted prefix,
//                    publish row j, kind and uniform v) and sum, in fp64,
//                    one chunk of the draw weights w = max(0, p_j - q_j) (or
//                    p_L for a bonus) of a still earlier sequence, whose rows
//                    are still in the last-level cache.
//   k_finish_decide  decisions nobody took during k_verify (the last
//                    sequences, which have no later rows to help them);
//   k_finish_sums    draw-weight chunks nobody summed;
//   k_finish_locate  every sequence's token: the chunk where the cumulative
//                    weight passes v * S, then the 2048-element tile, then
//                    the lane, then the element, with coalesced loads and
//                    fp64 block scans.
//
// Work is assigned statically, never to "whoever arrives first or last":
// workgroup i runs on XCD i % 8, and any timing-driven hand-off would give
// the work to whichever XCD lags and make it lag further.
//
// Nothing here is a dense contraction, so there is no MFMA: the step is bound
// by HBM bandwidth. No workgroup ever waits for another: work that is not
// ready is left to the finishing launches.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include "spec_verify.h"

namespace {

constexpr int kThreads = 256;       // 4 waves of 64 lanes
constexpr int kWave = 64;
constexpr int kWaves = kThreads / kWave;
constexpr int kChunkBytes = 32768;  // one row-statistics item
constexpr int kTiles = 8;           // 16-byte vectors per thread per chunk
constexpr int kLagDecide = 32;      // target-row-0 items of sequence b decide b - kLagDecide
constexpr int kLagSum = 80;         // ... and sum one draw chunk of b - kLagSum
constexpr int kMaxLdsChunks = 256;  // chunk sums staged in LDS by the locate
constexpr int kFoldBatch = 8;       // partial loads in flight per lane when folding
constexpr int kDeviceVersion = 200;  // 0.2.0

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte load

__host__ __device__ inline int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

// ---------------------------------------------------------------------------
// Storage types: 16 bytes hold 4 fp32 or 8 bf16 logits.
// ---------------------------------------------------------------------------
struct F32 {
    using Elem = float;
    static constexpr int kVec = 4;
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

__device__ inline Soft soft_merge(Soft a, Soft b, float scale)
{
    const float m = fmaxf(a.m, b.m);
    if (m == -INFINITY)
        return {m, 0.f};
    return {m, a.z * exp2_fast((a.m - m) * scale) + b.z * exp2_fast((b.m - m) * scale)};
}

template <int N>
__device__ inline void soft_update(Soft &st, const float (&x)[N], float scale)
{
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

// ---------------------------------------------------------------------------
// Workspace records.
// ---------------------------------------------------------------------------
struct __align__(16) Decision {
    int32_t row;   // row of the final draw
    int32_t kind;  // SPEC_DRAW_*
    float v;       // draw uniform
    float scale;   // log2(e) / tau
    float mt, zt;  // target row: max logit, normaliser
    float md, zd;  // draft row (residual draws only)
};

// Per-sequence synchronisation, zeroed by k_reset at the start of each call.
struct __align__(16) SeqState {
    int32_t rows_done;  // row-statistics chunks finished
    int32_t flag;       // see below
    int32_t unused0, unused1;
};
// Life of a sequence: kPending (row statistics running) -> kReady (every
// partial published) -> kDraw (decision published; draw-weight chunks to
// sum, then the locate) or kDone (greedy or error: finished).
enum { kPending = 0, kReady = 1, kDraw = 2, kDone = 3 };

struct AuxDev {
    float *p_g, *q_g, *resid_mass;
    int32_t *argmax, *seq_status, *draw_row, *draw_kind;
};

struct Params {
    const void *target, *draft;
    const int32_t *draft_tokens, *draft_len;
    const float *temperature;
    int32_t k, V, nc, B;
    uint32_t key0, key1, seq_base;
    int64_t n_row_items;  // B * (2k+1) * nc
    float2 *partials;     // [B][2k+1][nc]
    Decision *decisions;  // [B]
    double2 *masses;      // [B][nc]: (sum w, sum p) per chunk of the drawn row
    SeqState *state;      // [B]
    int32_t *chunk_claim; // [B][nc]: draw-weight chunk summed (0 / 1)
    int32_t *out_tokens, *num_accepted;
    AuxDev aux;
};

// Cross-workgroup exchange. Published values are written with device-scope
// (write-through) stores and read with device-scope loads, so no L2
// write-back or invalidate is ever needed; a writer drains its stores
// (s_waitcnt) before the relaxed device-scope counter or flag update that
// tells readers to look. Agent-scope release/acquire would instead write
// back / invalidate the whole L2 on every item, which costs more than the
// streaming itself on this part.
__device__ inline void publish64(void *ptr, uint64_t v)
{
    __hip_atomic_store(static_cast<uint64_t *>(ptr), v, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t fetch64(const void *ptr)
{
    return __hip_atomic_load(static_cast<const uint64_t *>(ptr), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void drain_stores() { __builtin_amdgcn_s_waitcnt(0); }
__device__ inline int counter_add(int32_t *ptr, int32_t v)
{
    return __hip_atomic_fetch_add(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline int flag_load(const int32_t *ptr)
{
    return __hip_atomic_load(ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void flag_store(int32_t *ptr, int32_t v)
{
    __hip_atomic_store(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


__device__ inline void publish_pair(void *ptr, uint32_t lo, uint32_t hi)
{
    publish64(ptr, (uint64_t)lo | ((uint64_t)hi << 32));
}
__device__ inline float2 fetch_float2(const float2 *ptr)
{
    const uint64_t v = fetch64(ptr);
    return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}
__device__ inline double fetch_double(const double *ptr)
{
    return __longlong_as_double((long long)fetch64(ptr));
}
__device__ inline void publish_double(double *ptr, double v)
{
    publish64(ptr, (uint64_t)__double_as_longlong(v));
}

__device__ inline void publish_decision(Decision *dst, const Decision &d)
{
    publish_pair(reinterpret_cast<char *>(dst) + 0, (uint32_t)d.row, (uint32_t)d.kind);
    publish_pair(reinterpret_cast<char *>(dst) + 8, __float_as_uint(d.v), __float_as_uint(d.scale));
    publish_pair(reinterpret_cast<char *>(dst) + 16, __float_as_uint(d.mt), __float_as_uint(d.zt));
    publish_pair(reinterpret_cast<char *>(dst) + 24, __float_as_uint(d.md), __float_as_uint(d.zd));
}
__device__ inline Decision fetch_decision(const Decision *src)
{
    const char *c = reinterpret_cast<const char *>(src);
    const uint64_t a = fetch64(c), b = fetch64(c + 8), x = fetch64(c + 16), y = fetch64(c + 24);
    Decision d;
    d.row = (int32_t)(uint32_t)a;
    d.kind = (int32_t)(uint32_t)(a >> 32);
    d.v = __uint_as_float((uint32_t)b);
    d.scale = __uint_as_float((uint32_t)(b >> 32));
    d.mt = __uint_as_float((uint32_t)x);
    d.zt = __uint_as_float((uint32_t)(x >> 32));
    d.md = __uint_as_float((uint32_t)y);
    d.zd = __uint_as_float((uint32_t)(y >> 32));
    return d;
}

// LDS shared by the phases of k_verify (one phase at a time).
struct Shared {
    float a[kWaves], b[kWaves];
    double wd[kWaves][kTiles], pd[kWaves], ht[2][kWaves];
    double cm[kMaxLdsChunks];
    Decision dec;
    int i0, i1;
    int flag;
    int tok;
};

// ===========================================================================
// Row statistics of one chunk: returns the block's partial in thread 0.
// ===========================================================================
template <class D>
__device__ __forceinline__ float2 chunk_stats(const typename D::Elem *row, int64_t s, int64_t e, bool greedy,
                              float scale, Shared &sh)
{
    constexpr int NX = kTiles * D::kVec;
    const Span sp = make_span<D>(row, s, e);
    const u32x4 *vrow = reinterpret_cast<const u32x4 *>(row + sp.a);
    const int tid = threadIdx.x;
    const u32x4 pad = {D::kNegInfWord, D::kNegInfWord, D::kNegInfWord, D::kNegInfWord};
    float2 out = make_float2(0.f, 0.f);

    if (!greedy) {
        Soft st{-INFINITY, 0.f};
        for (int64_t base = 0; base < sp.ngroups; base += (int64_t)kThreads * kTiles) {
            u32x4 r[kTiles];
#pragma unroll
            for (int u = 0; u < kTiles; ++u) {
                const int64_t vi = base + u * kThreads + tid;
                r[u] = vi < sp.ngroups ? vrow[vi] : pad;
            }
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
        {
            float x[2];
            const int64_t hi = sp.s + tid, ti = sp.z + tid;
            x[0] = hi < sp.a ? D::at(row, hi) : -INFINITY;
            x[1] = ti < sp.e ? D::at(row, ti) : -INFINITY;
            if (x[0] != -INFINITY || x[1] != -INFINITY)
                soft_update(st, x, scale);
        }
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
    } else {
        ArgMax am{-INFINITY, INT32_MAX};
        // head, vectors, tail: each thread sees ascending ids
        if (sp.s + tid < sp.a) {
            const float x = D::at(row, sp.s + tid);
            if (x > am.v) am = ArgMax{x, (int32_t)(sp.s + tid)};
        }
        for (int64_t base = 0; base < sp.ngroups; base += (int64_t)kThreads * kTiles) {
            u32x4 r[kTiles];
#pragma unroll
            for (int u = 0; u < kTiles; ++u) {
                const int64_t vi = base + u * kThreads + tid;
                r[u] = vi < sp.ngroups ? vrow[vi] : pad;
            }
#pragma unroll
            for (int u = 0; u < kTiles; ++u) {
                float f[D::kVec];
                D::unpack(r[u], f);
                const int32_t i0 = (int32_t)(sp.a + (base + u * kThreads + tid) * D::kVec);
#pragma unroll
                for (int j = 0; j < D::kVec; ++j)
                    if (f[j] > am.v) am = ArgMax{f[j], i0 + j};
            }
        }
        if (sp.z + tid < sp.e) {
            const float x = D::at(row, sp.z + tid);
            if (x > am.v) am = ArgMax{x, (int32_t)(sp.z + tid)};
        }
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
    }
    __syncthreads();  // sh is reused by the caller
    return out;
}

// ===========================================================================
// Decision of one sequence (wave 0 of the deciding workgroup). Fills
// sh.dec; writes the accepted prefix, num_accepted and diagnostics.
// ===========================================================================
template <class D>
__device__ __forceinline__ void decide(const Params &p, int64_t b, Shared &sh)
{
    using E = typename D::Elem;
    const int lane = threadIdx.x;
    if (lane >= kWave)
        return;
    const int k = p.k, V = p.V, nc = p.nc, rows = 2 * k + 1;
    const E *target = static_cast<const E *>(p.target);
    const E *draft = static_cast<const E *>(p.draft);
    const int L = p.draft_len ? p.draft_len[b] : k;
    const float tau = p.temperature[b];
    int32_t *out = p.out_tokens + b * (k + 1);

    int status = SPEC_SEQ_OK;
    int g = -1;
    if (!valid_len(L, k)) {
        status = SPEC_SEQ_BAD_LEN;
    } else if (!valid_temp(tau)) {
        status = SPEC_SEQ_BAD_TEMP;
    } else {
        g = lane < L ? p.draft_tokens[b * k + lane] : -1;
        if (__any(lane < L && (g < 0 || g >= V)))
            status = SPEC_SEQ_BAD_TOKEN;
    }

    Decision dec;
    dec.row = -1;
    dec.kind = SPEC_DRAW_NONE;
    dec.v = dec.scale = dec.mt = dec.zt = dec.md = dec.zd = 0.f;
    float pg = NAN, qg = NAN;
    int amax = -1;

    if (status == SPEC_SEQ_OK && tau == 0.f) {
        // Greedy: target argmax of rows 0..L, folded in chunk order.
        if (lane <= L) {
            const float2 *pp = p.partials + (b * rows + lane) * (int64_t)nc;
            ArgMax acc{-INFINITY, INT32_MAX};
            for (int c0 = 0; c0 < nc; c0 += kFoldBatch) {
                float2 t[kFoldBatch];
#pragma unroll
                for (int q = 0; q < kFoldBatch; ++q)
                    t[q] = c0 + q < nc ? fetch_float2(pp + c0 + q)
                                       : make_float2(-INFINITY, __int_as_float(INT32_MAX));
#pragma unroll
                for (int q = 0; q < kFoldBatch; ++q)
                    acc = argmax_merge(acc, ArgMax{t[q].x, __float_as_int(t[q].y)});
            }
            amax = acc.i;
        }
        const uint64_t stop = __ballot(lane < L && amax != g);
        const int j = stop ? __ffsll((unsigned long long)stop) - 1 : L;
        const int tok = __shfl(amax, j, kWave);
        if (lane <= k)
            out[lane] = lane < j ? g : (lane == j ? tok : -1);
        dec.row = j;
        dec.kind = SPEC_DRAW_GREEDY;
        if (lane == 0)
            p.num_accepted[b] = j;
    } else if (status == SPEC_SEQ_OK) {
        const float scale = temp_scale(tau);
        Soft ts{-INFINITY, 0.f}, ds{-INFINITY, 0.f};
        if (lane <= L) {
            const float2 *pp = p.partials + (b * rows + lane) * (int64_t)nc;
            for (int c0 = 0; c0 < nc; c0 += kFoldBatch) {
                float2 t[kFoldBatch];
#pragma unroll
                for (int q = 0; q < kFoldBatch; ++q)
                    t[q] = c0 + q < nc ? fetch_float2(pp + c0 + q) : make_float2(-INFINITY, 0.f);
#pragma unroll
                for (int q = 0; q < kFoldBatch; ++q)
                    ts = soft_merge(ts, Soft{t[q].x, t[q].y}, scale);
            }
        }
        if (lane < L) {
            const float2 *pp = p.partials + (b * rows + k + 1 + lane) * (int64_t)nc;
            for (int c0 = 0; c0 < nc; c0 += kFoldBatch) {
                float2 t[kFoldBatch];
#pragma unroll
                for (int q = 0; q < kFoldBatch; ++q)
                    t[q] = c0 + q < nc ? fetch_float2(pp + c0 + q) : make_float2(-INFINITY, 0.f);
#pragma unroll
                for (int q = 0; q < kFoldBatch; ++q)
                    ds = soft_merge(ds, Soft{t[q].x, t[q].y}, scale);
            }
            const float xt = D::at(target + (b * (k + 1) + lane) * (int64_t)V, g);
            const float xd = D::at(draft + (b * k + lane) * (int64_t)V, g);
            pg = exp2_fast((xt - ts.m) * scale) / ts.z;
            qg = exp2_fast((xd - ds.m) * scale) / ds.z;
        }
        const uint4 w = philox4x32_10(
            make_uint4((uint32_t)lane, p.seq_base + (uint32_t)b, 0u, 0u), p.key0, p.key1);
        const float u = uniform24(w.x), v = uniform24(w.y);
        const bool qzero = lane < L && !(qg > 0.f);
        const bool reject = lane < L && !qzero && !(u < fminf(1.f, pg / qg));
        const uint64_t stop = __ballot(qzero || reject);
        const int j = stop ? __ffsll((unsigned long long)stop) - 1 : L;
        if (__shfl((int)qzero, j, kWave)) {
            status = SPEC_SEQ_QZERO;
        } else {
            if (lane <= k && lane != j)
                out[lane] = lane < j ? g : -1;  // position j: written by the locate
            dec.row = j;
            dec.kind = j < L ? SPEC_DRAW_RESIDUAL : SPEC_DRAW_BONUS;
            dec.v = __shfl(v, j, kWave);
            dec.scale = scale;
            dec.mt = __shfl(ts.m, j, kWave);
            dec.zt = __shfl(ts.z, j, kWave);
            dec.md = __shfl(ds.m, j, kWave);
            dec.zd = __shfl(ds.z, j, kWave);
            if (lane == 0)
                p.num_accepted[b] = j;
        }
    }

    if (status != SPEC_SEQ_OK) {
        if (lane <= k)
            out[lane] = -1;
        if (lane == 0)
            p.num_accepted[b] = 0;
        dec.row = -1;
        dec.kind = SPEC_DRAW_NONE;
        pg = qg = NAN;
        amax = -1;
    }
    const AuxDev &aux = p.aux;
    if (lane < k) {
        if (aux.p_g) aux.p_g[b * k + lane] = lane < L ? pg : NAN;
        if (aux.q_g) aux.q_g[b * k + lane] = lane < L ? qg : NAN;
    }
    if (aux.argmax && lane <= k)
        aux.argmax[b * (k + 1) + lane] = (lane <= L) ? amax : -1;
    if (lane == 0) {
        publish_decision(p.decisions + b, dec);
        sh.dec = dec;
        if (aux.seq_status) aux.seq_status[b] = status;
        if (aux.draw_row) aux.draw_row[b] = dec.row;
        // Each output address has exactly one writer (L2s of different XCDs
        // write back independently): for a residual or bonus draw the
        // locating workgroup owns draw_kind and resid_mass.
        if (dec.kind != SPEC_DRAW_RESIDUAL && dec.kind != SPEC_DRAW_BONUS) {
            if (aux.draw_kind) aux.draw_kind[b] = dec.kind;
            if (aux.resid_mass) aux.resid_mass[b] = NAN;
        }
    }
}

// Draw weight of one token: w = max(0, p - q) for a residual (p alone for a
// bonus), and p itself (for the rounding fallback), in fp32. The difference
// is exact whenever p and q are within a factor of two (Sterbenz) and off by
// at most half an ulp of a large difference otherwise. Every reader of a
// weight goes through here, so all of them see bit-identical values.
struct Weights {
    float w, p;
};

__device__ inline Weights draw_weights(float xt, float xd, const Decision &dec, float inv_zt,
                                       float inv_zd, bool resid)
{
    const float pt = exp2_fast((xt - dec.mt) * dec.scale) * inv_zt;
    if (!resid)
        return {pt, pt};
    const float pd = exp2_fast((xd - dec.md) * dec.scale) * inv_zd;
    return {fmaxf(pt - pd, 0.f), pt};
}

// Pairwise fp32 sum of one group's 8 or 4 weights (fixed association).
template <int N>
__device__ inline float pairwise(const float (&v)[N])
{
    if constexpr (N == 8)
        return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    else
        return (v[0] + v[1]) + (v[2] + v[3]);
}

// Rows and normalisers of a sequence's decided draw.
template <class D>
struct DrawRows {
    const typename D::Elem *t, *d;
    float inv_zt, inv_zd;
    bool resid;
};

template <class D>
__device__ inline DrawRows<D> draw_rows(const Params &p, int64_t b, const Decision &dec)
{
    using E = typename D::Elem;
    DrawRows<D> r;
    r.resid = dec.kind == SPEC_DRAW_RESIDUAL;
    r.t = static_cast<const E *>(p.target) + (b * (p.k + 1) + dec.row) * (int64_t)p.V;
    r.d = r.resid ? static_cast<const E *>(p.draft) + (b * p.k + dec.row) * (int64_t)p.V : r.t;
    r.inv_zt = 1.f / dec.zt;
    r.inv_zd = r.resid ? 1.f / dec.zd : 0.f;
    return r;
}

// Weight of element x (any alignment).
template <class D>
__device__ inline Weights elem_weight(const DrawRows<D> &r, int64_t x, const Decision &dec)
{
    return draw_weights(D::at(r.t, x), r.resid ? D::at(r.d, x) : 0.f, dec, r.inv_zt, r.inv_zd,
                        r.resid);
}

// Pairwise fp32 sums (w and p) of the weights of one group of kVec
// elements; `last` tracks the last element with a positive selected weight.
template <class D>
__device__ inline void group_weight_sums(const DrawRows<D> &r, const Span &sp, int64_t gi,
                                         const Decision &dec, bool use_p, float &gw, float &gp,
                                         int &last)
{
    float ft[D::kVec], fd[D::kVec];
    load_group<D>(r.t, sp, gi, ft);
    if (r.resid)
        load_group<D>(r.d, sp, gi, fd);
    float w[D::kVec], pw[D::kVec];
#pragma unroll
    for (int j = 0; j < D::kVec; ++j) {
        const Weights x = draw_weights(ft[j], r.resid ? fd[j] : 0.f, dec, r.inv_zt, r.inv_zd,
                                       r.resid);
        w[j] = x.w;
        pw[j] = x.p;
        if ((use_p ? x.p : x.w) > 0.f)
            last = (int)(sp.a + gi * D::kVec + j);
    }
    gw = pairwise(w);
    gp = pairwise(pw);
}

// ===========================================================================
// fp64 sums of the draw weights over one chunk of the decided row.
// ===========================================================================
template <class D>
__device__ __forceinline__ void chunk_weight_sums(const Params &p, int64_t b, int c, const Decision &dec,
                                  Shared &sh)
{
    constexpr int64_t CH = chunk_elems<D>();
    const DrawRows<D> r = draw_rows<D>(p, b, dec);
    const int64_t s = (int64_t)c * CH, e = min64((int64_t)p.V, s + CH);
    const Span sp = make_span2<D>(r.t, r.d, s, e);
    const int tid = threadIdx.x;
    double aw = 0.0, ap = 0.0;
    if (sp.vec) {
        // kBatch 16-byte loads per row in flight before their arithmetic,
        // then one group of arithmetic at a time (the fp64 sums are one
        // dependent chain; unfenced, the scheduler hoists every weight)
        constexpr int kBatch = kTiles / 2;
        const u32x4 *vt = reinterpret_cast<const u32x4 *>(r.t + sp.a);
        const u32x4 *vd = reinterpret_cast<const u32x4 *>(r.d + sp.a);
#pragma unroll
        for (int h = 0; h < kTiles; h += kBatch) {
            u32x4 lt[kBatch], ld[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int64_t gi = (int64_t)(h + u) * kThreads + tid;
                const bool in = gi < sp.ngroups;
                lt[u] = in ? vt[gi] : u32x4{0u, 0u, 0u, 0u};
                ld[u] = in && r.resid ? vd[gi] : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if ((int64_t)(h + u) * kThreads + tid < sp.ngroups) {
                    float ft[D::kVec], fd[D::kVec], w[D::kVec], pw[D::kVec];
                    D::unpack(lt[u], ft);
                    D::unpack(ld[u], fd);
#pragma unroll
                    for (int j = 0; j < D::kVec; ++j) {
                        const Weights x = draw_weights(ft[j], fd[j], dec, r.inv_zt, r.inv_zd,
                                                       r.resid);
                        w[j] = x.w;
                        pw[j] = x.p;
                    }
                    aw += (double)pairwise(w);
                    ap += (double)pairwise(pw);
                }
            }
        }
    } else {
        int unused = -1;
        for (int64_t gi = tid; gi < sp.ngroups; gi += kThreads) {
            float gw, gp;
            group_weight_sums<D>(r, sp, gi, dec, false, gw, gp, unused);
            aw += (double)gw;
            ap += (double)gp;
        }
    }
    if (sp.s + tid < sp.a) {
        const Weights x = elem_weight<D>(r, sp.s + tid, dec);
        aw += (double)x.w;
        ap += (double)x.p;
    }
    if (sp.z + tid < sp.e) {
        const Weights x = elem_weight<D>(r, sp.z + tid, dec);
        aw += (double)x.w;
        ap += (double)x.p;
    }
    aw = wave_sum(aw);
    ap = wave_sum(ap);
    if ((tid & (kWave - 1)) == 0) {
        sh.wd[tid / kWave][0] = aw;
        sh.pd[tid / kWave] = ap;
    }
    __syncthreads();
    if (tid == 0) {
        double w = 0.0, pp = 0.0;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
            w += sh.wd[i][0];
            pp += sh.pd[i];
        }
        double *m = reinterpret_cast<double *>(p.masses + b * (int64_t)p.nc + c);
        publish_double(m, w);
        publish_double(m + 1, pp);
    }
    __syncthreads();
}

// Inclusive prefix sum over the block (fixed order).
__device__ inline double block_inclusive_scan(double v, Shared &sh)
{
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const double o = __shfl_up(v, off, kWave);
        if (lane >= off)
            v += o;
    }
    if (lane == kWave - 1)
        sh.pd[wave] = v;
    __syncthreads();
    double before = 0.0;
    for (int w = 0; w < wave; ++w)
        before += sh.pd[w];
    __syncthreads();
    return before + v;
}

// ===========================================================================
// Inverse-CDF locate of one sequence's correction / bonus token.
// ===========================================================================
template <class D>
__device__ __forceinline__ void locate(const Params &p, int64_t b, const Decision &dec, Shared &sh)
{
    constexpr int64_t CH = chunk_elems<D>();
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int nc = p.nc;
    const double2 *mb = p.masses + b * (int64_t)nc;
    const DrawRows<D> r = draw_rows<D>(p, b, dec);
    int kind = dec.kind;

    // The published chunk sums (device-scope loads, all in flight at once)
    // go to LDS; thread 0 picks the chunk; the block shares its choice.
    const double *mw = reinterpret_cast<const double *>(mb);  // (w, p) pairs
    const bool staged = nc <= kMaxLdsChunks / 2;
    if (staged) {
        for (int q = tid; q < 2 * nc; q += kThreads)
            sh.cm[q] = fetch_double(mw + q);
        __syncthreads();
    }
    if (tid == 0) {
        auto mass = [&](int q) { return staged ? sh.cm[q] : fetch_double(mw + q); };
        double Sw = 0.0, Sp = 0.0;
        for (int c = 0; c < nc; ++c) {
            Sw += mass(2 * c);
            Sp += mass(2 * c + 1);
        }
        bool up = !r.resid;
        int kd = dec.kind;
        if (r.resid && !(Sw > 0.0)) {  // residual mass rounded away: draw from p
            up = true;
            kd = SPEC_DRAW_RESIDUAL_AS_P;
        }
        const double S_ = up ? Sp : Sw;
        const double t_ = (double)dec.v * S_;
        const int sel = up ? 1 : 0;
        double cm = 0.0;
        int c_star = -1;
        for (int c = 0; c < nc; ++c) {  // first chunk whose cumulative weight exceeds t
            const double m = mass(2 * c + sel);
            if (cm + m > t_) {
                c_star = c;
                break;
            }
            cm += m;
        }
        const bool fb = c_star < 0;
        if (fb) {  // rounding left no crossing: last chunk with weight
            for (int c = nc - 1; c >= 0; --c)
                if (mass(2 * c + sel) > 0.0) {
                    c_star = c;
                    break;
                }
            if (c_star < 0)
                c_star = nc - 1;
        }
        sh.pd[0] = S_;
        sh.pd[1] = t_;
        sh.pd[2] = cm;
        sh.i0 = c_star;
        sh.i1 = (up ? 1 : 0) | (fb ? 2 : 0);
        sh.flag = kd;
    }
    __syncthreads();
    const double S = sh.pd[0], t = sh.pd[1], cum = sh.pd[2];
    const int cs = sh.i0;
    const bool use_p = (sh.i1 & 1) != 0, fallback = (sh.i1 & 2) != 0;
    kind = sh.flag;
    __syncthreads();

    const int64_t s = (int64_t)cs * CH, e = min64((int64_t)p.V, s + CH);
    const Span sp = make_span2<D>(r.t, r.d, s, e);

    // Element order inside the chunk: head [s, a), groups gi = 0..ngroups-1
    // (tile u = gi / 256 holds lane tid at gi = u * 256 + tid), tail [z, e).
    // Segment totals go to LDS: sh.wd[wave][u] for the tiles, sh.ht for
    // head (0) and tail (1).
    int last = -1;
    if (sp.vec) {
        // all of the chunk's 16-byte loads in flight at once
        const u32x4 *vt = reinterpret_cast<const u32x4 *>(r.t + sp.a);
        const u32x4 *vd = reinterpret_cast<const u32x4 *>(r.d + sp.a);
        u32x4 lt[kTiles], ld[kTiles];
#pragma unroll
        for (int u = 0; u < kTiles; ++u) {
            const int64_t gi = (int64_t)u * kThreads + tid;
            const bool in = gi < sp.ngroups;
            lt[u] = in ? vt[gi] : u32x4{0u, 0u, 0u, 0u};
            ld[u] = in && r.resid ? vd[gi] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kTiles; ++u) {
            const int64_t gi = (int64_t)u * kThreads + tid;
            float sel = 0.f;
            if (gi < sp.ngroups) {
                float ft[D::kVec], fd[D::kVec], w[D::kVec];
                D::unpack(lt[u], ft);
                D::unpack(ld[u], fd);
#pragma unroll
                for (int j = 0; j < D::kVec; ++j) {
                    const Weights x = draw_weights(ft[j], fd[j], dec, r.inv_zt, r.inv_zd,
                                                   r.resid);
                    w[j] = use_p ? x.p : x.w;
                    if (w[j] > 0.f)
                        last = (int)(sp.a + gi * D::kVec + j);
                }
                sel = pairwise(w);
            }
            const double v = wave_sum((double)sel);
            if (lane == 0)
                sh.wd[wave][u] = v;
        }
    } else {
#pragma unroll 1
        for (int u = 0; u < kTiles; ++u) {
            float gw = 0.f, gp = 0.f;
            const int64_t gi = (int64_t)u * kThreads + tid;
            if (gi < sp.ngroups)
                group_weight_sums<D>(r, sp, gi, dec, use_p, gw, gp, last);
            const double v = wave_sum((double)(use_p ? gp : gw));
            if (lane == 0)
                sh.wd[wave][u] = v;
        }
    }
    double hv = 0.0, tv = 0.0;
    if (sp.s + tid < sp.a) {
        const Weights x = elem_weight<D>(r, sp.s + tid, dec);
        hv = (double)(use_p ? x.p : x.w);
        if (hv > 0.0)
            last = max(last, (int)(sp.s + tid));
    }
    if (sp.z + tid < sp.e) {
        const Weights x = elem_weight<D>(r, sp.z + tid, dec);
        tv = (double)(use_p ? x.p : x.w);
        if (tv > 0.0)
            last = max(last, (int)(sp.z + tid));
    }
    hv = wave_sum(hv);
    tv = wave_sum(tv);
    if (lane == 0) {
        sh.ht[0][wave] = hv;
        sh.ht[1][wave] = tv;
    }
    if (tid == 0) {
        sh.tok = -1;
        sh.i1 = -1;
        sh.i0 = kThreads;
    }
    __syncthreads();

    // Which segment holds the crossing (same arithmetic on every thread):
    // 0 = head, 1..kTiles = tiles, kTiles + 1 = tail.
    int seg = -1;
    double base = cum;
    if (!fallback) {
#pragma unroll 1
        for (int u = 0; u < kTiles + 2; ++u) {
            double tot = 0.0;
            for (int w = 0; w < kWaves; ++w)
                tot += u == 0 ? sh.ht[0][w] : (u == kTiles + 1 ? sh.ht[1][w] : sh.wd[w][u - 1]);
            if (base + tot > t) {
                seg = u;
                break;
            }
            base += tot;
        }
    }
    if (seg == 0 || seg == kTiles + 1) {
        // head or tail: fewer than kVec elements, thread 0 walks them in order
        if (tid == 0) {
            const int64_t x0 = seg == 0 ? sp.s : sp.z, x1 = seg == 0 ? sp.a : sp.e;
            double run = base;
            for (int64_t x = x0; x < x1; ++x) {
                const Weights wx = elem_weight<D>(r, x, dec);
                run += (double)(use_p ? wx.p : wx.w);
                if (run > t) {
                    sh.tok = (int)x;
                    break;
                }
            }
        }
    } else if (seg > 0) {
        const int64_t gi = (int64_t)(seg - 1) * kThreads + tid;
        float gw = 0.f, gp = 0.f;
        int unused = -1;
        if (gi < sp.ngroups)
            group_weight_sums<D>(r, sp, gi, dec, use_p, gw, gp, unused);
        const double mine = (double)(use_p ? gp : gw);
        const double incl = block_inclusive_scan(mine, sh);
        if (base + incl > t)
            atomicMin(&sh.i0, tid);
        __syncthreads();
        if (tid == sh.i0 && gi < sp.ngroups) {
            float ft[D::kVec], fd[D::kVec];
            load_group<D>(r.t, sp, gi, ft);
            if (r.resid)
                load_group<D>(r.d, sp, gi, fd);
            // Walk the group in id order. The group's total came from the
            // pairwise sum; if rounding leaves the walk short of t, the
            // crossing is still inside this group: take its last token
            // with weight.
            double run = base + (incl - mine);
            int found = -1, lastpos = -1;
            for (int j = 0; j < D::kVec; ++j) {
                const Weights x = draw_weights(ft[j], r.resid ? fd[j] : 0.f, dec, r.inv_zt,
                                               r.inv_zd, r.resid);
                const float wj = use_p ? x.p : x.w;
                run += (double)wj;
                if (wj > 0.f)
                    lastpos = (int)(sp.a + gi * D::kVec + j);
                if (found < 0 && run > t)
                    found = (int)(sp.a + gi * D::kVec + j);
            }
            sh.tok = found >= 0 ? found : lastpos;
        }
    }
    // Rounding fallback: the last token with weight in the chunk.
    if (last >= 0)
        atomicMax(&sh.i1, last);
    __syncthreads();
    if (tid == 0) {
        const int chosen = sh.tok >= 0 ? sh.tok : (sh.i1 >= 0 ? sh.i1 : (int)s);
        p.out_tokens[b * (p.k + 1) + dec.row] = chosen;
        if (p.aux.resid_mass) p.aux.resid_mass[b] = (float)S;
        if (p.aux.draw_kind) p.aux.draw_kind[b] = kind;
    }
    __syncthreads();
}

// ===========================================================================
// Sum draw-weight chunk c of sequence h if its decision is published and
// the chunk is not summed yet, then mark it summed. Each chunk has exactly
// one designated workgroup in k_verify and one in k_finish_sums, which runs
// after k_verify, so a chunk is never summed twice and nothing needs a
// claim or a completion count: the launch boundary orders the marks.
// ===========================================================================
template <class D>
__device__ __forceinline__ void sum_chunk(const Params &p, int64_t h, int c, Shared &sh)
{
    const int tid = threadIdx.x;
    int32_t *mark = p.chunk_claim + h * (int64_t)p.nc + c;
    if (tid == 0) {
        // The decision is read only after the flag says it is published
        // (two device-scope loads from one thread are not ordered).
        const int f = flag_load(&p.state[h].flag);
        const int m = flag_load(mark);
        sh.i0 = f == kDraw && m == 0;
        if (sh.i0)
            sh.dec = fetch_decision(p.decisions + h);
    }
    __syncthreads();
    if (!sh.i0)
        return;
    const Decision dec = sh.dec;
    chunk_weight_sums<D>(p, h, c, dec, sh);
    if (tid == 0)
        flag_store(mark, 1);
    __syncthreads();
}

// Take the decision of sequence h if it is ready. Each sequence has one
// designated decider in k_verify and one in k_finish_decide, which runs
// after it, so no claim is needed.
template <class D>
__device__ __forceinline__ void try_decide(const Params &p, int64_t h, Shared &sh)
{
    const int tid = threadIdx.x;
    if (tid == 0)
        sh.i1 = flag_load(&p.state[h].flag) == kReady;
    __syncthreads();
    if (!sh.i1)
        return;
    decide<D>(p, h, sh);
    __syncthreads();
    if (tid == 0) {
        const bool draw = sh.dec.kind == SPEC_DRAW_RESIDUAL || sh.dec.kind == SPEC_DRAW_BONUS;
        drain_stores();  // decision published before the flag
        flag_store(&p.state[h].flag, draw ? kDraw : kDone);
    }
    __syncthreads();
}

// Error outputs of a sequence whose length or temperature is invalid (it
// has no row items, so no decider).
template <class D>
__device__ __forceinline__ void invalid_sequence(const Params &p, int64_t b, int L, float tau)
{
    const int lane = threadIdx.x;
    const int k = p.k;
    if (lane <= k)
        p.out_tokens[b * (k + 1) + lane] = -1;
    if (p.aux.p_g && lane < k) p.aux.p_g[b * k + lane] = NAN;
    if (p.aux.q_g && lane < k) p.aux.q_g[b * k + lane] = NAN;
    if (p.aux.argmax && lane <= k) p.aux.argmax[b * (k + 1) + lane] = -1;
    if (lane == 0) {
        flag_store(&p.state[b].flag, kDone);
        p.num_accepted[b] = 0;
        if (p.aux.seq_status)
            p.aux.seq_status[b] = !valid_len(L, k) ? SPEC_SEQ_BAD_LEN : SPEC_SEQ_BAD_TEMP;
        if (p.aux.draw_row) p.aux.draw_row[b] = -1;
        if (p.aux.draw_kind) p.aux.draw_kind[b] = SPEC_DRAW_NONE;
        if (p.aux.resid_mass) p.aux.resid_mass[b] = NAN;
    }
}

// ===========================================================================
// The step.
// ===========================================================================
__global__ __launch_bounds__(kThreads) void k_reset(SeqState *state, int32_t *chunk_claim,
                                                    int32_t B, int32_t nc)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < B)
        state[i] = SeqState{0, kPending, 0, 0};
    if (i < (int64_t)B * nc)
        chunk_claim[i] = 0;
}

template <class D>
__global__ __launch_bounds__(kThreads) void k_verify(Params p)
{
    using E = typename D::Elem;
    constexpr int64_t CH = chunk_elems<D>();
    __shared__ Shared sh;
    const int tid = threadIdx.x;
    const int64_t item = blockIdx.x;
    const int k = p.k, nc = p.nc, rows = 2 * k + 1;

    const int c = (int)(item % nc);
    const int64_t rs = item / nc;
    const int slot = (int)(rs % rows);
    const int64_t b = rs / rows;
    const int L = p.draft_len ? p.draft_len[b] : k;
    const float tau = p.temperature[b];
    if (!valid_len(L, k) || !valid_temp(tau)) {
        if (slot == 0 && c == 0)
            invalid_sequence<D>(p, b, L, tau);
        return;
    }
    const bool greedy = tau == 0.f;
    const bool is_target = slot <= k;
    const int i = is_target ? slot : slot - (k + 1);
    if (is_target ? i > L : (greedy || i >= L))
        return;  // row not needed by this sequence: never read

    const E *row = is_target ? static_cast<const E *>(p.target) + (b * (k + 1) + i) * (int64_t)p.V
                             : static_cast<const E *>(p.draft) + (b * k + i) * (int64_t)p.V;
    const int64_t s = (int64_t)c * CH;
    const float2 part = chunk_stats<D>(row, s, min64((int64_t)p.V, s + CH), greedy,
                                       greedy ? 0.f : temp_scale(tau), sh);
    if (tid == 0) {
        publish_pair(p.partials + item, __float_as_uint(part.x), __float_as_uint(part.y));
        drain_stores();  // partial published before the count
        const int items = nc * ((L + 1) + (greedy ? 0 : L));
        if (counter_add(&p.state[b].rows_done, 1) == items - 1)
            flag_store(&p.state[b].flag, kReady);
    }
    // The items of target row 0 (always read) take, by a fixed rule, the
    // decision of sequence b - kLagDecide and one draw-weight chunk of
    // sequence b - kLagSum, whose rows are still in the last-level cache.
    // The assignment is static: who finishes first or last decides nothing,
    // so an XCD that lags is never handed extra work (workgroup i runs on
    // XCD i % 8, and chunk c of a row is workgroup ... * nc + c).
    if (slot == 0) {
        const int64_t h1 = b - kLagDecide, h2 = b - kLagSum;
        if (h1 >= 0 && c == (int)(h1 % nc)) {
            __syncthreads();
            try_decide<D>(p, h1, sh);
        }
        if (h2 >= 0) {
            __syncthreads();
            sum_chunk<D>(p, h2, (int)((c + nc - h2 % nc) % nc), sh);
        }
    }
}

// Work left when k_verify ends (in practice the last kLagSum sequences), in
// three launches ordered by the stream, so nothing ever waits: decisions,
// then chunk sums, then every locate.
template <class D>
__global__ __launch_bounds__(kThreads) void k_finish_decide(Params p)
{
    __shared__ Shared sh;
    try_decide<D>(p, blockIdx.x, sh);
}

template <class D>
__global__ __launch_bounds__(kThreads) void k_finish_sums(Params p)
{
    __shared__ Shared sh;
    sum_chunk<D>(p, blockIdx.x / p.nc, (int)(blockIdx.x % p.nc), sh);
}

template <class D>
__global__ __launch_bounds__(kThreads) void k_finish_locate(Params p)
{
    __shared__ Shared sh;
    const int64_t b = blockIdx.x;
    if (threadIdx.x == 0) {
        sh.flag = flag_load(&p.state[b].flag);
        if (sh.flag == kDraw)
            sh.dec = fetch_decision(p.decisions + b);
    }
    __syncthreads();
    if (sh.flag == kDraw) {
        const Decision dec = sh.dec;
        locate<D>(p, b, dec, sh);
    }
}

// ===========================================================================
// Host side.
// ===========================================================================
struct Layout {
    int nc;
    size_t partials, decisions, masses, state, claims, total;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool layout_for(int32_t B, int32_t k, int32_t V, int32_t dtype, Layout *lay)
{
    if (B < 0 || k < 0 || k > SPEC_MAX_K || V < 1 || (dtype != SPEC_F32 && dtype != SPEC_BF16))
        return false;
    const int64_t ch = kChunkBytes / (dtype == SPEC_F32 ? 4 : 2);
    lay->nc = (int)((V + ch - 1) / ch);
    const size_t nb = (size_t)B;
    lay->partials = 0;
    lay->decisions = align_up(nb * (size_t)(2 * k + 1) * (size_t)lay->nc * sizeof(float2), 256);
    lay->masses = lay->decisions + align_up(nb * sizeof(Decision), 256);
    lay->state = lay->masses + align_up(nb * (size_t)lay->nc * sizeof(double2), 256);
    lay->claims = lay->state + align_up(nb * sizeof(SeqState), 256);
    lay->total = lay->claims + align_up(nb * (size_t)lay->nc * sizeof(int32_t), 256);
    if (lay->total == 0)
        lay->total = 256;
    return true;
}

template <class D>
int launch_all(const Params &base, const spec_verify_aux_t *aux, const Layout &lay, char *ws,
               hipStream_t stream)
{
    using E = typename D::Elem;
    const int B = base.B, k = base.k, nc = lay.nc;
    const int rows = 2 * k + 1;
    const int64_t per_seq_items = (int64_t)rows * nc;
    // Keep every grid well inside the 32-bit global thread-id range.
    const int64_t max_items = (int64_t)1 << 22;
    const int64_t slice = std::max<int64_t>(1, max_items / per_seq_items);
    hipEvent_t ev_begin = aux ? static_cast<hipEvent_t>(aux->event_begin) : nullptr;
    hipEvent_t ev_end = aux ? static_cast<hipEvent_t>(aux->event_end) : nullptr;

    for (int64_t b0 = 0; b0 < B; b0 += slice) {
        const int64_t nb = std::min<int64_t>((int64_t)B - b0, slice);
        Params p = base;
        p.B = (int32_t)nb;
        p.nc = nc;
        p.target = static_cast<const E *>(base.target) + b0 * (k + 1) * (int64_t)base.V;
        p.draft = base.draft ? static_cast<const E *>(base.draft) + b0 * k * (int64_t)base.V
                             : nullptr;
        p.draft_tokens = base.draft_tokens ? base.draft_tokens + b0 * k : nullptr;
        p.draft_len = base.draft_len ? base.draft_len + b0 : nullptr;
        p.temperature = base.temperature + b0;
        p.seq_base = base.seq_base + (uint32_t)b0;
        p.partials = reinterpret_cast<float2 *>(ws + lay.partials) + b0 * per_seq_items;
        p.decisions = reinterpret_cast<Decision *>(ws + lay.decisions) + b0;
        p.masses = reinterpret_cast<double2 *>(ws + lay.masses) + b0 * nc;
        p.state = reinterpret_cast<SeqState *>(ws + lay.state) + b0;
        p.chunk_claim = reinterpret_cast<int32_t *>(ws + lay.claims) + b0 * nc;
        p.out_tokens = base.out_tokens + b0 * (k + 1);
        p.num_accepted = base.num_accepted + b0;
        AuxDev &a = p.aux;
        if (a.p_g) a.p_g += b0 * k;
        if (a.q_g) a.q_g += b0 * k;
        if (a.resid_mass) a.resid_mass += b0;
        if (a.argmax) a.argmax += b0 * (k + 1);
        if (a.seq_status) a.seq_status += b0;
        if (a.draw_row) a.draw_row += b0;
        if (a.draw_kind) a.draw_kind += b0;
        p.n_row_items = nb * per_seq_items;

        hipLaunchKernelGGL(k_reset, dim3((unsigned)((nb * nc + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, stream, p.state, p.chunk_claim, (int32_t)nb, nc);
        if (ev_begin && b0 == 0 && hipEventRecord(ev_begin, stream) != hipSuccess)
            return SPEC_ELAUNCH;
        hipLaunchKernelGGL(k_verify<D>, dim3((unsigned)p.n_row_items), dim3(kThreads), 0, stream,
                           p);
        hipLaunchKernelGGL(k_finish_decide<D>, dim3((unsigned)nb), dim3(kThreads), 0, stream, p);
        hipLaunchKernelGGL(k_finish_sums<D>, dim3((unsigned)(nb * nc)), dim3(kThreads), 0, stream,
                           p);
        hipLaunchKernelGGL(k_finish_locate<D>, dim3((unsigned)nb), dim3(kThreads), 0, stream, p);
        if (ev_end && b0 + nb >= B && hipEventRecord(ev_end, stream) != hipSuccess)
            return SPEC_ELAUNCH;
        if (hipGetLastError() != hipSuccess)
            return SPEC_ELAUNCH;
    }
    return SPEC_OK;
}

bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

}  // namespace

extern "C" size_t spec_verify_workspace_size(int32_t B, int32_t k, int32_t V, int32_t dtype)
{
    Layout lay;
    return layout_for(B, k, V, dtype, &lay) ? lay.total : 0;
}

extern "C" int spec_verify(const void *target_logits, const void *draft_logits, int32_t dtype,
                           const int32_t *draft_tokens, const int32_t *draft_len,
                           const float *temperature, int32_t B, int32_t k, int32_t V,
                           uint64_t seed, uint32_t seq_base, int32_t *out_tokens,
                           int32_t *num_accepted, const spec_verify_aux_t *aux, void *workspace,
                           size_t workspace_bytes, void *stream)
{
    Layout lay;
    if (!layout_for(B, k, V, dtype, &lay))
        return SPEC_EINVAL;
    if (B == 0)
        return SPEC_OK;
    const size_t esz = dtype == SPEC_F32 ? 4 : 2;
    if (!target_logits || !temperature || !out_tokens || !num_accepted)
        return SPEC_EINVAL;
    if (k > 0 && (!draft_logits || !draft_tokens))
        return SPEC_EINVAL;
    if (!aligned(target_logits, esz) || (draft_logits && !aligned(draft_logits, esz)) ||
        !aligned(temperature, 4) || !aligned(out_tokens, 4) || !aligned(num_accepted, 4) ||
        (draft_tokens && !aligned(draft_tokens, 4)) || (draft_len && !aligned(draft_len, 4)))
        return SPEC_EINVAL;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < lay.total)
        return SPEC_EWORKSPACE;

    Params p{};
    p.target = target_logits;
    p.draft = k > 0 ? draft_logits : nullptr;
    p.draft_tokens = k > 0 ? draft_tokens : nullptr;
    p.draft_len = draft_len;
    p.temperature = temperature;
    p.k = k;
    p.V = V;
    p.B = B;
    p.key0 = (uint32_t)seed;
    p.key1 = (uint32_t)(seed >> 32);
    p.seq_base = seq_base;
    p.out_tokens = out_tokens;
    p.num_accepted = num_accepted;
    if (aux) {
        p.aux.p_g = aux->p_g;
        p.aux.q_g = aux->q_g;
        p.aux.resid_mass = aux->resid_mass;
        p.aux.argmax = aux->argmax;
        p.aux.seq_status = aux->seq_status;
        p.aux.draw_row = aux->draw_row;
        p.aux.draw_kind = aux->draw_kind;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    if (dtype == SPEC_F32)
        return launch_all<F32>(p, aux, lay, ws, st);
    return launch_all<BF16>(p, aux, lay, ws, st);
}

extern "C" const char *spec_verify_strerror(int status)
{
    switch (status) {
    case SPEC_OK: return "success";
    case SPEC_EINVAL: return "invalid argument (null pointer, size, dtype or alignment)";
    case SPEC_EWORKSPACE: return "workspace null, misaligned or smaller than spec_verify_workspace_size()";
    case SPEC_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

extern "C" int spec_verify_version(void) { return kDeviceVersion; }
