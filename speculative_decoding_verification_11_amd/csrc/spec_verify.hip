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
// Four launches, all stream-ordered, no host synchronisation:
//
//   K1 k_rowstats       one workgroup per 32 KiB chunk of every logit row the
//                       step needs. Streams the chunk once with 16-byte loads
//                       and writes an 8-byte partial: (max logit, sum of
//                       2^((x - max) * log2(e)/tau)) for sampling rows, or
//                       (max logit, lowest index of it) for greedy rows.
//                       This kernel carries ~all of the HBM traffic.
//   K2 k_decide         one wave per sequence. Folds the chunk partials in
//                       chunk order into per-row (max, normaliser), gathers
//                       p_i(g_i), q_i(g_i) from single logits, draws Philox,
//                       runs the left-to-right test and writes the accepted
//                       prefix plus a decision record (row, kind, uniform).
//   K3 k_residual_mass  one workgroup per chunk of the decided row: chunk sums
//                       of the draw weights w(x) = max(0, p(x) - q(x)) (or p
//                       for a bonus), accumulated in fp64.
//   K4 k_locate         one workgroup per sequence: finds the chunk where the
//                       cumulative weight passes v * S, then the token inside
//                       it with a block prefix scan; writes the last token.
//
// Nothing here is a dense contraction, so there is no MFMA: every kernel is
// bound by HBM bandwidth (K1) or latency (K2-K4).

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
constexpr int kChunkBytes = 32768;  // one K1 work item
constexpr int kUnroll = 8;          // 16-byte loads in flight per thread
constexpr int kDeviceVersion = 100;  // 0.1.0

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

__host__ __device__ inline int num_chunks(int64_t V, int64_t chunk)
{
    return (int)((V + chunk - 1) / chunk);
}

// Element range [s, e) of a row split into a scalar head [s, a), 16-byte
// aligned vectors [a, z) and a scalar tail [z, e).
template <class D>
struct Span {
    int64_t s, a, z, e, nvec;
};

template <class D>
__device__ inline Span<D> make_span(const typename D::Elem *row, int64_t s, int64_t e)
{
    using E = typename D::Elem;
    const uintptr_t addr = (uintptr_t)(row + s);
    const int64_t head = (int64_t)(((16u - (addr & 15u)) & 15u) / sizeof(E));
    Span<D> sp;
    sp.s = s;
    sp.e = e;
    sp.a = min64(e, s + head);
    sp.nvec = (e - sp.a) / D::kVec;
    sp.z = sp.a + sp.nvec * D::kVec;
    return sp;
}

// ---------------------------------------------------------------------------
// Online softmax statistics (Milakov & Gimelshein, "Online normalizer
// calculation for softmax", 2018): running max m of the raw logits and
// z = sum 2^((x - m) * scale), scale = log2(e) / tau. Merging two states
// rescales the smaller-max sum.
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

// Greedy: (max value, lowest index holding it).
struct ArgMax {
    float v;
    int32_t i;
};

__device__ inline ArgMax argmax_merge(ArgMax a, ArgMax b)
{
    return (b.v > a.v || (b.v == a.v && b.i < a.i)) ? b : a;
}

// ---------------------------------------------------------------------------
// Wave and block reductions (fixed order, so results do not depend on timing).
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

// Decision record written by K2 for K3/K4.
struct __align__(16) Decision {
    int32_t row;   // row of the final draw
    int32_t kind;  // SPEC_DRAW_*
    float v;       // draw uniform
    float scale;   // log2(e) / tau
    float mt, zt;  // target row: max logit, normaliser
    float md, zd;  // draft row (residual draws only)
};

struct AuxDev {
    float *p_g, *q_g, *resid_mass;
    int32_t *argmax, *seq_status, *draw_row, *draw_kind;
};

// ===========================================================================
// K1: per-chunk row statistics.
// ===========================================================================
template <class D>
__global__ __launch_bounds__(kThreads) void k_rowstats(
    const typename D::Elem *__restrict__ target, const typename D::Elem *__restrict__ draft,
    const int32_t *__restrict__ draft_len, const float *__restrict__ temperature, int32_t k,
    int32_t V, int32_t nc, float2 *__restrict__ partials)
{
    using E = typename D::Elem;
    constexpr int64_t CH = chunk_elems<D>();
    constexpr int NX = kUnroll * D::kVec;
    const int rows = 2 * k + 1;
    const int64_t item = blockIdx.x;
    const int c = (int)(item % nc);
    const int64_t rs = item / nc;
    const int slot = (int)(rs % rows);
    const int64_t b = rs / rows;

    const int L = draft_len ? draft_len[b] : k;
    const float tau = temperature[b];
    if (!valid_len(L, k) || !valid_temp(tau))
        return;
    const bool greedy = tau == 0.f;
    const bool is_target = slot <= k;
    const int i = is_target ? slot : slot - (k + 1);
    if (is_target ? i > L : (greedy || i >= L))
        return;  // row not needed by this sequence: never read

    const E *row = is_target ? target + (b * (k + 1) + i) * (int64_t)V
                             : draft + (b * k + i) * (int64_t)V;
    const Span<D> sp = make_span<D>(row, (int64_t)c * CH, min64((int64_t)V, (int64_t)(c + 1) * CH));
    const u32x4 *vrow = reinterpret_cast<const u32x4 *>(row + sp.a);
    const int tid = threadIdx.x;
    const u32x4 pad = {D::kNegInfWord, D::kNegInfWord, D::kNegInfWord, D::kNegInfWord};

    __shared__ float sh_a[kWaves];
    __shared__ float sh_b[kWaves];

    if (!greedy) {
        const float scale = temp_scale(tau);
        Soft st{-INFINITY, 0.f};
        for (int64_t base = 0; base < sp.nvec; base += (int64_t)kThreads * kUnroll) {
            u32x4 r[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t vi = base + u * kThreads + tid;
                r[u] = vi < sp.nvec ? vrow[vi] : pad;
            }
            float x[NX];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                float f[D::kVec];
                D::unpack(r[u], f);
#pragma unroll
                for (int j = 0; j < D::kVec; ++j)
                    x[u * D::kVec + j] = f[j];
            }
            soft_update(st, x, scale);
        }
        // scalar head and tail (misaligned rows, or V not a multiple of the vector)
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
            sh_a[tid / kWave] = st.m;
            sh_b[tid / kWave] = st.z;
        }
        __syncthreads();
        if (tid == 0) {
            Soft acc{sh_a[0], sh_b[0]};
#pragma unroll
            for (int w = 1; w < kWaves; ++w)
                acc = soft_merge(acc, Soft{sh_a[w], sh_b[w]}, scale);
            partials[item] = make_float2(acc.m, acc.z);
        }
    } else {
        ArgMax am{-INFINITY, INT32_MAX};
        // head first, then vectors, then tail: each thread sees ascending ids
        if (sp.s + tid < sp.a) {
            const float x = D::at(row, sp.s + tid);
            if (x > am.v) am = ArgMax{x, (int32_t)(sp.s + tid)};
        }
        for (int64_t base = 0; base < sp.nvec; base += (int64_t)kThreads * kUnroll) {
            u32x4 r[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t vi = base + u * kThreads + tid;
                r[u] = vi < sp.nvec ? vrow[vi] : pad;
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
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
            sh_a[tid / kWave] = am.v;
            sh_b[tid / kWave] = __int_as_float(am.i);
        }
        __syncthreads();
        if (tid == 0) {
            ArgMax acc{sh_a[0], __float_as_int(sh_b[0])};
#pragma unroll
            for (int w = 1; w < kWaves; ++w)
                acc = argmax_merge(acc, ArgMax{sh_a[w], __float_as_int(sh_b[w])});
            partials[item] = make_float2(acc.v, __int_as_float(acc.i));
        }
    }
}

// ===========================================================================
// K2: fold partials, gather p(g), q(g), draw, scan. One wave per sequence.
// ===========================================================================
template <class D>
__global__ __launch_bounds__(kWave) void k_decide(
    const typename D::Elem *__restrict__ target, const typename D::Elem *__restrict__ draft,
    const int32_t *__restrict__ draft_tokens, const int32_t *__restrict__ draft_len,
    const float *__restrict__ temperature, int32_t k, int32_t V, int32_t nc, uint32_t key0,
    uint32_t key1, uint32_t seq_base, const float2 *__restrict__ partials,
    Decision *__restrict__ decisions, int32_t *__restrict__ out_tokens,
    int32_t *__restrict__ num_accepted, AuxDev aux)
{
    const int64_t b = blockIdx.x;
    const int lane = threadIdx.x;
    const int rows = 2 * k + 1;
    const int L = draft_len ? draft_len[b] : k;
    const float tau = temperature[b];
    int32_t *out = out_tokens + b * (k + 1);

    int status = SPEC_SEQ_OK;
    int g = -1;
    if (!valid_len(L, k)) {
        status = SPEC_SEQ_BAD_LEN;
    } else if (!valid_temp(tau)) {
        status = SPEC_SEQ_BAD_TEMP;
    } else {
        g = lane < L ? draft_tokens[b * k + lane] : -1;
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
            const float2 *pp = partials + (b * rows + lane) * (int64_t)nc;
            ArgMax acc{-INFINITY, INT32_MAX};
            for (int c = 0; c < nc; ++c) {
                const float2 t = pp[c];
                acc = argmax_merge(acc, ArgMax{t.x, __float_as_int(t.y)});
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
            num_accepted[b] = j;
    } else if (status == SPEC_SEQ_OK) {
        const float scale = temp_scale(tau);
        Soft ts{-INFINITY, 0.f}, ds{-INFINITY, 0.f};
        if (lane <= L) {
            const float2 *pp = partials + (b * rows + lane) * (int64_t)nc;
            for (int c = 0; c < nc; ++c) {
                const float2 t = pp[c];
                ts = soft_merge(ts, Soft{t.x, t.y}, scale);
            }
        }
        if (lane < L) {
            const float2 *pp = partials + (b * rows + k + 1 + lane) * (int64_t)nc;
            for (int c = 0; c < nc; ++c) {
                const float2 t = pp[c];
                ds = soft_merge(ds, Soft{t.x, t.y}, scale);
            }
            const float xt = D::at(target + (b * (k + 1) + lane) * (int64_t)V, g);
            const float xd = D::at(draft + (b * k + lane) * (int64_t)V, g);
            pg = exp2_fast((xt - ts.m) * scale) / ts.z;
            qg = exp2_fast((xd - ds.m) * scale) / ds.z;
        }
        const uint4 w = philox4x32_10(make_uint4((uint32_t)lane, seq_base + (uint32_t)b, 0u, 0u),
                                      key0, key1);
        const float u = uniform24(w.x), v = uniform24(w.y);
        const bool qzero = lane < L && !(qg > 0.f);
        const bool reject = lane < L && !qzero && !(u < fminf(1.f, pg / qg));
        const uint64_t stop = __ballot(qzero || reject);
        const int j = stop ? __ffsll((unsigned long long)stop) - 1 : L;
        if (__shfl((int)qzero, j, kWave)) {
            status = SPEC_SEQ_QZERO;
        } else {
            if (lane <= k)
                out[lane] = lane < j ? g : -1;  // position j is written by K4
            dec.row = j;
            dec.kind = j < L ? SPEC_DRAW_RESIDUAL : SPEC_DRAW_BONUS;
            dec.v = __shfl(v, j, kWave);
            dec.scale = scale;
            dec.mt = __shfl(ts.m, j, kWave);
            dec.zt = __shfl(ts.z, j, kWave);
            dec.md = __shfl(ds.m, j, kWave);
            dec.zd = __shfl(ds.z, j, kWave);
            if (lane == 0)
                num_accepted[b] = j;
        }
    }

    if (status != SPEC_SEQ_OK) {
        if (lane <= k)
            out[lane] = -1;
        if (lane == 0)
            num_accepted[b] = 0;
        dec.row = -1;
        dec.kind = SPEC_DRAW_NONE;
        pg = qg = NAN;
        amax = -1;
    }
    if (lane < k) {
        if (aux.p_g) aux.p_g[b * k + lane] = lane < L ? pg : NAN;
        if (aux.q_g) aux.q_g[b * k + lane] = lane < L ? qg : NAN;
    }
    if (aux.argmax && lane <= k)
        aux.argmax[b * (k + 1) + lane] = (lane <= L) ? amax : -1;
    if (lane == 0) {
        decisions[b] = dec;
        if (aux.seq_status) aux.seq_status[b] = status;
        if (aux.draw_row) aux.draw_row[b] = dec.row;
        if (aux.draw_kind) aux.draw_kind[b] = dec.kind;
        if (aux.resid_mass) aux.resid_mass[b] = NAN;  // K4 fills sampled rows
    }
}

// Draw weight of one token: w = max(0, p - q) for a residual (p alone for a
// bonus), and p itself (for the rounding fallback). Shared by K3 and K4 so
// both see bit-identical weights.
struct Weights {
    double w, p;
};

__device__ inline Weights draw_weights(float xt, float xd, const Decision &dec, float inv_zt,
                                       float inv_zd, bool resid)
{
    const float pt = exp2_fast((xt - dec.mt) * dec.scale) * inv_zt;
    if (!resid)
        return {(double)pt, (double)pt};
    const float pd = exp2_fast((xd - dec.md) * dec.scale) * inv_zd;
    const double d = (double)pt - (double)pd;
    return {d > 0.0 ? d : 0.0, (double)pt};
}

// ===========================================================================
// K3: chunk masses of the draw weights of each sequence's decided row.
// ===========================================================================
template <class D>
__global__ __launch_bounds__(kThreads) void k_residual_mass(
    const typename D::Elem *__restrict__ target, const typename D::Elem *__restrict__ draft,
    int32_t k, int32_t V, int32_t nc, const Decision *__restrict__ decisions,
    double2 *__restrict__ masses)
{
    using E = typename D::Elem;
    constexpr int64_t CH = chunk_elems<D>();
    const int64_t item = blockIdx.x;
    const int c = (int)(item % nc);
    const int64_t b = item / nc;
    const Decision dec = decisions[b];
    if (dec.kind != SPEC_DRAW_RESIDUAL && dec.kind != SPEC_DRAW_BONUS)
        return;
    const bool resid = dec.kind == SPEC_DRAW_RESIDUAL;
    const E *trow = target + (b * (k + 1) + dec.row) * (int64_t)V;
    const E *drow = resid ? draft + (b * k + dec.row) * (int64_t)V : trow;
    const float inv_zt = 1.f / dec.zt;
    const float inv_zd = resid ? 1.f / dec.zd : 0.f;
    const int64_t s = (int64_t)c * CH, e = min64((int64_t)V, s + CH);
    const int tid = threadIdx.x;

    double aw = 0.0, ap = 0.0;
    const Span<D> st = make_span<D>(trow, s, e);
    const Span<D> sd = make_span<D>(drow, s, e);
    if (st.a == sd.a) {
        const u32x4 *vt = reinterpret_cast<const u32x4 *>(trow + st.a);
        const u32x4 *vd = reinterpret_cast<const u32x4 *>(drow + st.a);
        for (int64_t vi = tid; vi < st.nvec; vi += kThreads) {
            float ft[D::kVec], fd[D::kVec];
            D::unpack(vt[vi], ft);
            if (resid)
                D::unpack(vd[vi], fd);
#pragma unroll
            for (int j = 0; j < D::kVec; ++j) {
                const Weights wt = draw_weights(ft[j], resid ? fd[j] : 0.f, dec, inv_zt, inv_zd,
                                                resid);
                aw += wt.w;
                ap += wt.p;
            }
        }
        for (int64_t x = st.s + tid; x < st.a; x += kThreads) {
            const Weights wt = draw_weights(D::at(trow, x), resid ? D::at(drow, x) : 0.f, dec,
                                            inv_zt, inv_zd, resid);
            aw += wt.w;
            ap += wt.p;
        }
        for (int64_t x = st.z + tid; x < st.e; x += kThreads) {
            const Weights wt = draw_weights(D::at(trow, x), resid ? D::at(drow, x) : 0.f, dec,
                                            inv_zt, inv_zd, resid);
            aw += wt.w;
            ap += wt.p;
        }
    } else {
        // target and draft rows disagree in 16-byte alignment: element loads
        for (int64_t x = s + tid; x < e; x += kThreads) {
            const Weights wt = draw_weights(D::at(trow, x), resid ? D::at(drow, x) : 0.f, dec,
                                            inv_zt, inv_zd, resid);
            aw += wt.w;
            ap += wt.p;
        }
    }
    __shared__ double sh_w[kWaves], sh_p[kWaves];
    aw = wave_sum(aw);
    ap = wave_sum(ap);
    if ((tid & (kWave - 1)) == 0) {
        sh_w[tid / kWave] = aw;
        sh_p[tid / kWave] = ap;
    }
    __syncthreads();
    if (tid == 0) {
        double w = 0.0, p = 0.0;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
            w += sh_w[i];
            p += sh_p[i];
        }
        masses[item] = make_double2(w, p);
    }
}

// Inclusive prefix sum over the block (fixed order).
__device__ inline double block_inclusive_scan(double v, double *sh_wave)
{
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const double o = __shfl_up(v, off, kWave);
        if (lane >= off)
            v += o;
    }
    if (lane == kWave - 1)
        sh_wave[wave] = v;
    __syncthreads();
    double before = 0.0;
    for (int w = 0; w < wave; ++w)
        before += sh_wave[w];
    return before + v;
}

// ===========================================================================
// K4: inverse-CDF locate of each sequence's correction / bonus token.
// ===========================================================================
template <class D>
__global__ __launch_bounds__(kThreads) void k_locate(
    const typename D::Elem *__restrict__ target, const typename D::Elem *__restrict__ draft,
    int32_t k, int32_t V, int32_t nc, const Decision *__restrict__ decisions,
    const double2 *__restrict__ masses, int32_t *__restrict__ out_tokens, AuxDev aux)
{
    using E = typename D::Elem;
    constexpr int64_t CH = chunk_elems<D>();
    const int64_t b = blockIdx.x;
    const int tid = threadIdx.x;
    const Decision dec = decisions[b];
    if (dec.kind != SPEC_DRAW_RESIDUAL && dec.kind != SPEC_DRAW_BONUS)
        return;
    bool resid = dec.kind == SPEC_DRAW_RESIDUAL;
    int kind = dec.kind;
    const double2 *mb = masses + b * (int64_t)nc;

    double Sw = 0.0, Sp = 0.0;
    for (int c = 0; c < nc; ++c) {
        const double2 m = mb[c];
        Sw += m.x;
        Sp += m.y;
    }
    bool use_p = !resid;
    if (resid && !(Sw > 0.0)) {  // residual mass rounded away: draw from p
        use_p = true;
        kind = SPEC_DRAW_RESIDUAL_AS_P;
    }
    const double S = use_p ? Sp : Sw;
    const double t = (double)dec.v * S;

    // chunk where the cumulative weight first exceeds t
    double cum = 0.0;
    int cs = -1;
    for (int c = 0; c < nc; ++c) {
        const double m = use_p ? mb[c].y : mb[c].x;
        if (cum + m > t) {
            cs = c;
            break;
        }
        cum += m;
    }
    bool fallback = false;
    if (cs < 0) {  // rounding left no crossing: last token with weight
        fallback = true;
        for (int c = nc - 1; c >= 0; --c)
            if ((use_p ? mb[c].y : mb[c].x) > 0.0) {
                cs = c;
                break;
            }
        if (cs < 0)
            cs = nc - 1;
    }

    const E *trow = target + (b * (k + 1) + dec.row) * (int64_t)V;
    const E *drow = resid ? draft + (b * k + dec.row) * (int64_t)V : trow;
    const float inv_zt = 1.f / dec.zt;
    const float inv_zd = resid ? 1.f / dec.zd : 0.f;
    const int64_t s = (int64_t)cs * CH, e = min64((int64_t)V, s + CH);
    const int64_t seg = (e - s + kThreads - 1) / kThreads;
    const int64_t x0 = min64(e, s + tid * seg), x1 = min64(e, x0 + seg);

    auto weight = [&](int64_t x) -> double {
        const Weights wt = draw_weights(D::at(trow, x), resid ? D::at(drow, x) : 0.f, dec, inv_zt,
                                        inv_zd, resid);
        return use_p ? wt.p : wt.w;
    };

    double mine = 0.0;
    int64_t last_pos = -1;
    for (int64_t x = x0; x < x1; ++x) {
        const double w = weight(x);
        mine += w;
        if (w > 0.0)
            last_pos = x;
    }
    __shared__ double sh_wave[kWaves];
    __shared__ int sh_first;
    __shared__ int sh_last;
    if (tid == 0) {
        sh_first = kThreads;
        sh_last = -1;
    }
    const double incl = block_inclusive_scan(mine, sh_wave);
    const double excl = incl - mine;
    __syncthreads();
    if (!fallback && cum + incl > t)
        atomicMin(&sh_first, tid);
    if (last_pos >= 0)
        atomicMax(&sh_last, (int)last_pos);
    __syncthreads();
    const int first = sh_first;
    int64_t tok = -1;
    if (first < kThreads) {
        if (tid == first) {
            double run = cum + excl;
            for (int64_t x = x0; x < x1; ++x) {
                const double w = weight(x);
                run += w;
                if (run > t) {
                    tok = x;
                    break;
                }
            }
            if (tok < 0)
                tok = last_pos >= 0 ? last_pos : (int64_t)sh_last;
        }
    } else if (tid == 0) {
        tok = sh_last >= 0 ? (int64_t)sh_last : s;
    }
    if (tok >= 0) {
        out_tokens[b * (k + 1) + dec.row] = (int32_t)tok;
        if (aux.resid_mass) aux.resid_mass[b] = (float)S;
        if (aux.draw_kind) aux.draw_kind[b] = kind;
    }
}

// ===========================================================================
// Host side.
// ===========================================================================
struct Layout {
    int nc;
    size_t partials, decisions, masses, total;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool layout_for(int32_t B, int32_t k, int32_t V, int32_t dtype, Layout *lay)
{
    if (B < 0 || k < 0 || k > SPEC_MAX_K || V < 1 || (dtype != SPEC_F32 && dtype != SPEC_BF16))
        return false;
    const int64_t ch = kChunkBytes / (dtype == SPEC_F32 ? 4 : 2);
    lay->nc = num_chunks(V, ch);
    const size_t nb = (size_t)B;
    const size_t part = nb * (size_t)(2 * k + 1) * (size_t)lay->nc * sizeof(float2);
    const size_t decs = nb * sizeof(Decision);
    const size_t mass = nb * (size_t)lay->nc * sizeof(double2);
    lay->partials = 0;
    lay->decisions = align_up(part, 256);
    lay->masses = lay->decisions + align_up(decs, 256);
    lay->total = lay->masses + align_up(mass, 256);
    if (lay->total == 0)
        lay->total = 256;
    return true;
}

template <class D>
int launch_all(const void *target_v, const void *draft_v, const int32_t *draft_tokens,
               const int32_t *draft_len, const float *temperature, int32_t B, int32_t k,
               int32_t V, uint64_t seed, uint32_t seq_base, int32_t *out_tokens,
               int32_t *num_accepted, const spec_verify_aux_t *aux, const Layout &lay,
               char *ws, hipStream_t stream)
{
    using E = typename D::Elem;
    const E *target = static_cast<const E *>(target_v);
    const E *draft = static_cast<const E *>(draft_v);
    const int rows = 2 * k + 1;
    const int nc = lay.nc;
    float2 *partials = reinterpret_cast<float2 *>(ws + lay.partials);
    Decision *decisions = reinterpret_cast<Decision *>(ws + lay.decisions);
    double2 *masses = reinterpret_cast<double2 *>(ws + lay.masses);
    const uint32_t key0 = (uint32_t)seed, key1 = (uint32_t)(seed >> 32);

    // Keep every grid well inside the 32-bit global thread-id range.
    const int64_t per_seq_items = (int64_t)rows * nc;
    const int64_t max_items = (int64_t)1 << 22;
    const int64_t slice = per_seq_items > max_items ? 1 : max_items / per_seq_items;

    AuxDev a{};
    if (aux) {
        a.p_g = aux->p_g;
        a.q_g = aux->q_g;
        a.resid_mass = aux->resid_mass;
        a.argmax = aux->argmax;
        a.seq_status = aux->seq_status;
        a.draw_row = aux->draw_row;
        a.draw_kind = aux->draw_kind;
    }
    hipEvent_t ev_begin = aux ? static_cast<hipEvent_t>(aux->event_begin) : nullptr;
    hipEvent_t ev_end = aux ? static_cast<hipEvent_t>(aux->event_end) : nullptr;

    for (int64_t b0 = 0; b0 < B; b0 += slice) {
        const int64_t nb = std::min<int64_t>((int64_t)B - b0, slice);
        const E *t0 = target + b0 * (k + 1) * (int64_t)V;
        const E *d0 = draft ? draft + b0 * k * (int64_t)V : nullptr;
        const int32_t *g0 = draft_tokens ? draft_tokens + b0 * k : nullptr;
        const int32_t *l0 = draft_len ? draft_len + b0 : nullptr;
        AuxDev as = a;
        if (as.p_g) as.p_g += b0 * k;
        if (as.q_g) as.q_g += b0 * k;
        if (as.resid_mass) as.resid_mass += b0;
        if (as.argmax) as.argmax += b0 * (k + 1);
        if (as.seq_status) as.seq_status += b0;
        if (as.draw_row) as.draw_row += b0;
        if (as.draw_kind) as.draw_kind += b0;
        float2 *p0 = partials + b0 * per_seq_items;
        Decision *dc0 = decisions + b0;
        double2 *m0 = masses + b0 * nc;
        int32_t *o0 = out_tokens + b0 * (k + 1);

        if (ev_begin && b0 == 0 && hipEventRecord(ev_begin, stream) != hipSuccess)
            return SPEC_ELAUNCH;
        hipLaunchKernelGGL(k_rowstats<D>, dim3((unsigned)(nb * per_seq_items)), dim3(kThreads),
                           0, stream, t0, d0, l0, temperature + b0, k, V, nc, p0);
        if (ev_end && b0 + nb >= B && hipEventRecord(ev_end, stream) != hipSuccess)
            return SPEC_ELAUNCH;
        hipLaunchKernelGGL(k_decide<D>, dim3((unsigned)nb), dim3(kWave), 0, stream, t0, d0, g0,
                           l0, temperature + b0, k, V, nc, key0, key1,
                           seq_base + (uint32_t)b0, p0, dc0, o0, num_accepted + b0, as);
        hipLaunchKernelGGL(k_residual_mass<D>, dim3((unsigned)(nb * nc)), dim3(kThreads), 0,
                           stream, t0, d0, k, V, nc, dc0, m0);
        hipLaunchKernelGGL(k_locate<D>, dim3((unsigned)nb), dim3(kThreads), 0, stream, t0, d0, k,
                           V, nc, dc0, m0, o0, as);
        if (hipGetLastError() != hipSuccess)
            return SPEC_ELAUNCH;
    }
    return SPEC_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

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
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    if (dtype == SPEC_F32)
        return launch_all<F32>(target_logits, draft_logits, draft_tokens, draft_len, temperature,
                               B, k, V, seed, seq_base, out_tokens, num_accepted, aux, lay, ws,
                               st);
    return launch_all<BF16>(target_logits, draft_logits, draft_tokens, draft_len, temperature, B,
                            k, V, seed, seq_base, out_tokens, num_accepted, aux, lay, ws, st);
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
