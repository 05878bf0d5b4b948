// nucleus.hip -- the top-k and top-p (nucleus) filters of the verification
// step on MI355X (gfx950): one workgroup per filtered row finds the row's
// threshold logit and kept mass (k_filter for bf16 rows, k_nucleus for fp32
// rows; launched from verify.hip).
#include "verify.h"

namespace spv {

// ===========================================================================
// Top-k and top-p. The pages require verification to use the target's own
// sampling parameters, temperature and top-p ("Speculative Decoding and the
// Art of Fast LLM Inference", "Why It Stays Exact", key limitation). Top-k
// keeps whole levels (equal logits) from the top until they hold at least
// top_k tokens; top-p then keeps whole levels from the top until their mass
// reaches top_p of what is left; the row is renormalised over what is kept,
// and the draft rows get the same rule. Masses are fixed-point integers:
// each token weighs floor(2^((x-m)s) * 2^fix_bits), m the row max, so every
// sum is exact and independent of the order of the adds, and the target mass
// ceil(top_p * total) is formed exactly in 128 bits.
//
// bf16 rows (k_filter) take one pass that counts the tokens of each bf16
// value: tokens of one value weigh the same, so a value's mass is its count
// times one token's weight, and neither the counts nor the window they live
// in depend on the row max, which comes out of the counts. fp32 rows
// (k_nucleus), and the bf16 rows the count cannot settle, go through an
// exact radix select over an order-preserving key of the logit: digits of
// 12 bits (then the rest), most significant first; each pass streams the row
// and adds every token's weight (and count) to a 4096-bin LDS histogram of
// the next digit among the tokens that match the digits found so far.
// ===========================================================================
constexpr int kDigitBits = 12;
constexpr int kBins = 1 << kDigitBits;

template <class D>
__device__ inline uint32_t order_key(float x)
{
    uint32_t u = x == 0.f ? 0u : __float_as_uint(x);  // -0 and +0: one level
    if (D::kKeyBits == 16)
        u >>= 16;  // a widened bf16 has 16 low zero bits
    const uint32_t top = 1u << (D::kKeyBits - 1);
    const uint32_t mask = D::kKeyBits == 32 ? 0xffffffffu : 0xffffu;
    return (u & top) ? (~u & mask) : (u | top);
}

template <class D>
__device__ inline float key_value(uint32_t key)
{
    const uint32_t top = 1u << (D::kKeyBits - 1);
    const uint32_t mask = D::kKeyBits == 32 ? 0xffffffffu : 0xffffu;
    uint32_t u = (key & top) ? (key & ~top) : (~key & mask);
    if (D::kKeyBits == 16)
        u <<= 16;
    return __uint_as_float(u);
}

// ceil(top_p * total) for 0 < top_p < 1, exactly.
__device__ inline uint64_t mass_target(uint64_t total, float top_p)
{
    int e;
    const float fr = frexpf(top_p, &e);  // top_p = fr * 2^e, fr in [0.5, 1)
    const uint64_t mant = (uint64_t)(fr * 16777216.0f);  // 24-bit integer, exact
    const uint64_t lo = total * mant, hi = __umul64hi(total, mant);
    const int sh = 24 - e;  // top_p = mant * 2^-sh, sh >= 24
    if (sh >= 128)
        return (hi | lo) ? 1 : 0;
    if (sh >= 64) {
        const int r = sh - 64;
        const uint64_t q = r == 0 ? hi : hi >> r;
        const bool rem = lo != 0 || (r > 0 && (hi & ((1ull << r) - 1)) != 0);
        return q + (rem ? 1 : 0);
    }
    const uint64_t q = (hi << (64 - sh)) | (lo >> sh);
    return q + ((lo & ((1ull << sh) - 1)) != 0 ? 1 : 0);
}

constexpr int kNucWaves = kNucThreads / kWave;
constexpr int kNucTiles = 8;  // 16-byte loads in flight per thread (counting pass)

struct RadixBins {
    unsigned long long hist[kBins];  // fixed-point mass per digit
    uint32_t cnt[kBins];             // elements per digit (top-k)
};

// The counting window of a bf16 row: entry (u - kTinyBits) | sign << 12 for
// the magnitude bits u of the values in [2^-14, 2^18) of either sign, so one
// entry per bf16 value and 8192 in all. In value order (position q from the
// top): the positive entries from the largest (q < kSmallPos), the values
// below 2^-14 in magnitude (q = kSmallPos), the negative entries from the
// smallest magnitude.
constexpr int kWinKeys = 8192;
constexpr uint32_t kTinyBits = 113u << 7;  // bf16 magnitude bits of 2^-14
constexpr int kSmallPos = kWinKeys / 2;
constexpr int kOrderPos = kWinKeys + 1;
constexpr int kSmallCap = 2048;  // listed values below 2^-14 (not zero) per row

// LDS of the radix passes (k_nucleus, k_filter_fallback).
struct NucleusShared {
    RadixBins rx;
    unsigned long long wsum[kNucWaves];
    unsigned long long above;
    int digit;
    float rs;  // row max
};

// LDS of the counting pass (k_filter).
struct alignas(16) CountShared {
    uint32_t cnt[kWinKeys];           // tokens per window entry
    unsigned short small[kSmallCap];  // bits of the values below 2^-14
    // Tokens below 2^-14 (listed), zeros, tokens at or below -2^18; the
    // largest order key seen (+1 for the low ones); any NaN or value at or
    // above 2^18.
    uint32_t n_small, n_zero, n_low, max_key, low_key, low_min, odd;
    // Thresholds from the counts: the mass of the small values, the count
    // and mass totals per wave, the kept mass of top-k, and whether the
    // crossing fell where the counts cannot settle it.
    unsigned long long small_mass, kept;
    unsigned long long wcnt[kNucWaves], wsum[kNucWaves];
    uint32_t found;
    // A crossing among the small values or the low ones: where (kSmall,
    // kLow; top-k, then the nucleus), the count and mass before the small
    // values, the level found.
    uint32_t where, where_p, level_key;
    unsigned long long before_c, before_m;
};

// Visits every element of row[0, V) as fp32 (16-byte loads where aligned).
template <class D, class F>
__device__ __forceinline__ void for_each_logit(const typename D::Elem *row, int64_t V, F &&f)
{
    const Span sp = make_span<D>(row, 0, V);
    const u32x4 *vrow = reinterpret_cast<const u32x4 *>(row + sp.a);
    const int tid = threadIdx.x;
    for (int64_t base = 0; base < sp.ngroups; base += (int64_t)kNucThreads * kTiles) {
        u32x4 r[kTiles];
#pragma unroll
        for (int u = 0; u < kTiles; ++u) {
            const int64_t vi = base + u * kNucThreads + tid;
            r[u] = vi < sp.ngroups ? vrow[vi] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kTiles; ++u) {
            if (base + u * kNucThreads + tid < sp.ngroups) {
                float x[D::kVec];
                D::unpack(r[u], x);
#pragma unroll
                for (int j = 0; j < D::kVec; ++j)
                    f(x[j]);
            }
        }
    }
    if (sp.s + tid < sp.a)
        f(D::at(row, sp.s + tid));
    if (sp.z + tid < sp.e)
        f(D::at(row, sp.z + tid));
}

// Two 16-bit lanes of one 32-bit register (packed integer arithmetic).
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

__device__ inline u16x2 as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }
__device__ inline uint32_t as_u32(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ inline uint32_t as_u32(i16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// Sum over the workgroup of one value per thread.
__device__ inline uint64_t block_sum(uint64_t v, NucleusShared &sh)
{
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    __syncthreads();  // wsum is free
    if (lane == 0)
        sh.wsum[wave] = v;
    __syncthreads();
    uint64_t t = 0;
    for (int q = 0; q < kNucWaves; ++q)
        t += sh.wsum[q];
    return t;
}

// Crossing search over n masses in the order i = 0, 1, ... (thread t owns
// [t*per, (t+1)*per), per = ceil(n / threads), and `mass` returns 0 from n
// on): the first i at which the running sum reaches `need` (>= 1) goes to
// sh.digit, the sum before it to sh.above; sh.digit = -1 if all n together
// stay below `need`. Integer sums: the result does not
// depend on the order of any addition.
template <class M>
__device__ inline void crossing(int n, uint64_t need, M &&mass, NucleusShared &sh)
{
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int per = (n + kNucThreads - 1) / kNucThreads;  // mass(q) is 0 for q >= n
    const bool owns = tid * per < n;
    uint64_t loc = 0;
    if (owns)
        for (int q = 0; q < per; ++q)
            loc += mass(tid * per + q);
    uint64_t incl = loc;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint64_t o = __shfl_up(incl, off, kWave);
        if (lane >= off)
            incl += o;
    }
    if (tid == 0)
        sh.digit = -1;
    __syncthreads();  // wsum is free; digit is reset
    if (lane == kWave - 1)
        sh.wsum[wave] = incl;
    __syncthreads();
    uint64_t before = 0;
    for (int q = 0; q < wave; ++q)
        before += sh.wsum[q];
    const uint64_t excl = before + incl - loc;
    if (owns && excl < need && need <= excl + loc) {
        uint64_t cum = excl;
        for (int q = 0; q < per; ++q) {
            const uint64_t mq = mass(tid * per + q);
            if (cum + mq >= need) {
                sh.digit = tid * per + q;
                sh.above = cum;
                break;
            }
            cum += mq;
        }
    }
    __syncthreads();
}

// Result of a selection: the threshold key (keep keys >= it) and the
// fixed-point mass of the kept tokens.
struct Selection {
    uint32_t key;
    unsigned long long kept;
};

// Radix select over the order keys of a row, kDigitBits at a time from the
// top, among the tokens with key >= lo. BY_COUNT: the crossing of the
// running count reaching `count` (top-k); otherwise of the running
// fixed-point mass reaching ceil(top_p * the mass of those tokens).
template <class D, bool BY_COUNT>
__device__ __forceinline__ Selection radix_select(const typename D::Elem *row, int64_t V, float m, float scale,
                                  float fscale, float zlim, uint32_t lo, int64_t count,
                                  float top_p, NucleusShared &sh)
{
    constexpr int KB = D::kKeyBits;
    const int tid = threadIdx.x;
    auto fixed = [&](float x) {
        return (unsigned long long)(exp2_fast((x - m) * scale) * fscale);
    };
    uint64_t need = 0, above = 0, mass_above = 0;
    uint32_t prefix = 0;
    int done = 0;
    Selection res{0u, 0ull};
    while (done < KB) {
        const int w = min(kDigitBits, KB - done);
        const int nb = 1 << w;
        for (int q = tid; q < nb; q += kNucThreads) {
            sh.rx.hist[q] = 0;
            sh.rx.cnt[q] = 0;
        }
        __syncthreads();
        unsigned long long mine = 0;
        for_each_logit<D>(row, V, [&](float x) {
            const float t = (x - m) * scale;
            if (!BY_COUNT && t < zlim)
                return;  // weighs 0 (a count still counts it)
            const uint32_t key = order_key<D>(x);
            if (key < lo || (done != 0 && (key >> (KB - done)) != prefix))
                return;
            const uint32_t bin = (key >> (KB - done - w)) & (uint32_t)(nb - 1);
            if (BY_COUNT)
                atomicAdd(&sh.rx.cnt[bin], 1u);
            if (t >= zlim) {
                const unsigned long long wf = fixed(x);
                atomicAdd(&sh.rx.hist[bin], wf);
                mine += wf;
            }
        });
        if (done == 0)
            need = BY_COUNT ? (uint64_t)count : mass_target(block_sum(mine, sh), top_p);
        __syncthreads();
        if (BY_COUNT)
            crossing(nb, need - above,
                     [&](int q) -> uint64_t { return sh.rx.cnt[nb - 1 - q]; }, sh);
        else
            crossing(nb, need - above, [&](int q) -> uint64_t { return sh.rx.hist[nb - 1 - q]; },
                     sh);
        const int d = nb - 1 - max(sh.digit, 0);  // the crossing always exists here
        above += sh.above;
        if (BY_COUNT) {  // the masses of the bins above d
            uint64_t mm = 0;
            for (int q = tid; q < nb; q += kNucThreads)
                mm += q > d ? sh.rx.hist[q] : 0ull;
            mass_above += block_sum(mm, sh);
        }
        prefix = (prefix << w) | (uint32_t)d;
        done += w;
        if (done == KB)
            res = Selection{prefix, (BY_COUNT ? mass_above : above) + sh.rx.hist[d]};
        __syncthreads();  // the bins are cleared next pass
    }
    return res;
}

// Top-k, then top-p, by radix selects (m the row max); the result goes to
// *out as (threshold logit, kept mass, m, 0).
template <class D>
__device__ __forceinline__ void radix_filter(const typename D::Elem *row, int64_t V, float m,
                                             float scale, float fscale, float zlim, bool k_on,
                                             int64_t top_k, bool p_on, float top_p, float4 *out,
                                             NucleusShared &sh)
{
    uint32_t lo = 0;
    if (k_on) {
        const Selection sk =
            radix_select<D, true>(row, V, m, scale, fscale, zlim, 0u, top_k, top_p, sh);
        if (!p_on) {
            if (threadIdx.x == 0)
                *out = make_float4(key_value<D>(sk.key), (float)sk.kept / fscale, m, 0.f);
            return;
        }
        lo = sk.key;
    }
    const Selection sp = radix_select<D, false>(row, V, m, scale, fscale, zlim, lo, 0, top_p, sh);
    if (threadIdx.x == 0)
        *out = make_float4(key_value<D>(sp.key), (float)sp.kept / fscale, m, 0.f);
}

// The row max by a pass over the row (the largest non-NaN logit).
template <class D>
__device__ inline float row_max(const typename D::Elem *row, int64_t V, NucleusShared &sh)
{
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    float mx = -INFINITY;
    for_each_logit<D>(row, V, [&](float x) { mx = fmaxf(mx, x); });
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1)
        mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
    __syncthreads();  // wsum is free
    if (lane == 0)
        sh.wsum[wave] = __float_as_uint(mx);
    __syncthreads();
    float m = -INFINITY;
    for (int q = 0; q < kNucWaves; ++q)
        m = fmaxf(m, __uint_as_float((uint32_t)sh.wsum[q]));
    return m;
}

// Value and order key of window entry e.
__device__ inline uint32_t entry_bits(uint32_t e)
{
    const uint32_t mag = kTinyBits + (e & 0xfffu);
    return (e & 0x1000u) ? (0x8000u | mag) : mag;
}
__device__ inline float entry_value(uint32_t e) { return __uint_as_float(entry_bits(e) << 16); }
__device__ inline uint32_t bf16_key(uint32_t r)  // order key of bf16 bits (+0 and -0: one)
{
    return (r & 0x8000u) ? ((r & 0x7fffu) ? (~r & 0xffffu) : 0x8000u) : (r | 0x8000u);
}
// Window entry at order position q (q != kSmallPos).
__device__ inline uint32_t pos_entry(int q)
{
    return q < kSmallPos ? (uint32_t)(kSmallPos - 1 - q) : (uint32_t)(q - 1);
}

// The counting pass over a bf16 row: window counts, the listed small values,
// the zeros and low values, and the row max key, all in sh.
template <class D>
__device__ __forceinline__ void count_row(const typename D::Elem *row, int64_t V,
                                          CountShared &sh)
{
    const int tid = threadIdx.x;
    for (int q = tid; q < kWinKeys; q += kNucThreads)
        sh.cnt[q] = 0;
    if (tid == 0) {
        sh.n_small = sh.n_zero = sh.n_low = 0;
        sh.max_key = sh.low_key = sh.odd = 0;
        sh.low_min = 0xffffffffu;
        sh.small_mass = 0;
        sh.found = 0;
        sh.where = sh.where_p = 0;
        sh.level_key = 0;
    }
    __syncthreads();
    uint32_t zeros = 0, lows = 0, low_key = 0, low_min = 0xffffffffu, odd = 0;
    u16x2 kmax = (u16x2)0;  // largest order key, per 16-bit lane
    // A token outside the window (its count, if any, is taken back by the
    // caller).
    auto rare = [&](uint32_t r) {
        const uint32_t u = r & 0x7fffu;
        if (u == 0) {
            ++zeros;
        } else if (u < kTinyBits) {
            const uint32_t i = atomicAdd(&sh.n_small, 1u);
            if (i < (uint32_t)kSmallCap)
                sh.small[i] = (unsigned short)r;
        } else if ((r & 0x8000u) && u <= 0x7f80u) {  // at or below -2^18, -inf included
            ++lows;
            low_key = max(low_key, bf16_key(r) + 1u);
            low_min = min(low_min, bf16_key(r) + 1u);
        } else {
            odd = 1;  // at or above 2^18, or NaN
        }
    };
    // Eight tokens (one 16-byte load), two per 32-bit word in 16-bit lanes:
    // t = r - kTinyBits; a window token has t in [0, 0x1000) (positive) or
    // [0x8000, 0x9000) (negative), so bits 12..14 of t are zero exactly for
    // the window, and its entry is t's low 12 bits with the sign (bit 15)
    // moved to bit 12. Every token is counted at that entry; the few outside
    // the window are taken back afterwards (see below). Returns whether the
    // group holds any.
    const uint32_t tb2 = kTinyBits * 0x10001u;
    auto visit_group = [&](const u32x4 &g) -> bool {
        const uint32_t w[4] = {g.x, g.y, g.z, g.w};
        uint32_t any = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t t = as_u32(as_u16x2(w[j]) - as_u16x2(tb2));
            const uint32_t e =
                (t & 0x0fff0fffu) | (as_u32(as_u16x2(t) >> (unsigned short)3) & 0x10001000u);
            any |= t;
            // order key: positive r -> r | 0x8000, negative r -> ~r
            const uint32_t neg = as_u32(__builtin_bit_cast(i16x2, w[j]) >> (i16x2)15);
            kmax = __builtin_elementwise_max(kmax, as_u16x2(w[j] ^ (neg | 0x80008000u)));
            atomicAdd(&sh.cnt[e & 0xffffu], 1u);
            atomicAdd(&sh.cnt[e >> 16], 1u);
        }
        return (any & 0x70007000u) != 0;
    };
    // The tokens outside the window of one group, read again: their counts
    // taken back, each handled by `rare` (one copy of this code, however
    // many groups the loop unrolls).
    auto visit_rare_group = [&](const u32x4 *gp) {
        const u32x4 g = *gp;
        const uint32_t w[4] = {g.x, g.y, g.z, g.w};
#pragma unroll 1
        for (int j = 0; j < 8; ++j) {
            const uint32_t r = (w[j >> 1] >> ((j & 1) * 16)) & 0xffffu;
            const uint32_t t = (r - kTinyBits) & 0xffffu;
            if (t & 0x7000u) {
                atomicSub(&sh.cnt[(t & 0xfffu) | ((t >> 3) & 0x1000u)], 1u);
                rare(r);
            }
        }
    };
    auto visit_one = [&](uint32_t r) {
        const uint32_t neg = (r & 0x8000u) ? 0xffffu : 0u;
        kmax = __builtin_elementwise_max(kmax, (u16x2)(unsigned short)(r ^ (neg | 0x8000u)));
        const uint32_t t = (r - kTinyBits) & 0xffffu;
        if (t & 0x7000u)
            rare(r);
        else
            atomicAdd(&sh.cnt[(t & 0xfffu) | ((t >> 3) & 0x1000u)], 1u);
    };
    const Span sp = make_span<D>(row, 0, V);
    const u32x4 *vrow = reinterpret_cast<const u32x4 *>(row + sp.a);
    for (int64_t base = 0; base < sp.ngroups; base += (int64_t)kNucThreads * kNucTiles) {
        u32x4 r[kNucTiles];
#pragma unroll
        for (int u = 0; u < kNucTiles; ++u) {
            const int64_t vi = base + u * kNucThreads + tid;
            r[u] = vi < sp.ngroups ? stream_load(vrow + vi) : u32x4{0u, 0u, 0u, 0u};
        }
        uint32_t rare_groups = 0;  // bit u: group u holds tokens outside the window
#pragma unroll
        for (int u = 0; u < kNucTiles; ++u)
            if (base + u * kNucThreads + tid < sp.ngroups && visit_group(r[u]))
                rare_groups |= 1u << u;
        while (rare_groups) {
            const int u = __builtin_ctz(rare_groups);
            rare_groups &= rare_groups - 1;
            visit_rare_group(vrow + base + u * kNucThreads + tid);
        }
    }
    if (sp.s + tid < sp.a)
        visit_one((uint32_t)__builtin_bit_cast(unsigned short, row[sp.s + tid]));
    if (sp.z + tid < sp.e)
        visit_one((uint32_t)__builtin_bit_cast(unsigned short, row[sp.z + tid]));
    if (zeros)
        atomicAdd(&sh.n_zero, zeros);
    if (lows) {
        atomicAdd(&sh.n_low, lows);
        atomicMax(&sh.low_key, low_key);
        atomicMin(&sh.low_min, low_min);
    }
    if (odd)
        atomicOr(&sh.odd, 1u);
    // The row max key (-0 may stand for +0: the same value).
    uint32_t mk = max((uint32_t)kmax.x, (uint32_t)kmax.y);
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1)
        mk = max(mk, (uint32_t)__shfl_xor((int)mk, off, kWave));
    if ((tid & (kWave - 1)) == 0)
        atomicMax(&sh.max_key, mk);
    __syncthreads();
}

// Where a crossing fell when it is not in the window (CountShared::where).
constexpr uint32_t kSmall = 1, kLow = 2;

// Sum over the workgroup of one value per thread.
__device__ inline uint64_t block_sum(uint64_t v, CountShared &sh)
{
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    __syncthreads();  // wsum is free
    if (lane == 0)
        sh.wsum[wave] = v;
    __syncthreads();
    uint64_t t = 0;
    for (int q = 0; q < kNucWaves; ++q)
        t += sh.wsum[q];
    return t;
}

// Window entries of thread t, 16 in value order: for t < 256 the positive
// entries 4095 - 16t - j, for t >= 256 the negative entries 16t + j
// (j = 0..15); the small values come after thread 255's.
__device__ inline uint32_t own_entry(int t, int j)
{
    return t < kNucThreads / 2 ? (uint32_t)(kWinKeys / 2 - 1 - 16 * t - j) : (uint32_t)(16 * t + j);
}

// Inclusive block scan of one pair of sums per thread (counts, masses), in
// thread order; returns the exclusive prefixes. wsum / wcnt hold the wave
// totals afterwards.
__device__ inline void scan_pair(uint64_t &c, uint64_t &m, CountShared &sh)
{
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    uint64_t ic = c, im = m;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint64_t oc = __shfl_up(ic, off, kWave), om = __shfl_up(im, off, kWave);
        if (lane >= off) {
            ic += oc;
            im += om;
        }
    }
    if (lane == kWave - 1) {
        sh.wcnt[wave] = ic;
        sh.wsum[wave] = im;
    }
    __syncthreads();
    uint64_t bc = 0, bm = 0;
    for (int q = 0; q < wave; ++q) {
        bc += sh.wcnt[q];
        bm += sh.wsum[q];
    }
    c = bc + ic - c;
    m = bm + im - m;
}

// Filter record flags (the record's fourth value), written by k_filter for
// every row and read by k_filter_fallback: settled by the counts, or nothing
// to do; radix passes needed, with the row max in the record; radix passes
// needed after a pass for the row max (NaN or a value at or above 2^18);
// a row without a filter (k_rowstats gives its row statistics).
constexpr float kSettled = 0.f, kRadix = 1.f, kRadixMax = 2.f, kRowStats = 3.f;

// Per-row set-up shared by k_filter and k_filter_fallback.
template <class D>
struct FilterRow {
    const typename D::Elem *row;
    float4 *out;
    float tau, top_p;
    int64_t top_k;
    bool valid, greedy, filtered, needed, p_on, k_on;
};

template <class D>
__device__ inline FilterRow<D> filter_row(const Params &p, uint32_t rb)
{
    using E = typename D::Elem;
    const int k = p.k, rows = 2 * k + 1;
    // rb = b * rows + slot; 32-bit decode: the row index fits
    const int slot = (int)(rb % (uint32_t)rows);
    const int64_t b = rb / (uint32_t)rows;
    const int L = p.draft_len ? p.draft_len[b] : k;
    FilterRow<D> f;
    f.tau = p.temperature[b];
    f.valid = valid_len(L, k) && valid_temp(f.tau);  // else the decision reports it
    f.greedy = f.tau == 0.f;
    f.filtered = f.valid && !f.greedy && seq_filtered(p, b);
    f.top_p = p.top_p ? p.top_p[b] : 1.f;
    f.top_k = p.top_k ? (int64_t)p.top_k[b] : 0;
    f.p_on = f.top_p < 1.f;
    f.k_on = f.top_k > 0 && f.top_k < (int64_t)p.V;
    const bool is_target = slot <= k;
    const int i = is_target ? slot : slot - (k + 1);
    // A filtered row with top_p <= 0 or NaN is never read: the decision
    // reports the sequence.
    f.needed = f.valid && (is_target ? i <= L : (!f.greedy && i < L)) &&
               (!f.filtered || f.top_p > 0.f);
    f.row = is_target ? static_cast<const E *>(p.target) + (b * (k + 1) + i) * (int64_t)p.V
                      : static_cast<const E *>(p.draft) + (b * k + i) * (int64_t)p.V;
    f.out = p.nucleus + b * rows + slot;
    return f;
}

// One workgroup per row of a call with top-k or top-p parameters (bf16
// logits): for a row of a sampling sequence with a filter, the counting pass
// and the thresholds from the counts, with the row max. What the counts
// cannot settle is left to k_filter_fallback (kept apart so that this
// kernel's registers hold its loop without spilling); the rows without a
// filter are left to k_rowstats.
template <class D>
__global__ __launch_bounds__(kNucThreads, 6) void k_filter(Params p)
{
    static_assert(D::kKeyBits == 16, "the counting window is for bf16 rows");
    __shared__ CountShared sh;
    const FilterRow<D> f = filter_row<D>(p, blockIdx.x);
    const int tid = threadIdx.x;
    if (!f.filtered || !f.needed) {
        if (tid == 0)
            *f.out = make_float4(0.f, 0.f, 0.f, f.needed ? kRowStats : kSettled);
        return;
    }
    const bool p_on = f.p_on, k_on = f.k_on;
    const int64_t top_k = f.top_k;
    const float top_p = f.top_p;
    const float scale = temp_scale(f.tau);
    const float fscale = __uint_as_float((uint32_t)(127 + p.fix_bits) << 23);  // 2^fix_bits
    float4 *const out = f.out;

    count_row<D>(f.row, p.V, sh);
    if (sh.odd) {  // NaN or a value at or above 2^18: the row max by a pass of its own
        if (tid == 0)
            *out = make_float4(0.f, 0.f, 0.f, kRadixMax);
        return;
    }
    const float m = key_value<D>(sh.max_key);
    auto fixed = [&](float x) {
        return (unsigned long long)(exp2_fast((x - m) * scale) * fscale);
    };
    const uint32_t n_small = sh.n_small, n_zero = sh.n_zero, n_low = sh.n_low;
    // The tokens at or below -2^18: one level (all equal, as masked tokens
    // usually are) or several; the weight of the largest of them.
    const bool low_one = n_low == 0 || sh.low_min == sh.low_key;
    const float low_val = n_low ? key_value<D>(sh.low_key - 1u) : 0.f;
    const uint64_t low_w = n_low ? fixed(low_val) : 0;
    const uint64_t low_mass = low_one ? (uint64_t)n_low * low_w : 0;
    // Settled by the counts unless the list is full, or (top-p alone) the
    // low tokens weigh something and hold several levels.
    if (n_small <= (uint32_t)kSmallCap && (k_on || low_one || low_w == 0)) {
        // The small values: zeros weigh one amount, the listed ones each
        // their own.
        if (n_small + n_zero) {
            uint64_t part = tid == 0 ? (uint64_t)n_zero * fixed(0.f) : 0;
            for (uint32_t q = tid; q < n_small; q += kNucThreads)
                part += fixed(__uint_as_float((uint32_t)sh.small[q] << 16));
            if (part)
                atomicAdd(&sh.small_mass, (unsigned long long)part);
        }
        // This thread's 16 entries: counts and masses.
        constexpr int kOwn = kWinKeys / kNucThreads;
        static_assert(kOwn == 16, "16 window entries per thread");
        const bool upper = tid < kNucThreads / 2;
        const uint32_t lo_entry = upper ? own_entry(tid, kOwn - 1) : own_entry(tid, 0);
        uint32_t cnt[kOwn];
#pragma unroll
        for (int v = 0; v < kOwn / 4; ++v) {
            const uint4 q4 = *reinterpret_cast<const uint4 *>(&sh.cnt[lo_entry + 4 * v]);
            cnt[4 * v] = q4.x;
            cnt[4 * v + 1] = q4.y;
            cnt[4 * v + 2] = q4.z;
            cnt[4 * v + 3] = q4.w;
        }
        // Count and mass of position j (value order); the owner of a
        // crossing computes them again rather than keep 16 masses live.
        auto count_of = [&](int j) -> uint32_t { return upper ? cnt[kOwn - 1 - j] : cnt[j]; };
        auto mass_of = [&](int j) -> uint64_t {
            const uint32_t n = count_of(j);
            return n ? (uint64_t)n * fixed(entry_value(own_entry(tid, j))) : 0;
        };
        uint64_t csum = 0, msum = 0;
#pragma unroll
        for (int j = 0; j < kOwn; ++j) {
            csum += count_of(j);
            msum += mass_of(j);
        }
        const uint64_t small_count = (uint64_t)n_small + n_zero;
        const bool last_upper = tid == kNucThreads / 2 - 1;
        if (last_upper)
            csum += small_count;
        uint64_t ec = csum, em = msum;
        scan_pair(ec, em, sh);  // exclusive prefixes; the barrier completes small_mass
        const uint64_t small_mass = sh.small_mass;
        if (!upper)
            em += small_mass;
        uint64_t tot_m = small_mass, tot_c = 0;  // window and small values
        for (int q = 0; q < kNucWaves; ++q) {
            tot_m += sh.wsum[q];
            tot_c += sh.wcnt[q];
        }
        // A crossing among the small values: the workgroup ranks the listed
        // values (and the zeros, one level) by their order key and finds the
        // level where the running count or mass, from the largest, reaches
        // `need` (counted from the first small value). The window counts
        // are no longer read, so their LDS holds the listed values' masses.
        auto small_level = [&](bool by_count, uint64_t need) -> uint32_t {
            uint64_t *const smass = reinterpret_cast<uint64_t *>(sh.cnt);
            if (!by_count)
                for (uint32_t q = tid; q < n_small; q += kNucThreads)
                    smass[q] = fixed(__uint_as_float((uint32_t)sh.small[q] << 16));
            if (tid == 0)
                sh.level_key = 0;
            __syncthreads();
            const uint64_t zero_amt = by_count ? n_zero : (uint64_t)n_zero * fixed(0.f);
            for (uint32_t q = tid; q < n_small + (n_zero ? 1u : 0u); q += kNucThreads) {
                const uint32_t key = q < n_small ? bf16_key(sh.small[q]) : 0x8000u;
                uint64_t gt = n_zero && 0x8000u > key ? zero_amt : 0;
                uint64_t eq = q == n_small ? zero_amt : 0;
                for (uint32_t j = 0; j < n_small; ++j) {
                    const uint32_t kj = bf16_key(sh.small[j]);
                    const uint64_t amt = by_count ? 1u : smass[j];
                    gt += kj > key ? amt : 0;
                    eq += kj == key ? amt : 0;
                }
                if (gt < need && need <= gt + eq)
                    atomicMax(&sh.level_key, key + 1u);  // every value of the level agrees
            }
            __syncthreads();
            return sh.level_key - 1u;
        };
        // The mass of the small values at or above order key `key`.
        auto small_mass_from = [&](uint32_t key) -> uint64_t {
            uint64_t part = tid == 0 && n_zero && 0x8000u >= key ? (uint64_t)n_zero * fixed(0.f) : 0;
            for (uint32_t q = tid; q < n_small; q += kNucThreads)
                if (bf16_key(sh.small[q]) >= key)
                    part += fixed(__uint_as_float((uint32_t)sh.small[q] << 16));
            return block_sum(part, sh);
        };
        auto result = [&](float thr, uint64_t kept) {
            if (tid == 0)
                *out = make_float4(thr, (float)kept / fscale, m, 0.f);
        };
        uint64_t kept_total = tot_m + low_mass;  // top-p alone: the whole row
        if (k_on) {
            // The top-k threshold: the position where the running count
            // reaches top_k (position kOwn: thread 255's small values;
            // beyond the window and the small values: the low ones).
            const uint64_t need = (uint64_t)top_k;
            if (ec < need && need <= ec + csum) {
                uint64_t cc = ec, cm = em, kept = 0;
                int jk = kOwn;
#pragma unroll
                for (int j = 0; j < kOwn; ++j) {
                    if (jk == kOwn) {
                        cc += count_of(j);
                        cm += mass_of(j);
                        if (cc >= need) {
                            jk = j;
                            kept = cm;
                        }
                    }
                }
                if (jk == kOwn) {
                    sh.where = kSmall;
                    sh.before_c = cc;  // the count and mass before the small values
                    sh.before_m = cm;
                } else {
                    sh.kept = kept;
                    sh.found = 1;
                    if (!p_on)
                        *out = make_float4(entry_value(own_entry(tid, jk)), (float)kept / fscale,
                                           m, 0.f);
                }
            }
            if (tid == 0 && tot_c < need)
                sh.where = kLow;
            __syncthreads();
            const uint32_t where = sh.where;
            if (where == kSmall) {
                const uint32_t key = small_level(true, need - sh.before_c);
                kept_total = sh.before_m + small_mass_from(key);
                if (!p_on) {
                    result(key_value<D>(key), kept_total);
                    return;
                }
            } else if (where == kLow) {
                if (!low_one)
                    goto radix;  // the top_k-th token among several low levels
                kept_total = tot_m + low_mass;
                if (!p_on) {
                    result(low_val, kept_total);
                    return;
                }
            } else {
                if (!sh.found)
                    goto radix;  // no crossing: cannot happen, kept for safety
                if (!p_on)
                    return;  // top-k alone: written by the owner
                kept_total = sh.kept;
            }
        }
        {
            // The nucleus: the position where the running mass reaches
            // ceil(top_p * kept_total); with top-k it lies at or above the
            // top-k threshold.
            const uint64_t need = mass_target(kept_total, top_p);
            const uint64_t own = msum + (last_upper ? small_mass : 0);
            if (em < need && need <= em + own) {
                uint64_t cm = em, kept = 0;
                int jm = kOwn;
#pragma unroll
                for (int j = 0; j < kOwn; ++j) {
                    if (jm == kOwn) {
                        cm += mass_of(j);
                        if (cm >= need) {
                            jm = j;
                            kept = cm;
                        }
                    }
                }
                if (jm == kOwn) {
                    sh.where_p = kSmall;
                    sh.before_m = cm;  // the mass before the small values
                } else {
                    *out = make_float4(entry_value(own_entry(tid, jm)), (float)kept / fscale, m,
                                       0.f);
                }
            }
            if (tid == 0 && tot_m < need)
                sh.where_p = kLow;  // only when the low tokens weigh something
            __syncthreads();
            const uint32_t where = sh.where_p;
            if (where == kSmall) {
                const uint32_t key = small_level(false, need - sh.before_m);
                result(key_value<D>(key), sh.before_m + small_mass_from(key));
                return;
            }
            if (where == kLow) {
                if (!low_one)
                    goto radix;
                result(low_val, tot_m + low_mass);
                return;
            }
            return;  // written by the owner
        }
    }
radix:
    if (tid == 0)
        *out = make_float4(0.f, 0.f, m, kRadix);
}

// After k_filter, in a call with top-k or top-p parameters (bf16 logits):
// the radix passes for the filtered rows that k_filter flagged (a few rows a
// call, if any; the rows without a filter get their row statistics from
// k_rowstats, launched after this kernel). One workgroup per kFallbackRows
// rows: each wave reads one row's flag, and the workgroup takes the flagged
// ones in turn. With nothing to do, as in most calls, a workgroup per row
// cost about 9 us on c5 just in launching and retiring them.
constexpr int kFallbackRows = kNucWaves;  // the host's grid assumes kNucThreads / kWave
template <class D>
__global__ __launch_bounds__(kNucThreads, 6) void k_filter_fallback(Params p)
{
    __shared__ NucleusShared sh;
    __shared__ uint32_t todo;
    const int tid = threadIdx.x, wave = tid / kWave;
    const uint32_t nrows = (uint32_t)p.B * (uint32_t)(2 * p.k + 1);
    const uint32_t r0 = blockIdx.x * (uint32_t)kFallbackRows;  // 32-bit: the row index fits
    if (tid == 0)
        todo = 0;
    __syncthreads();
    if ((tid & (kWave - 1)) == 0 && r0 + wave < nrows) {
        const float w = p.nucleus[r0 + wave].w;
        if (!(w == kSettled || w == kRowStats))
            atomicOr(&todo, 1u << wave);
    }
    __syncthreads();
    uint32_t mask = todo;  // the same in every thread
    const float fscale = __uint_as_float((uint32_t)(127 + p.fix_bits) << 23);  // 2^fix_bits
    const float zlim = -(float)(p.fix_bits + 2);  // (x - m) * scale below this: weight 0
    while (mask) {
        const uint32_t rb = r0 + (uint32_t)__builtin_ctz(mask);
        mask &= mask - 1;
        const float4 rec = p.nucleus[rb];
        const FilterRow<D> f = filter_row<D>(p, rb);
        const float scale = temp_scale(f.tau);
        const float m = rec.w == kRadixMax ? row_max<D>(f.row, p.V, sh) : rec.z;
        __syncthreads();
        radix_filter<D>(f.row, p.V, m, scale, fscale, zlim, f.k_on, f.top_k, f.p_on, f.top_p,
                        f.out, sh);
        __syncthreads();  // sh is reused by the next flagged row
    }
}

// One workgroup per fp32 row of every sampling sequence with a top-k or
// top-p filter (the row max from the row statistics), by the radix passes.
template <class D>
__global__ __launch_bounds__(kNucThreads, 6) void k_nucleus(Params p)
{
    using E = typename D::Elem;
    __shared__ NucleusShared sh;
    const int k = p.k, nc = p.nc, rows = 2 * k + 1;
    const uint32_t rb = blockIdx.x;  // 32-bit decode: the grid index fits
    const int slot = (int)(rb % (uint32_t)rows);
    const int64_t b = rb / (uint32_t)rows;
    const int tid = threadIdx.x;
    const int L = p.draft_len ? p.draft_len[b] : k;
    const float tau = p.temperature[b];
    const float top_p = p.top_p ? p.top_p[b] : 1.f;
    const int64_t top_k = p.top_k ? (int64_t)p.top_k[b] : 0;
    if (!valid_len(L, k) || !valid_temp(tau) || tau == 0.f || !(top_p > 0.f))
        return;
    const bool p_on = top_p < 1.f;
    const bool k_on = top_k > 0 && top_k < (int64_t)p.V;
    if (!p_on && !k_on)
        return;
    const bool is_target = slot <= k;
    const int i = is_target ? slot : slot - (k + 1);
    if (is_target ? i > L : i >= L)
        return;
    const E *row = is_target ? static_cast<const E *>(p.target) + (b * (k + 1) + i) * (int64_t)p.V
                             : static_cast<const E *>(p.draft) + (b * k + i) * (int64_t)p.V;
    const float scale = temp_scale(tau);
    const float fscale = __uint_as_float((uint32_t)(127 + p.fix_bits) << 23);  // 2^fix_bits
    const float zlim = -(float)(p.fix_bits + 2);  // (x - m) * scale below this: weight 0
    if (tid == 0) {
        const float2 *pp = p.partials + (b * rows + slot) * (int64_t)nc;
        float m = -INFINITY;  // the row max: the largest chunk max
        for (int c = 0; c < nc; ++c)
            m = fmaxf(m, pp[c].x);
        sh.rs = m;
    }
    __syncthreads();
    radix_filter<D>(row, p.V, sh.rs, scale, fscale, zlim, k_on, top_k, p_on, top_p,
                    p.nucleus + b * rows + slot, sh);
}

template __global__ void k_nucleus<F32>(Params p);
template __global__ void k_filter<BF16>(Params p);
template __global__ void k_filter_fallback<BF16>(Params p);

}  // namespace spv
