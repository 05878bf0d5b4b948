// nucleus.hip -- the top-k and top-p (nucleus) filters of the verification
// step on MI355X (gfx950): one workgroup per filtered row finds the row's
// threshold logit and kept mass (k_nucleus, launched from verify.hip).
#include "verify.h"

namespace spv {

// ===========================================================================
// Top-p. The pages require verification to use the target's own sampling
// parameters, temperature and top-p ("Speculative Decoding and the Art of
// Fast LLM Inference", "Why It Stays Exact", key limitation). Each row keeps
// whole probability levels (equal logits) from the top until their mass
// reaches top_p of the row's mass, and is renormalised over them; the draft
// rows get the same rule. k_nucleus finds, per row, the smallest kept logit
// and the kept mass by an exact radix select over an order-preserving key of
// the logit: digits of 12 bits (then the rest), most significant first.
// Each pass streams the row and adds every element's weight 2^((x-m)s), in
// fixed point (fix_bits fraction bits), to a 4096-bin LDS histogram of the
// next digit among the elements that match the digits found so far; 64-bit
// integer sums make the result independent of the order of the adds. The
// crossing is found by an integer scan from the top bin; the target mass
// ceil(top_p * total) is formed exactly in 128 bits. A bf16 row first takes
// one pass that counts the elements of each key within kWinKeys keys below
// the row max (a key's fixed-point mass is its count times one element's)
// and adds up the rest; only when the crossing lies below that window does
// the row go through the radix passes. Both give the same integers, and both
// skip the elements whose fixed-point mass is 0.
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

// bf16 rows: exact counts per key over kWinKeys entries of a compressed key
// order below the row max. Magnitudes under 2^-14 (and zero) share the entry
// kTinyIdx, whose mass is summed element by element instead; every other
// entry is one bf16 value. From a max of about 16, 8192 entries reach below
// -2^30, so the rows' mass lies inside the window. One more counter, at
// kWinKeys, takes the values beyond the window.
constexpr int kWinKeys = 8192;
constexpr uint32_t kTinyBits = 113u << 7;  // bf16 magnitude bits of 2^-14
constexpr uint32_t kTinyIdx = 0x8000u - kTinyBits;

// Compressed index of a 16-bit order key: monotone, and one-to-one except
// that all magnitudes below 2^-14 map to kTinyIdx.
__device__ inline uint32_t compress_key(uint32_t key)
{
    if (key >= 0x8000u) {
        const uint32_t u = key - 0x8000u;  // magnitude bits of a positive value
        return u < kTinyBits ? kTinyIdx : kTinyIdx + 1u + (u - kTinyBits);
    }
    const uint32_t u = 0x7fffu - key;  // magnitude bits of a negative value
    return u < kTinyBits ? kTinyIdx : kTinyIdx - 1u - (u - kTinyBits);
}

// The order key of a compressed index other than kTinyIdx.
__device__ inline uint32_t expand_key(uint32_t c)
{
    return c > kTinyIdx ? 0x8000u + (c - kTinyIdx - 1u + kTinyBits)
                        : 0x7fffu - (kTinyIdx - 1u - c + kTinyBits);
}

constexpr int kNucWaves = kNucThreads / kWave;
constexpr int kNucTiles = 4;  // 16-byte loads in flight per thread (counting pass)

struct RadixBins {
    unsigned long long hist[kBins];  // fixed-point mass per digit
    uint32_t cnt[kBins];             // elements per digit (top-k)
};

struct NucleusShared {
    union {
        RadixBins rx;                 // radix passes
        uint32_t cnt[kWinKeys + 1];   // window pass: elements per key
    };
    unsigned long long wsum[kNucWaves];
    unsigned long long above;
    int digit;
    float rs;  // row max
    float tc;  // window pass: entries below this (x - m) * scale are not counted
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
// [t*per, (t+1)*per)): the first i at which the running sum reaches `need`
// (>= 1) goes to sh.digit, the sum before it to sh.above; sh.digit = -1 if
// all n together stay below `need`. Integer sums: the result does not
// depend on the order of any addition.
template <class M>
__device__ inline void crossing(int n, uint64_t need, M &&mass, NucleusShared &sh)
{
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int per = n >= kNucThreads ? n / kNucThreads : 1;
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

// One counting pass over a bf16 row (see the top-p notes above). Top-p
// alone: only the entries that can hold the crossing are counted, the
// rest add their weight from the table. With top-k: every window entry is
// counted, the top-k threshold is the entry where the running count
// reaches top_k, and the nucleus, if any, is taken among the entries up
// to it. Returns false when the answer is not in the window (then the
// radix passes decide).
template <class D>
__device__ __forceinline__ bool window_select(const typename D::Elem *row, int64_t V, float m, float scale,
                              int fix_bits, float zlim, float tc_mass, bool k_on, int64_t top_k,
                              bool p_on, float top_p, float2 *out, NucleusShared &sh)
{
    const int tid = threadIdx.x;
    const float fscale = __uint_as_float((uint32_t)(127 + fix_bits) << 23);  // 2^fix_bits
    auto fixed = [&](float x) {
        return (unsigned long long)(exp2_fast((x - m) * scale) * fscale);
    };
    // In raw bits r, with magnitude u = r & 0x7fff and
    // d = max(u - kTinyBits + 1, 0), the window entry is A - d for a
    // positive and A + d for a negative value, A being the entry of the
    // tiny values (d = 0), all of it in 16-bit arithmetic: two elements per
    // 32-bit word.
    const uint32_t cm = compress_key(order_key<D>(m));
    const uint32_t A = cm - kTinyIdx;
    // Window entry of the lowest bf16 value at or below x (x rounded down
    // to bf16).
    auto entry_below = [&](float x) {
        const uint32_t bx = __float_as_uint(x);
        uint32_t r = bx >> 16;
        if ((bx & 0xffffu) && (bx & 0x80000000u))
            r += 1u;  // a truncated negative value: one step further down
        return cm - compress_key((r & 0x8000u) ? (~r & 0xffffu) : (r | 0x8000u));
    };
    // Entries from iz on hold values below m + (zlim - 2) / scale: they
    // weigh 0. Top-p alone: entries in [kWinKeys, iz) have mass but no
    // counter (summed one by one); with top-k they lie below every counted
    // entry and play no part.
    const uint32_t iz =
        __builtin_amdgcn_readfirstlane(entry_below(m + (zlim - 2.f) / scale) + 1u);
    const bool wide = !k_on && iz > (uint32_t)kWinKeys;
    // Top-p alone: entries from wc on hold values with (x - m) * scale < tc.
    // Together those weigh at most V * 2^tc = (1 - top_p) / 4 of the row, so
    // the crossing lies above them; and each weighs below 2^31 in fixed
    // point. They are not counted: their entries hold that weight instead,
    // which each element adds to the total. With top-k, wc = kWinKeys.
    const float tc = fminf(tc_mass, (float)(30 - fix_bits));
    const uint32_t wc = k_on ? (uint32_t)kWinKeys
                             : __builtin_amdgcn_readfirstlane(
                                   min(entry_below(m + tc / scale) + 1u, (uint32_t)kWinKeys));
    for (int q = tid; q <= kWinKeys; q += kNucThreads) {
        uint32_t v = 0;
        if ((uint32_t)q >= wc && q < kWinKeys && (uint32_t)q != A && (uint32_t)q <= cm)
            v = (uint32_t)fixed(key_value<D>(expand_key(cm - (uint32_t)q)));
        sh.cnt[q] = v;
    }
    __syncthreads();
    unsigned long long below = 0, tiny = 0;
    const u16x2 a2 = (u16x2)(unsigned short)A;
    const u16x2 w2 = (u16x2)(unsigned short)kWinKeys;
    const u16x2 wm2 = (u16x2)(unsigned short)(kWinKeys - 1);
    const u16x2 tb2 = (u16x2)(unsigned short)kTinyBits;
    const u16x2 tbm2 = (u16x2)(unsigned short)(kTinyBits - 1u);
    // Tiny values and values beyond the window with mass: one by one
    // (their entries, A and kWinKeys, hold no weight).
    auto rare = [&](uint32_t r, uint32_t idx) {
        const bool is_tiny = (r & 0x7fffu) < kTinyBits;
        const bool beyond = wide && idx >= (uint32_t)kWinKeys && idx < iz;
        const unsigned long long f = fixed(__uint_as_float(r << 16));
        tiny += is_tiny ? f : 0ull;
        below += !is_tiny && beyond ? f : 0ull;
    };
    auto visit_slot = [&](uint32_t slot) {
        const uint32_t v = sh.cnt[slot];
        if (slot < wc)
            atomicAdd(&sh.cnt[slot], 1u);
        below += slot < wc ? 0u : v;
    };
    // Eight elements (one 16-byte load): all window reads are issued before
    // the counts and the sums, so one wait covers them.
    auto visit_group = [&](const u32x4 &g) {
        const uint32_t w[4] = {g.x, g.y, g.z, g.w};
        uint32_t idx[4], slot[8];
        bool any_rare = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u16x2 u = as_u16x2(w[j] & 0x7fff7fffu);
            const u16x2 d = __builtin_bit_cast(
                u16x2, __builtin_elementwise_max(__builtin_bit_cast(i16x2, u - tbm2), (i16x2)0));
            const uint32_t neg = as_u32(__builtin_bit_cast(i16x2, w[j]) >> (i16x2)15);
            idx[j] = (as_u32(a2 + d) & neg) | (as_u32(a2 - d) & ~neg);
            const uint32_t s2 = as_u32(__builtin_elementwise_min(as_u16x2(idx[j]), w2));
            slot[2 * j] = s2 & 0xffffu;
            slot[2 * j + 1] = s2 >> 16;
            const bool has_tiny = as_u32(__builtin_elementwise_min(u, tb2)) != as_u32(tb2);
            const bool has_beyond =
                as_u32(__builtin_elementwise_min(as_u16x2(idx[j]), wm2)) != idx[j];
            any_rare |= has_tiny || (wide && has_beyond);
        }
        uint32_t v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            v[j] = sh.cnt[slot[j]];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (slot[j] < wc)
                atomicAdd(&sh.cnt[slot[j]], 1u);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            below += slot[j] < wc ? 0u : v[j];
        if (any_rare) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                rare(w[j] & 0xffffu, idx[j] & 0xffffu);
                rare(w[j] >> 16, idx[j] >> 16);
            }
        }
    };
    {
        const Span sp = make_span<D>(row, 0, V);
        const u32x4 *vrow = reinterpret_cast<const u32x4 *>(row + sp.a);
        for (int64_t base = 0; base < sp.ngroups; base += (int64_t)kNucThreads * kNucTiles) {
            u32x4 r[kNucTiles];
#pragma unroll
            for (int u = 0; u < kNucTiles; ++u) {
                const int64_t vi = base + u * kNucThreads + tid;
                r[u] = vi < sp.ngroups ? vrow[vi] : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < kNucTiles; ++u)
                if (base + u * kNucThreads + tid < sp.ngroups)
                    visit_group(r[u]);
        }
        auto visit_one = [&](uint32_t r) {
            const uint32_t u = r & 0x7fffu;
            const uint32_t d = u < kTinyBits ? 0u : u - (kTinyBits - 1u);
            const uint32_t idx = ((r & 0x8000u) ? A + d : A - d) & 0xffffu;
            visit_slot(min(idx, (uint32_t)kWinKeys));
            rare(r, idx);
        };
        if (sp.s + tid < sp.a)
            visit_one((uint32_t)row[sp.s + tid]);
        if (sp.z + tid < sp.e)
            visit_one((uint32_t)row[sp.z + tid]);
    }
    const uint64_t tiny_total = block_sum(tiny, sh);
    auto key_mass = [&](int idx) -> uint64_t {
        if ((uint32_t)idx == A)
            return tiny_total;
        const uint32_t n = (uint32_t)idx < wc ? sh.cnt[idx] : 0u;
        return n ? (uint64_t)n * fixed(key_value<D>(expand_key(cm - (uint32_t)idx))) : 0;
    };
    constexpr int kPer = kWinKeys / kNucThreads;
    uint64_t total, need;
    int last = kWinKeys - 1;  // the nucleus is taken among entries [0, last]
    if (k_on) {
        // The top-k threshold: the entry where the running count reaches
        // top_k (the count of the tiny entry is its number of tiny values).
        crossing(kWinKeys, (uint64_t)top_k, [&](int q) -> uint64_t { return sh.cnt[q]; }, sh);
        const int dk = sh.digit;
        if (dk < 0 || (uint32_t)dk == A)
            return false;  // fewer than top_k values in the window, or tiny
        last = dk;
        uint64_t mine = 0;
        for (int q = 0; q < kPer; ++q)
            mine += tid * kPer + q <= last ? key_mass(tid * kPer + q) : 0ull;
        total = block_sum(mine, sh);
        if (!p_on) {
            if (tid == 0)
                *out = make_float2(key_value<D>(expand_key(cm - (uint32_t)dk)),
                                   (float)total / fscale);
            return true;
        }
        need = mass_target(total, top_p);
    } else {
        uint64_t win = 0;
        for (int q = 0; q < kPer; ++q)
            win += key_mass(tid * kPer + q);
        if (tid == 0 && A >= (uint32_t)kWinKeys)
            win += tiny_total;  // the tiny entry lies beyond the window
        total = block_sum(win + below, sh);
        need = mass_target(total, top_p);
    }
    crossing(kWinKeys, need, [&](int q) -> uint64_t { return q <= last ? key_mass(q) : 0ull; },
             sh);
    const int d = sh.digit;
    if (d < 0 || (uint32_t)d == A)
        return false;  // among the tiny magnitudes or below the counted entries
    if (tid == 0) {
        const uint64_t kept = sh.above + key_mass(d);
        *out = make_float2(key_value<D>(expand_key(cm - (uint32_t)d)), (float)kept / fscale);
    }
    return true;
}

// One workgroup per row of every sampling sequence with a top-k or top-p
// filter. Top-k keeps whole levels from the top until they hold at least
// top_k tokens; the nucleus is the smallest run of keys from the top (of
// what top-k kept) whose fixed-point mass reaches ceil(top_p * total).
// Every mass is an integer sum, so the threshold and the kept mass do not
// depend on how the row is split or visited.
template <class D>
__global__ __launch_bounds__(kNucThreads, 6) void k_nucleus(Params p)
{
    using E = typename D::Elem;
    constexpr int KB = D::kKeyBits;
    __shared__ NucleusShared sh;
    const int k = p.k, nc = p.nc, rows = 2 * k + 1;
    const int64_t rb = blockIdx.x;
    const int slot = (int)(rb % rows);
    const int64_t b = rb / rows;
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
    // Elements with (x - m) * scale below this weigh 0 in fixed point.
    const float zlim = -(float)(p.fix_bits + 2);
    if (tid == 0) {
        const float2 *pp = p.partials + (b * rows + slot) * (int64_t)nc;
        float m = -INFINITY;  // the row max: the largest chunk max
        for (int c = 0; c < nc; ++c)
            m = fmaxf(m, pp[c].x);
        float z = 0.f;  // the row's mass relative to its max
        for (int c = 0; c < nc; ++c)
            z += pp[c].y * exp2_fast((pp[c].x - m) * scale);
        sh.rs = m;
        // (x - m) * scale < tc: together at most V * 2^tc = (1 - top_p) z / 4
        sh.tc = p_on ? fmaxf(zlim, __log2f((1.f - top_p) * z / (float)p.V) - 2.f) : zlim;
        sh.above = 0;
    }
    __syncthreads();
    const float m = sh.rs, tc = sh.tc;
    float2 *const out = p.nucleus + b * rows + slot;

    if constexpr (KB == 16) {
        if (window_select<D>(row, p.V, m, scale, p.fix_bits, zlim, tc, k_on, top_k, p_on, top_p,
                             out, sh))
            return;
        __syncthreads();  // the radix passes reuse the shared memory
    }
    uint32_t lo = 0;
    if (k_on) {
        const Selection sk = radix_select<D, true>(row, p.V, m, scale, fscale, zlim, 0u, top_k,
                                                   top_p, sh);
        if (!p_on) {
            if (tid == 0)
                *out = make_float2(key_value<D>(sk.key), (float)sk.kept / fscale);
            return;
        }
        lo = sk.key;
    }
    const Selection sp = radix_select<D, false>(row, p.V, m, scale, fscale, zlim, lo, 0, top_p, sh);
    if (tid == 0)
        *out = make_float2(key_value<D>(sp.key), (float)sp.kept / fscale);
}

template __global__ void k_nucleus<F32>(Params p);
template __global__ void k_nucleus<BF16>(Params p);

}  // namespace spv
