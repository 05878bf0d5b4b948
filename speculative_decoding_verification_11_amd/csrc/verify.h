// verify.h -- records and kernels shared by the verification sources
// (verify.hip: the step and the host side; nucleus.hip: top-k / top-p;
// early_exit.hip: the early-exit schedule). Internal to the library.
#pragma once

#include "common.h"

namespace spv {

// Workgroup of the nucleus search: eight waves share one row's table.
constexpr int kNucThreads = 512;



// ---------------------------------------------------------------------------
// Records handed from one workgroup to another inside one launch (the
// early-exit schedule). The writer stores them with agent-scope
// atomic stores and drains them (s_waitcnt) before the relaxed agent-scope
// counter add or flag store that announces them; the reader, once it has seen
// that count, loads them with agent-scope atomic loads. On gfx950 the
// compiler emits these stores and loads with the sc1 (device scope) bit: the
// store writes through the issuing XCD's L2 and has completed, at the
// device's coherence point, when its vmcnt is drained; the load is served
// from that coherence point, never from a line the reading XCD's L2 may still
// hold from an earlier call. Each access is 8 bytes, the widest atomic.
// Template argument C selects these accesses; without it, plain loads and
// stores (records that cross a launch boundary only).
// ---------------------------------------------------------------------------
__device__ inline void st_agent_u64(void *ptr, uint64_t v)
{
    __hip_atomic_store(static_cast<uint64_t *>(ptr), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t ld_agent_u64(const void *ptr)
{
    return __hip_atomic_load(static_cast<const uint64_t *>(ptr), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until every store this wave has issued has completed.
__device__ inline void drain_stores() { __builtin_amdgcn_s_waitcnt(0); }
__device__ inline int counter_add(int32_t *ptr, int32_t v)
{
    return __hip_atomic_fetch_add(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool C>
__device__ inline float2 ld_f2(const float2 *ptr)
{
    if constexpr (C) {
        const uint64_t v = ld_agent_u64(ptr);
        return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
    } else {
        return *ptr;
    }
}
template <bool C>
__device__ inline void st_f2(float2 *ptr, float2 v)
{
    if constexpr (C)
        st_agent_u64(ptr, (uint64_t)__float_as_uint(v.x) | ((uint64_t)__float_as_uint(v.y) << 32));
    else
        *ptr = v;
}
// ---------------------------------------------------------------------------
// Workspace records.
// ---------------------------------------------------------------------------
struct __align__(16) Decision {
    int32_t row;     // row of the final draw
    int32_t kind;    // SPEC_DRAW_*
    float v;         // draw uniform
    float scale;     // log2(e) / tau
    float mt, zt;    // target row: max logit, normaliser (kept mass under top-p)
    float md, zd;    // draft row (residual draws only)
    float tht, thd;  // top-p: smallest kept logit of the target / draft row (-inf: all)
    // A bonus draw on an unfiltered row is located to its chunk from the row
    // statistics (bonus_chunk); -1 otherwise (every chunk is summed).
    int32_t chunk;
    float mass;      // that chunk's weight
    double base;     // weight of the chunks before it
    double total;    // weight of the row: S of the draw
};

static_assert(sizeof(Decision) == 64, "decision record");

// ---------------------------------------------------------------------------
// The chunk of a bonus draw, from the row statistics alone. The draw weights
// of a bonus row are its softmax p, and the mass of chunk c is fixed by the
// chunk's partial (m_c, z_c) and the row's folded (m, z): z_c * 2^((m_c - m)
// * scale) / z. The chunk holding the draw is the first whose cumulative
// mass, summed in chunk order in fp64, exceeds v * S, S the sum of all of
// them. The draw then re-reads that chunk only and places the token inside it
// from its own weights, scaled to the chunk's mass.
// ---------------------------------------------------------------------------
__device__ inline float chunk_mass(float2 part, float m, float z, float scale)
{
#pragma clang fp contract(off)
    return part.y * exp2_fast((part.x - m) * scale) / z;
}

// One wave (`lane` in [0, 64)) locates the chunk; `part(c)` loads chunk c's
// partial. Lane c computes chunk c's mass (in batches of 64 chunks), and
// every lane sums the masses in chunk order from the shuffles, so every lane,
// and every caller, gets the same result. chunk = -1 if no chunk has mass
// (the draw then sums every chunk).
template <class F>
__device__ inline void bonus_chunk(int nc, float v, float m, float z, float scale, int lane,
                                   F part, int32_t &chunk, float &cmass, double &base,
                                   double &total)
{
    auto masses = [&](int c0) {  // lane's mass in the batch from c0
        const int c = c0 + lane;
        return c < nc ? chunk_mass(part(c), m, z, scale) : 0.f;
    };
    double S = 0.0;
    for (int c0 = 0; c0 < nc; c0 += kWave) {
        const float mc = masses(c0);
        const int n = min(kWave, nc - c0);
        for (int q = 0; q < n; ++q)
            S += (double)__shfl(mc, q, kWave);
    }
    const double t = (double)v * S;
    double run = 0.0, at = 0.0, last_at = 0.0;
    int cs = -1, last = -1;
    float mcs = 0.f, last_m = 0.f;
    for (int c0 = 0; c0 < nc && cs < 0; c0 += kWave) {
        const float mc = masses(c0);
        const int n = min(kWave, nc - c0);
        for (int q = 0; q < n; ++q) {
            const float mq = __shfl(mc, q, kWave);
            if (mq > 0.f) {
                last = c0 + q;
                last_m = mq;
                last_at = run;
            }
            if (run + (double)mq > t) {
                cs = c0 + q;
                mcs = mq;
                at = run;
                break;
            }
            run += (double)mq;
        }
    }
    if (cs < 0) {  // rounding left no crossing: the last chunk with mass
        cs = last;
        mcs = last_m;
        at = last_at;
    }
    chunk = cs;
    cmass = mcs;
    base = at;
    total = S;
}

__device__ inline Decision no_decision()
{
    Decision d;
    d.row = -1;
    d.kind = SPEC_DRAW_NONE;
    d.v = d.scale = d.mt = d.zt = d.md = d.zd = 0.f;
    d.tht = d.thd = -INFINITY;
    d.chunk = -1;
    d.mass = 0.f;
    d.base = d.total = 0.0;
    return d;
}

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
    float2 *partials;     // [B][2k+1][nc], written by k_rowstats
    Decision *decisions;  // [B], written by the decision (k_draw, or early exit)
    double2 *masses;      // [B][nc]: (sum w, sum p) per chunk of the draw row
    double *segs;         // [B][nc][2][kSegs]: segment sums of w, then of p
    const float *top_p;   // [B] or null: nucleus parameter per sequence
    const int32_t *top_k; // [B] or null: top-k parameter per sequence
    float4 *nucleus;      // [B][2k+1]: filtered rows (threshold logit, kept mass, row max, flag)
    int32_t fix_bits;     // top-p: fixed-point fraction bits of the row masses
    int32_t *ee_count;    // [k+2]: early exit: length of each position's list
    int32_t *ee_list;     // [k+1][B]: early exit: sequences to stream at each position
    int32_t *ee_done;     // [k+1][B]: early exit: chunks finished per position
    int32_t decide_in_draw;  // k_draw takes the decisions itself (small batches)
    int32_t skip_filtered;   // k_rowstats leaves the rows k_filter reads (bf16 filter calls)
    int32_t *out_tokens, *num_accepted;
    AuxDev aux;
};

// Whether sequence b's rows go through a top-k or top-p filter (for a
// sampling sequence whose inputs are valid): top_p below 1, or top_k
// strictly between 0 and V.
__device__ inline bool seq_filtered(const Params &p, int64_t b)
{
    return (p.top_p && p.top_p[b] < 1.f) ||
           (p.top_k && p.top_k[b] > 0 && p.top_k[b] < p.V);
}

// Kernels defined in the other sources. k_filter, k_filter_fallback: bf16
// rows only.
template <class D>
__global__ __launch_bounds__(kNucThreads, 6) void k_nucleus(Params p);
template <class D>
__global__ __launch_bounds__(kNucThreads, 6) void k_filter(Params p);
template <class D>
__global__ __launch_bounds__(kNucThreads, 6) void k_filter_fallback(Params p);
template <class D, int Per>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Per == 2 ? 5 : 1, 8))) void k_ee_rowstats0(Params p);
template <class D>
__global__ __launch_bounds__(kThreads) void k_ee_decide0(Params p);
template <class D, int Per>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Per == 2 ? 5 : 1, 8))) void k_ee_rowstats(Params p, int i);
template <class D, int Per>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Per == 2 ? 5 : 1, 8))) void k_ee_tail(Params p, int P);

}  // namespace spv
