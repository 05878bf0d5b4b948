// verify.h -- records and kernels shared by the verification sources
// (verify.hip: the step and the host side; nucleus.hip: top-k / top-p;
// early_exit.hip: the early-exit schedule). Internal to the library.
#pragma once

#include "common.h"

namespace spv {

// Workgroup of the nucleus search: eight waves share one row's table.
constexpr int kNucThreads = 512;


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
};

__device__ inline Decision no_decision()
{
    Decision d;
    d.row = -1;
    d.kind = SPEC_DRAW_NONE;
    d.v = d.scale = d.mt = d.zt = d.md = d.zd = 0.f;
    d.tht = d.thd = -INFINITY;
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
template <class D>
__global__ __launch_bounds__(kThreads) void k_ee_rowstats0(Params p);
template <class D>
__global__ __launch_bounds__(kThreads) void k_ee_decide0(Params p);
template <class D>
__global__ __launch_bounds__(kThreads) void k_ee_rowstats(Params p, int i);
template <class D>
__global__ __launch_bounds__(kThreads) void k_ee_tail(Params p, int P);

}  // namespace spv
