// verify.hip -- HIP kernels and C ABI of the speculative-sampling
// verification step on MI355X (gfx950): spec_verify, spec_verify_top_p,
// spec_verify_top_k_top_p and spec_verify_early_exit. The top-k / top-p
// kernels (k_filter and k_filter_fallback for bf16 rows, k_nucleus for fp32
// rows) are in nucleus.hip, the early-exit kernels in early_exit.hip; all
// are launched from the host side here.
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
// Three or four launches per call (with a filter on bf16 logits, k_filter
// and k_filter_fallback come first; k_nucleus follows k_rowstats for fp32),
// stream-ordered, no host synchronisation. Every hand-over between
// workgroups crosses a launch boundary, so no workgroup ever waits for
// another and nothing needs device-scope atomics:
//
//   k_rowstats  one workgroup per 32 KiB chunk of every logit row the step
//               needs (b-major), or per two chunks of a row on grids of at
//               least kRowPairChunks chunks. Each streams its chunks once
//               with 16-byte loads and stores an 8-byte partial per chunk:
//               (max logit, sum 2^((x - max) * log2(e)/tau)) for sampling
//               rows, (max logit, lowest index of it) for greedy rows. This
//               kernel carries all of the algorithmic HBM traffic and runs
//               at copy speed. With a top-k or top-p filter on bf16 logits,
//               k_filter reads each filtered row once (counts, thresholds and
//               the row max; k_filter_fallback settles the rows it flags),
//               and k_rowstats, one workgroup per row, streams only the rows
//               without a filter.
//   k_decide    one wave per sequence: fold the partials in chunk order,
//               gather p_i(g_i) and q_i(g_i), draw Philox, run the
//               left-to-right test, write the accepted prefix, and record
//               the draw row j, its kind, the uniform v and the normalisers.
//               For batches whose draw grid is small (kFoldDecisionItems),
//               the first wave of every k_draw workgroup takes its sequence's
//               decision instead (all get the same; the first one writes it)
//               and this launch is skipped.
//   k_draw      one workgroup per chunk of each sequence's draw row: sums
//               of the draw weights w = max(0, p_j - q_j) (or p_L for a
//               bonus), scaled by the target row's normaliser, over its
//               chunk in fp64, per segment and in all. A
//               bonus draw on an unfiltered row reads only the chunk that
//               the decision located from the row statistics.
//   k_locate    one wave per sequence: the chunk where the cumulative weight
//               passes v * S, then the segment, the group and the element,
//               from those sums and one read of the group.
//
// k_draw re-reads the one or two draw rows of each sequence (about a fifth
// of the bytes k_rowstats reads). Doing those sums inside k_rowstats while
// the rows are still in the last-level cache was measured to cost more than
// re-reading them afterwards: the sums wait on decisions, and the waiting
// workgroups hold slots the streaming needs. Folding the locate into k_draw
// (last workgroup of a sequence) costs more than its own launch: its
// registers halve the occupancy of the latency-bound sums. The decision in
// k_draw costs each workgroup a few microseconds of one wave before its
// reads: worth a launch when the draw grid fits the chip about once, not
// when it takes several rounds.
//
// Nothing here is a dense contraction, so there is no MFMA: the step is bound
// by HBM bandwidth.
#include "verify.h"

#include <mutex>

namespace spv {

struct DrawShared {
    float tr[kWaves][2 * kTiles][kTrStride];  // per-lane group sums, transposed
    double seg[2][kSegs];                       // segment sums of w and p
};
struct LocateShared {
    double cm[kMaxLdsChunks];  // chunk masses (w, p) of one sequence
};

// Partial q of chunk batch c0 of a row (`pp`; `pre`: its first batch,
// loaded early), `pad` past the row's end.
template <bool Eager>
__device__ __forceinline__ float2 fold_part(const float2 *pp, const float2 (&pre)[kFoldBatch],
                                            int nc, int c0, int q, float2 pad)
{
    if constexpr (Eager) {
        if (c0 == 0)
            return q < nc ? pre[q] : pad;
    }
    return c0 + q < nc ? pp[c0 + q] : pad;
}

// ===========================================================================
// Decision of one sequence (one wave; `lane` in [0, 64)). Writes the
// accepted prefix, num_accepted, diagnostics and the decision record.
// Eager (the decision's own launch): the loads that do not depend on the
// draft length -- the drafted tokens (lane < k), the first kFoldBatch chunk
// partials of target row `lane` and draft row `lane`, and the two logits of
// each drafted token whose id is in range -- go out together with the
// length, so the decision waits on two memory round trips instead of four;
// a bonus draw's chunk takes the bonus row's partials from the lane that
// holds them. The values, and the order of every fold, are those of the
// plain form, which the draw kernel's workgroups use (there the extra
// registers would cost the draw sums their occupancy).
// ===========================================================================
template <class D, bool Eager>
__device__ __forceinline__ Decision decide(const Params &p, int64_t b, int lane, bool write)
{
    using E = typename D::Elem;
    const int k = p.k, V = p.V, nc = p.nc, rows = 2 * k + 1;
    const E *target = static_cast<const E *>(p.target);
    const E *draft = static_cast<const E *>(p.draft);
    const int L = p.draft_len ? p.draft_len[b] : k;
    const float tau = p.temperature[b];
    int32_t *out = p.out_tokens + b * (k + 1);

    // Eager loads (nothing here depends on L; every address is in range).
    float2 tpre[kFoldBatch], dpre[kFoldBatch];
    int gpre = -1;
    float xtpre = 0.f, xdpre = 0.f;
    if constexpr (Eager) {
        if (lane < k)
            gpre = p.draft_tokens[b * k + lane];
        const float2 *pt = p.partials + (b * rows + lane) * (int64_t)nc;
        const float2 *pd = p.partials + (b * rows + k + 1 + lane) * (int64_t)nc;
#pragma unroll
        for (int q = 0; q < kFoldBatch; ++q) {
            tpre[q] = lane <= k && q < nc ? pt[q] : make_float2(0.f, 0.f);
            dpre[q] = lane < k && q < nc ? pd[q] : make_float2(0.f, 0.f);
        }
        if (lane < k && gpre >= 0 && gpre < V) {
            xtpre = D::at(target + (b * (k + 1) + lane) * (int64_t)V, gpre);
            xdpre = D::at(draft + (b * k + lane) * (int64_t)V, gpre);
        }
    }

    int status = SPEC_SEQ_OK;
    int g = -1;
    if (!valid_len(L, k)) {
        status = SPEC_SEQ_BAD_LEN;
    } else if (!valid_temp(tau)) {
        status = SPEC_SEQ_BAD_TEMP;
    } else if (p.top_p && !(p.top_p[b] > 0.f)) {
        status = SPEC_SEQ_BAD_TOP_P;
    } else {
        g = lane < L ? (Eager ? gpre : p.draft_tokens[b * k + lane]) : -1;
        if (__any(lane < L && (g < 0 || g >= V)))
            status = SPEC_SEQ_BAD_TOKEN;
    }

    Decision dec = no_decision();
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
                    t[q] = Eager ? fold_part<Eager>(pp, tpre, nc, c0, q,
                                                    make_float2(-INFINITY,
                                                                __int_as_float(INT32_MAX)))
                                 : (c0 + q < nc ? pp[c0 + q]
                                                : make_float2(-INFINITY,
                                                              __int_as_float(INT32_MAX)));
#pragma unroll
                for (int q = 0; q < kFoldBatch; ++q)
                    acc = argmax_merge(acc, ArgMax{t[q].x, __float_as_int(t[q].y)});
            }
            amax = acc.i;
        }
        const uint64_t stop = __ballot(lane < L && amax != g);
        const int j = stop ? __ffsll((unsigned long long)stop) - 1 : L;
        const int tok = __shfl(amax, j, kWave);
        if (write && lane <= k)
            out[lane] = lane < j ? g : (lane == j ? tok : -1);
        dec.row = j;
        dec.kind = SPEC_DRAW_GREEDY;
        if (write && lane == 0)
            p.num_accepted[b] = j;
    } else if (status == SPEC_SEQ_OK) {
        const float scale = temp_scale(tau);
        Soft ts{-INFINITY, 0.f}, ds{-INFINITY, 0.f};
        // Top-k / top-p: each row keeps its logits >= its threshold,
        // normalised by the kept mass; the filter pass also gives the row
        // max. Otherwise: the whole row, max and Z folded from the partials.
        float tth = -INFINITY, dth = -INFINITY;
        if (seq_filtered(p, b)) {
            if (lane <= L) {
                const float4 n = p.nucleus[b * rows + lane];
                tth = n.x;
                ts = Soft{n.z, n.y};
            }
            if (lane < L) {
                const float4 n = p.nucleus[b * rows + k + 1 + lane];
                dth = n.x;
                ds = Soft{n.z, n.y};
            }
        } else {
            if (lane <= L) {
                const float2 *pp = p.partials + (b * rows + lane) * (int64_t)nc;
                for (int c0 = 0; c0 < nc; c0 += kFoldBatch) {
                    float2 t[kFoldBatch];
#pragma unroll
                    for (int q = 0; q < kFoldBatch; ++q)
                        t[q] = Eager ? fold_part<Eager>(pp, tpre, nc, c0, q,
                                                        make_float2(-INFINITY, 0.f))
                                     : (c0 + q < nc ? pp[c0 + q] : make_float2(-INFINITY, 0.f));
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
                        t[q] = Eager ? fold_part<Eager>(pp, dpre, nc, c0, q,
                                                        make_float2(-INFINITY, 0.f))
                                     : (c0 + q < nc ? pp[c0 + q] : make_float2(-INFINITY, 0.f));
#pragma unroll
                    for (int q = 0; q < kFoldBatch; ++q)
                        ds = soft_merge(ds, Soft{t[q].x, t[q].y}, scale);
                }
            }
        }
        const float tz = ts.z, dz = ds.z;
        if (lane < L) {
            const float xt = Eager ? xtpre : D::at(target + (b * (k + 1) + lane) * (int64_t)V, g);
            const float xd = Eager ? xdpre : D::at(draft + (b * k + lane) * (int64_t)V, g);
            pg = xt >= tth ? exp2_fast((xt - ts.m) * scale) / tz : 0.f;
            qg = xd >= dth ? exp2_fast((xd - ds.m) * scale) / dz : 0.f;
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
            if (write && lane <= k && lane != j)
                out[lane] = lane < j ? g : -1;  // position j: written by the locate
            dec.row = j;
            dec.kind = j < L ? SPEC_DRAW_RESIDUAL : SPEC_DRAW_BONUS;
            dec.v = __shfl(v, j, kWave);
            dec.scale = scale;
            dec.mt = __shfl(ts.m, j, kWave);
            dec.zt = __shfl(tz, j, kWave);
            dec.md = __shfl(ds.m, j, kWave);
            dec.zd = __shfl(dz, j, kWave);
            dec.tht = __shfl(tth, j, kWave);
            dec.thd = __shfl(dth, j, kWave);
            if (dec.kind == SPEC_DRAW_BONUS && !seq_filtered(p, b)) {
                // every lane reads the bonus row's partials and gets the same
                const float2 *pb = p.partials + (b * rows + j) * (int64_t)nc;
                if (Eager && nc <= kFoldBatch) {
                    // lane j holds them all: lane c takes chunk c's (bonus_chunk
                    // asks each lane for its own chunk, c == lane, when nc <= 64)
                    float2 mine = make_float2(0.f, 0.f);
#pragma unroll
                    for (int q = 0; q < kFoldBatch; ++q) {
                        const float2 v2 = make_float2(__shfl(tpre[q].x, j, kWave),
                                                      __shfl(tpre[q].y, j, kWave));
                        if (lane == q)
                            mine = v2;
                    }
                    bonus_chunk(nc, dec.v, dec.mt, dec.zt, scale, lane,
                                [&](int) { return mine; }, dec.chunk, dec.mass, dec.base,
                                dec.total);
                } else {
                    bonus_chunk(nc, dec.v, dec.mt, dec.zt, scale, lane,
                                [&](int c) { return pb[c]; }, dec.chunk, dec.mass, dec.base,
                                dec.total);
                }
            }
            if (write && lane == 0)
                p.num_accepted[b] = j;
        }
    }

    if (status != SPEC_SEQ_OK) {
        if (write && lane <= k)
            out[lane] = -1;
        if (write && lane == 0)
            p.num_accepted[b] = 0;
        dec.row = -1;
        dec.kind = SPEC_DRAW_NONE;
        pg = qg = NAN;
        amax = -1;
    }
    if (!write)
        return dec;
    const AuxDev &aux = p.aux;
    if (lane < k) {
        if (aux.p_g) aux.p_g[b * k + lane] = lane < L ? pg : NAN;
        if (aux.q_g) aux.q_g[b * k + lane] = lane < L ? qg : NAN;
    }
    if (aux.argmax && lane <= k)
        aux.argmax[b * (k + 1) + lane] = (lane <= L) ? amax : -1;
    if (lane == 0) {
        p.decisions[b] = dec;
        if (aux.seq_status) aux.seq_status[b] = status;
        if (aux.draw_row) aux.draw_row[b] = dec.row;
        // For a residual or bonus draw the locating workgroup of k_draw
        // writes draw_kind and resid_mass.
        if (dec.kind != SPEC_DRAW_RESIDUAL && dec.kind != SPEC_DRAW_BONUS) {
            if (aux.draw_kind) aux.draw_kind[b] = dec.kind;
            if (aux.resid_mass) aux.resid_mass[b] = NAN;
        }
    }
    return dec;
}

// Draw weight of one token, in units of the target row's normaliser z_t
// (the sums and the cut point v * S scale alike, so the token drawn is the
// same): w = z_t max(0, p - q) = max(0, e_t - e_d (z_t / z_d)) for a residual
// (e = 2^((x - m) * scale), the unnormalised softmax terms), e_t alone for a
// bonus, and z_t p = e_t itself (for the rounding fallback), in fp32. The
// difference is one fused multiply-add: e_t - e_d (z_t / z_d) exactly, then
// one rounding. Every reader of a weight goes through here, so all of them
// see bit-identical values.
struct Weights {
    float w, p;
};

//
// The specialised form below fixes, per workgroup, whether the draw is a
// residual (Resid) and whether a filter threshold applies (Thresh); with no
// filter the thresholds are -inf, which every finite logit passes, so both
// forms give the same bits. Contraction stays off in both, so that the only
// fused product is the explicit one, in both forms.
template <bool Resid, bool Thresh>
__device__ inline Weights draw_weights_t(float xt, float xd, const Decision &dec, float ratio)
{
#pragma clang fp contract(off)
    const float et = exp2_fast((xt - dec.mt) * dec.scale);
    const float pt = !Thresh || xt >= dec.tht ? et : 0.f;  // outside the target's nucleus: 0
    if constexpr (!Resid)
        return {pt, pt};
    const float ed = exp2_fast((xd - dec.md) * dec.scale);
    const float pd = !Thresh || xd >= dec.thd ? ed : 0.f;
    return {fmaxf(fmaf(-pd, ratio, pt), 0.f), pt};
}

__device__ inline Weights draw_weights(float xt, float xd, const Decision &dec, float ratio,
                                       bool resid)
{
    return resid ? draw_weights_t<true, true>(xt, xd, dec, ratio)
                 : draw_weights_t<false, true>(xt, xd, dec, ratio);
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
    float ratio;  // z_t / z_d (residual draws)
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
    r.ratio = r.resid ? dec.zt / dec.zd : 0.f;
    return r;
}

// Weight of element x (any alignment).
template <class D>
__device__ inline Weights elem_weight(const DrawRows<D> &r, int64_t x, const Decision &dec)
{
    return draw_weights(D::at(r.t, x), r.resid ? D::at(r.d, x) : 0.f, dec, r.ratio, r.resid);
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
        const Weights x = draw_weights(ft[j], r.resid ? fd[j] : 0.f, dec, r.ratio, r.resid);
        w[j] = x.w;
        pw[j] = x.p;
        if ((use_p ? x.p : x.w) > 0.f)
            last = (int)(sp.a + gi * D::kVec + j);
    }
    gw = pairwise(w);
    gp = pairwise(pw);
}

// Group sums of one chunk with 16-byte aligned groups, kTiles groups per
// lane: kBatch 16-byte loads per row in flight before their arithmetic.
// Full: the chunk is one whole block (kTiles groups for every lane), so no
// load is bounds-tested; a test per load costs each a branch around it.
template <class D, bool Resid, bool Thresh, bool Full>
__device__ __forceinline__ void vec_group_sums(const DrawRows<D> &r, const Span &sp,
                                               const Decision &dec, int tid, float (&gw)[kTiles],
                                               float (&gp)[kTiles])
{
    constexpr int kBatch = kTiles / 2;
    const u32x4 *vt = reinterpret_cast<const u32x4 *>(r.t + sp.a);
    const u32x4 *vd = reinterpret_cast<const u32x4 *>(r.d + sp.a);
#pragma unroll
    for (int h = 0; h < kTiles; h += kBatch) {
        u32x4 lt[kBatch], ld[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t gi = (int64_t)(h + u) * kThreads + tid;
            const bool in = Full || gi < sp.ngroups;
            lt[u] = in ? stream_load(vt + gi) : u32x4{0u, 0u, 0u, 0u};
            if constexpr (Resid)
                ld[u] = in ? stream_load(vd + gi) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            float ft[D::kVec], fd[D::kVec], w[D::kVec], pw[D::kVec];
            D::unpack(lt[u], ft);
            if constexpr (Resid)
                D::unpack(ld[u], fd);
#pragma unroll
            for (int j = 0; j < D::kVec; ++j) {
                const Weights x = draw_weights_t<Resid, Thresh>(ft[j], Resid ? fd[j] : 0.f, dec,
                                                                r.ratio);
                w[j] = x.w;
                pw[j] = x.p;
            }
            const bool in = Full || (int64_t)(h + u) * kThreads + tid < sp.ngroups;
            gp[h + u] = in ? pairwise(pw) : 0.f;
            gw[h + u] = Resid ? (in ? pairwise(w) : 0.f) : gp[h + u];  // a bonus draws from p
        }
    }
}

template <class D, bool Resid, bool Thresh>
__device__ __forceinline__ void vec_group_sums_of(bool full, const DrawRows<D> &r, const Span &sp,
                                                  const Decision &dec, int tid,
                                                  float (&gw)[kTiles], float (&gp)[kTiles])
{
    if (full)
        vec_group_sums<D, Resid, Thresh, true>(r, sp, dec, tid, gw, gp);
    else
        vec_group_sums<D, Resid, Thresh, false>(r, sp, dec, tid, gw, gp);
}

// ===========================================================================
// Sums of the draw weights over one chunk of the decided row: per segment
// (fp64 sums of the fp32 pairwise group sums) and over the chunk, for w and
// for p. The locate reads these instead of the chunk.
// ===========================================================================
template <class D>
__device__ __forceinline__ void chunk_weight_sums(const Params &p, int64_t b, int c,
                                                  const Decision &dec, DrawShared &sh)
{
    constexpr int64_t CH = chunk_elems<D>();
    const DrawRows<D> r = draw_rows<D>(p, b, dec);
    const int64_t s = (int64_t)c * CH, e = min64((int64_t)p.V, s + CH);
    const Span sp = make_span2<D>(r.t, r.d, s, e);
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    float gw[kTiles], gp[kTiles];  // this lane's group sums, tile by tile
    if (sp.vec) {
        // Uniform per workgroup: pick the loop without per-token tests, and
        // without per-load tests where the chunk is one whole block (every
        // chunk of a row but its last, on rows of 16-byte aligned length).
        const bool thresh = dec.tht != -INFINITY || (r.resid && dec.thd != -INFINITY);
        const bool full = sp.ngroups == (int64_t)kTiles * kThreads;
        if (r.resid) {
            if (thresh)
                vec_group_sums_of<D, true, true>(full, r, sp, dec, tid, gw, gp);
            else
                vec_group_sums_of<D, true, false>(full, r, sp, dec, tid, gw, gp);
        } else {
            if (thresh)
                vec_group_sums_of<D, false, true>(full, r, sp, dec, tid, gw, gp);
            else
                vec_group_sums_of<D, false, false>(full, r, sp, dec, tid, gw, gp);
        }
    } else {
        int unused = -1;
#pragma unroll
        for (int u = 0; u < kTiles; ++u) {
            const int64_t gi = (int64_t)u * kThreads + tid;
            gw[u] = gp[u] = 0.f;
            if (gi < sp.ngroups)
                group_weight_sums<D>(r, sp, gi, dec, false, gw[u], gp[u], unused);
        }
    }
    // Segment (tile u, this wave) = sum over the wave's 64 lanes. Transpose
    // through LDS: row q * kTiles + u holds the 64 lanes' values; four lanes
    // per row each add 16 of them (lane part, part + 4, ...), then combine.
    float (*tr)[kTrStride] = sh.tr[wave];
#pragma unroll
    for (int u = 0; u < kTiles; ++u) {
        tr[u][lane] = gw[u];
        tr[kTiles + u][lane] = gp[u];
    }
    __syncthreads();
    {
        const int row = lane >> 2, part = lane & 3;
        double acc = 0.0;
#pragma unroll
        for (int i = 0; i < kWave / 4; ++i)
            acc += (double)tr[row][part + 4 * i];
        acc += __shfl_xor(acc, 1, kWave);
        acc += __shfl_xor(acc, 2, kWave);
        if (part == 0)
            sh.seg[row / kTiles][1 + (row % kTiles) * kWaves + wave] = acc;
    }
    if (tid == 0) {  // head and tail: fewer than kVec elements each, in order
        double hw = 0.0, hp = 0.0, tw = 0.0, tp = 0.0;
        for (int64_t x = sp.s; x < sp.a; ++x) {
            const Weights y = elem_weight<D>(r, x, dec);
            hw += (double)y.w;
            hp += (double)y.p;
        }
        for (int64_t x = sp.z; x < sp.e; ++x) {
            const Weights y = elem_weight<D>(r, x, dec);
            tw += (double)y.w;
            tp += (double)y.p;
        }
        sh.seg[0][0] = hw;
        sh.seg[1][0] = hp;
        sh.seg[0][kSegs - 1] = tw;
        sh.seg[1][kSegs - 1] = tp;
    }
    __syncthreads();
    if (wave == 0) {
        const int64_t chunk = b * (int64_t)p.nc + c;
        double *dst = p.segs + chunk * (2 * kSegs);
        const double *src = &sh.seg[0][0];
        for (int q = lane; q < 2 * kSegs; q += kWave)
            dst[q] = src[q];
        const double mw = wave_sum(lane < kSegs ? sh.seg[0][lane] : 0.0);
        const double mp = wave_sum(lane < kSegs ? sh.seg[1][lane] : 0.0);
        if (lane == 0)
            p.masses[chunk] = make_double2(mw, mp);
    }
}

// Inclusive prefix sum over a wave (fixed order).
__device__ inline double wave_inclusive_scan(double v, int lane)
{
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const double o = __shfl_up(v, off, kWave);
        if (lane >= off)
            v += o;
    }
    return v;
}

// ===========================================================================
// Inverse-CDF locate of one sequence's correction / bonus token (one wave):
// the smallest token x whose cumulative weight exceeds t = v * S, found
// level by level -- the chunk (masses), the segment (segment sums), the
// group of kVec tokens (one 16-byte load per lane), the token. The sums at
// each level are those k_draw formed, so the levels agree up to fp64
// rounding of the order of summation; where rounding leaves no crossing at
// some level, the crossing is at the end of what that level covers, and the
// locate takes the last token with weight there (also the rule when t
// reaches S itself).
// ===========================================================================
template <class D>
__device__ __forceinline__ void locate(const Params &p, int64_t b, int lane, LocateShared &sh)
{
    constexpr int64_t CH = chunk_elems<D>();
    const int nc = p.nc;
    // The chunk masses are loaded with the decision, not after it: their
    // address does not depend on it (one round trip less).
    const double *mw = reinterpret_cast<const double *>(p.masses + b * (int64_t)nc);
    const bool staged = nc <= kMaxLdsChunks / 2;
    const Decision dec = p.decisions[b];
    if (staged) {
        for (int q = lane; q < 2 * nc; q += kWave)
            sh.cm[q] = mw[q];
        __syncthreads();
    }
    if (dec.kind != SPEC_DRAW_RESIDUAL && dec.kind != SPEC_DRAW_BONUS)
        return;  // greedy or error: the decision wrote everything
    const DrawRows<D> r = draw_rows<D>(p, b, dec);

    // Chunk level (every lane runs the same scalar loop over LDS).
    auto mass = [&](int q) { return staged ? sh.cm[q] : mw[q]; };
    int kind = dec.kind;
    bool use_p = !r.resid;
    double S, t, base = 0.0;
    int cs = -1;
    bool fallback = false;
    const bool located = dec.chunk >= 0;  // a bonus draw whose chunk the decision found
    if (located) {
        S = dec.total;
        t = (double)dec.v * S;
        cs = dec.chunk;
    } else {
        double Sw = 0.0, Sp = 0.0;
        for (int c = 0; c < nc; ++c) {
            Sw += mass(2 * c);
            Sp += mass(2 * c + 1);
        }
        if (r.resid && !(Sw > 0.0)) {  // residual mass rounded away: draw from p
            use_p = true;
            kind = SPEC_DRAW_RESIDUAL_AS_P;
        }
        S = use_p ? Sp : Sw;
        t = (double)dec.v * S;
        for (int c = 0; c < nc; ++c) {  // first chunk whose cumulative weight exceeds t
            const double m = mass(2 * c + (use_p ? 1 : 0));
            if (base + m > t) {
                cs = c;
                break;
            }
            base += m;
        }
        fallback = cs < 0;
        if (fallback) {  // no crossing: the last chunk with weight
            cs = nc - 1;
            for (int c = nc - 1; c >= 0; --c)
                if (mass(2 * c + (use_p ? 1 : 0)) > 0.0) {
                    cs = c;
                    break;
                }
        }
    }
    const int sel = use_p ? 1 : 0;
    const int64_t s = (int64_t)cs * CH, e = min64((int64_t)p.V, s + CH);
    const Span sp = make_span2<D>(r.t, r.d, s, e);

    // Segment level: one segment sum per lane, scanned in order.
    const double *segs = p.segs + (b * (int64_t)nc + cs) * (2 * kSegs) + sel * kSegs;
    const double sv = lane < kSegs ? segs[lane] : 0.0;
    if (located) {
        // the chunk's own weights, scaled to its mass from the row
        // statistics: the crossing inside it is at (t - base) / mass of them
        const double in = wave_sum(sv);
        t = (t - dec.base) * (in / (double)dec.mass);
        base = 0.0;
    }
    const double sincl = wave_inclusive_scan(sv, lane);
    int sg = -1;
    if (!fallback) {
        const uint64_t cross = __ballot(lane < kSegs && base + sincl > t);
        if (cross) {
            sg = __ffsll((unsigned long long)cross) - 1;
            base += __shfl(sincl - sv, sg, kWave);
        }
    }
    if (sg < 0) {  // no crossing: the last segment with weight
        fallback = true;
        const uint64_t pos = __ballot(lane < kSegs && sv > 0.0);
        sg = pos ? 63 - __clzll((long long)pos) : 0;
    }

    int tok = -1;
    if (sg == 0 || sg == kSegs - 1) {
        // head or tail: fewer than kVec tokens, walked in order by every lane
        const int64_t x0 = sg == 0 ? sp.s : sp.z, x1 = sg == 0 ? sp.a : sp.e;
        double run = base;
        int lastpos = -1;
        for (int64_t x = x0; x < x1; ++x) {
            const Weights y = elem_weight<D>(r, x, dec);
            const float wx = use_p ? y.p : y.w;
            run += (double)wx;
            if (wx > 0.f)
                lastpos = (int)x;
            if (!fallback && tok < 0 && run > t)
                tok = (int)x;
        }
        if (tok < 0)
            tok = lastpos;
    } else {
        // Segment (tile u, wave wv): lane l holds group u * 256 + wv * 64 + l.
        const int u = (sg - 1) / kWaves, wv = (sg - 1) % kWaves;
        const int64_t gi = (int64_t)u * kThreads + wv * kWave + lane;
        const bool in = gi < sp.ngroups;
        float ft[D::kVec], fd[D::kVec];
#pragma unroll
        for (int j = 0; j < D::kVec; ++j)
            ft[j] = fd[j] = 0.f;
        if (in) {
            load_group<D>(r.t, sp, gi, ft);
            if (r.resid)
                load_group<D>(r.d, sp, gi, fd);
        }
        float w[D::kVec];
#pragma unroll
        for (int j = 0; j < D::kVec; ++j) {
            const Weights y = draw_weights(ft[j], fd[j], dec, r.ratio, r.resid);
            w[j] = in ? (use_p ? y.p : y.w) : 0.f;
        }
        const float gsum = pairwise(w);
        const double gincl = wave_inclusive_scan((double)gsum, lane);
        int gl = -1;
        if (!fallback) {
            const uint64_t cross = __ballot(base + gincl > t);
            if (cross)
                gl = __ffsll((unsigned long long)cross) - 1;
        }
        if (gl < 0) {  // no crossing: the last group with weight
            fallback = true;
            const uint64_t pos = __ballot(gsum > 0.f);
            gl = pos ? 63 - __clzll((long long)pos) : 0;
        }
        // Lane gl walks its group in token order.
        int found = -1, lastpos = -1;
        double run = base + (gincl - (double)gsum);
#pragma unroll
        for (int j = 0; j < D::kVec; ++j) {
            run += (double)w[j];
            const int x = (int)(sp.a + gi * D::kVec + j);
            if (w[j] > 0.f)
                lastpos = x;
            if (!fallback && found < 0 && run > t)
                found = x;
        }
        tok = __shfl(found >= 0 ? found : lastpos, gl, kWave);
    }
    if (lane == 0) {
        p.out_tokens[b * (p.k + 1) + dec.row] = tok >= 0 ? tok : (int)s;
        // S of a located draw is the row statistics' (a probability mass);
        // otherwise it is the draw weights' sum, in units of z_t.
        if (p.aux.resid_mass) p.aux.resid_mass[b] = (float)(located ? S : S / (double)dec.zt);
        if (p.aux.draw_kind) p.aux.draw_kind[b] = kind;
    }
}

// ===========================================================================
// The step.
// ===========================================================================
// Two chunks of one row per workgroup (chunks 2j and 2j + 1): when both are
// single blocks, the second one's loads are issued before the first one is
// reduced, so the workgroup has a chunk in flight through each reduction and
// its barriers; and the workgroups of rows the step does not need, which
// only read the sequence's length and temperature, are half as many. Each
// chunk's partial is the one chunk_stats gives.

// Chunks consecutive chunks of one row per workgroup (Chunks == 0: the whole
// row). Where they are all single blocks, each chunk's values fold into the
// lane's (max, sum) or argmax, then the next chunk's loads go out, in flight
// through this chunk's reduction and its barriers; and the workgroups of
// rows the step does not need, which only read the sequence's length and
// temperature and leave, are fewer. Each chunk's partial is the one
// chunk_stats gives. Several chunks per workgroup are compiled for at least
// 5 waves per SIMD (96 VGPRs) for two chunks, written out; unbounded the
// compiler keeps both chunks' values live and runs 4. The whole-row loop is
// bounded at 4 (as a loop it spills at 5).
template <class D, int Chunks>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(Chunks == 1 ? 1 : (Chunks == 2 ? 5 : 4), 8))) void
k_rowstats(Params p)
{
    using E = typename D::Elem;
    constexpr int64_t CH = chunk_elems<D>();
    __shared__ RowShared sh;
    const uint32_t item = blockIdx.x;
    const int k = p.k, nc = p.nc, rows = 2 * k + 1;
    // 32-bit decode of the grid index (64-bit division is a long scalar
    // sequence every workgroup would run before its first load).
    const int per = Chunks == 0 ? nc : Chunks;
    const uint32_t np = (uint32_t)(nc + per - 1) / (uint32_t)per;
    const int c0 = per * (int)(item % np), cend = min(nc, c0 + per);
    const uint32_t rs = item / np;
    const int slot = (int)(rs % (uint32_t)rows);
    const int64_t b = rs / (uint32_t)rows;
    const int L = p.draft_len ? p.draft_len[b] : k;
    const float tau = p.temperature[b];
    // In a filtered call (whole rows; most workgroups leave here) the filter
    // parameters are loaded with the length, not after it.
    float top_p = 1.f;
    int32_t top_k = 0;
    if (Chunks == 0 && p.skip_filtered) {
        if (p.top_p)
            top_p = p.top_p[b];
        if (p.top_k)
            top_k = p.top_k[b];
    }
    if (!valid_len(L, k) || !valid_temp(tau))
        return;  // the decision reports the sequence
    const bool greedy = tau == 0.f;
    if (Chunks == 0 && p.skip_filtered && !greedy &&
        (top_p < 1.f || (top_k > 0 && top_k < p.V)))
        return;  // k_filter reads this sequence's rows (seq_filtered)
    const bool is_target = slot <= k;
    const int i = is_target ? slot : slot - (k + 1);
    if (is_target ? i > L : (greedy || i >= L))
        return;  // row not needed by this sequence: never read

    const E *row = is_target ? static_cast<const E *>(p.target) + (b * (k + 1) + i) * (int64_t)p.V
                             : static_cast<const E *>(p.draft) + (b * k + i) * (int64_t)p.V;
    const float scale = greedy ? 0.f : temp_scale(tau);
    const int tid = threadIdx.x;
    float2 *out = p.partials + (b * rows + slot) * (int64_t)nc;
    auto s_of = [&](int c) { return (int64_t)c * CH; };
    auto e_of = [&](int c) { return min64((int64_t)p.V, (int64_t)(c + 1) * CH); };
    const bool pipelined = Chunks != 1 && chunks_single_blocks<D>(row, p.V, nc, cend);
    if (pipelined && Chunks == 2) {
        chunk_pair_stats<D>(row, p.V, c0, cend, greedy, scale, sh, tid,
                            [&](int c, float2 v) { out[c] = v; });
        return;
    }
    if (pipelined) {
        u32x4 r[kTiles];
        load_single_block<D>(row, s_of(c0), e_of(c0), tid, r);
        for (int c = c0; c < cend; ++c) {
            Soft st{-INFINITY, 0.f};
            ArgMax am{-INFINITY, INT32_MAX};
            if (greedy)
                block_argmax<D>(am, r, (int32_t)(s_of(c) + tid * D::kVec));
            else
                block_soft<D>(st, r, scale);
            if (c + 1 < cend)
                load_single_block<D>(row, s_of(c + 1), e_of(c + 1), tid, r);
            const float2 v = greedy ? reduce_argmax(am, sh, tid) : reduce_soft(st, scale, sh, tid);
            if (tid == 0)
                out[c] = v;
        }
        return;
    }
    for (int c = c0; c < cend; ++c) {
        const float2 v = chunk_stats<D>(row, s_of(c), e_of(c), greedy, scale, sh);
        if (tid == 0)
            out[c] = v;
    }
}

// The early-exit schedule's row launches (positions 0..k) and position 0's
// decisions, with Per chunks per workgroup.
template <class D, int Per>
void early_exit_rows(const Params &p, int64_t nb, hipStream_t stream)
{
    const int k = p.k;
    const int64_t np = (p.nc + Per - 1) / Per;  // workgroups per row
    hipLaunchKernelGGL((k_ee_rowstats0<D, Per>), dim3((unsigned)(nb * 2 * np)), dim3(kThreads),
                       0, stream, p);
    hipLaunchKernelGGL(k_ee_decide0<D>, dim3((unsigned)((nb + kWaves - 1) / kWaves)),
                       dim3(kThreads), 0, stream, p);
    const int P = std::min(k + 1, kEarlyExitSingle);
    for (int i = 1; i < P; ++i)
        hipLaunchKernelGGL((k_ee_rowstats<D, Per>), dim3((unsigned)(nb * 2 * np)), dim3(kThreads),
                           0, stream, p, i);
    if (P <= k)
        hipLaunchKernelGGL((k_ee_tail<D, Per>), dim3((unsigned)(nb * (2 * (k - P + 1) - 1) * np)),
                           dim3(kThreads), 0, stream, p, P);
}

// One wave per sequence (large batches: see kFoldDecisionItems).
template <class D>
__global__ __launch_bounds__(kThreads) void k_decide(Params p)
{
    const int64_t b = (int64_t)blockIdx.x * kWaves + threadIdx.x / kWave;
    if (b < p.B)
        decide<D, true>(p, b, (int)(threadIdx.x % kWave), true);
}

// One workgroup per chunk of each sequence's draw row, sequences in reverse
// order: the rows k_rowstats read last may still be in the last-level cache.
template <class D>
__global__ __launch_bounds__(kThreads) void k_draw(Params p)
{
    __shared__ DrawShared sh;
    __shared__ Decision sdec;
    const int nc = p.nc;
    const int64_t b = (int64_t)p.B - 1 - (int64_t)(blockIdx.x / nc);
    const int c = (int)(blockIdx.x % nc);
    Decision dec;
    if (p.decide_in_draw) {
        // Every workgroup of the sequence takes its decision (the first one
        // also writes the prefix, the counts and the record for the locate).
        if (threadIdx.x < kWave) {
            const Decision d = decide<D, false>(p, b, (int)threadIdx.x, c == 0);
            if (threadIdx.x == 0)
                sdec = d;
        }
        __syncthreads();
        dec = sdec;
    } else {
        dec = p.decisions[b];  // uniform: one scalar load
    }
    if (dec.kind != SPEC_DRAW_RESIDUAL && dec.kind != SPEC_DRAW_BONUS)
        return;  // greedy or error: the decision wrote everything
    if (dec.chunk >= 0 && c != dec.chunk)
        return;  // a located bonus draw: only its chunk is read
    chunk_weight_sums<D>(p, b, c, dec, sh);
}

// One single-wave workgroup per sequence.
template <class D>
__global__ __launch_bounds__(kWave) void k_locate(Params p)
{
    __shared__ LocateShared sh;
    locate<D>(p, blockIdx.x, (int)threadIdx.x, sh);
}

}  // namespace spv

// ===========================================================================
// Allocation-free entry: the workspace is a file-scope device array, one
// copy per GPU, held until the process ends. Its name is a host-side stand-in
// for that memory; host code uses only the device address that
// hipGetSymbolAddress returns for it, looked up once per device with that
// device current. Nothing in the step needs the workspace cleared (every
// record is written before it is read within a call), so calls need no
// clearing launch; calls that overlap on one GPU share the array and race.
// ===========================================================================

static __device__ __align__(256) unsigned char scratch[SPEC_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace spv;

// ===========================================================================
// Host side.
// ===========================================================================
struct Layout {
    int nc;
    size_t partials, decisions, masses, segs, nucleus, ee_count, ee_list, ee_done, total;
};

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
    lay->segs = lay->masses + align_up(nb * (size_t)lay->nc * sizeof(double2), 256);
    lay->nucleus = lay->segs + align_up(nb * (size_t)lay->nc * 2 * kSegs * sizeof(double), 256);
    lay->ee_count = lay->nucleus + align_up(nb * (size_t)(2 * k + 1) * sizeof(float4), 256);
    lay->ee_list = lay->ee_count + align_up((size_t)(k + 2) * sizeof(int32_t), 256);
    lay->ee_done = lay->ee_list + align_up((size_t)(k + 1) * nb * sizeof(int32_t), 256);
    lay->total = lay->ee_done + align_up((size_t)(k + 1) * nb * sizeof(int32_t), 256);
    if (lay->total == 0)
        lay->total = 256;
    return true;
}

template <class D>
int launch_all(const Params &base, const spec_verify_aux_t *aux, const Layout &lay, char *ws,
               hipStream_t stream, bool early_exit)
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
        p.segs = reinterpret_cast<double *>(ws + lay.segs) + b0 * nc * 2 * kSegs;
        p.nucleus = reinterpret_cast<float4 *>(ws + lay.nucleus) + b0 * rows;
        if (p.top_p) p.top_p += b0;
        if (p.top_k) p.top_k += b0;
        // Early-exit lists and counters are per slice (indexed by the
        // slice's own B), so each slice uses the arrays from their start.
        p.ee_count = reinterpret_cast<int32_t *>(ws + lay.ee_count);
        p.ee_list = reinterpret_cast<int32_t *>(ws + lay.ee_list);
        p.ee_done = reinterpret_cast<int32_t *>(ws + lay.ee_done);
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

        // The events bracket the row pass (row statistics and filter pass;
        // for early exit, the per-position decisions) of the first slice.
        if (ev_begin && b0 == 0 && hipEventRecord(ev_begin, stream) != hipSuccess)
            return SPEC_ELAUNCH;
        if (!early_exit) {
            const bool filters = p.top_p || p.top_k;
            if (filters && D::kKeyBits == 16) {
                // k_filter reads every filtered row; k_rowstats the others
                // (greedy sequences, top_p >= 1 without top-k)
                hipLaunchKernelGGL(k_filter<D>, dim3((unsigned)(nb * rows)), dim3(kNucThreads),
                                   0, stream, p);
                // eight rows per workgroup (one wave reads each row's flag)
                constexpr int64_t fb_rows = kNucThreads / kWave;
                hipLaunchKernelGGL(k_filter_fallback<D>,
                                   dim3((unsigned)((nb * rows + fb_rows - 1) / fb_rows)),
                                   dim3(kNucThreads), 0, stream, p);
                // one workgroup per row: with every row filtered, all of
                // them leave at once, and there are few to dispatch
                p.skip_filtered = 1;
                hipLaunchKernelGGL((k_rowstats<D, 0>), dim3((unsigned)(nb * rows)),
                                   dim3(kThreads), 0, stream, p);
                p.skip_filtered = 0;
            } else {
                if (p.n_row_items >= kRowPairChunks)
                    hipLaunchKernelGGL((k_rowstats<D, 2>),
                                       dim3((unsigned)(nb * rows * (int64_t)((nc + 1) / 2))),
                                       dim3(kThreads), 0, stream, p);
                else
                    hipLaunchKernelGGL((k_rowstats<D, 1>), dim3((unsigned)p.n_row_items),
                                       dim3(kThreads), 0, stream, p);
                if (filters)
                    hipLaunchKernelGGL(k_nucleus<D>, dim3((unsigned)(nb * rows)),
                                       dim3(kNucThreads), 0, stream, p);
            }
            if (ev_end && b0 == 0 && hipEventRecord(ev_end, stream) != hipSuccess)
                return SPEC_ELAUNCH;
            if (nb * nc <= kFoldDecisionItems)
                p.decide_in_draw = 1;
            else
                hipLaunchKernelGGL(k_decide<D>, dim3((unsigned)((nb + kWaves - 1) / kWaves)),
                                   dim3(kThreads), 0, stream, p);
        } else {
            // Two chunks per workgroup on grids as large as k_rowstats
            // pairs them on (position 0's chunks: every target and draft row).
            if (nb * 2 * nc >= kRowPairChunks)
                early_exit_rows<D, 2>(p, nb, stream);
            else
                early_exit_rows<D, 1>(p, nb, stream);
            if (ev_end && b0 == 0 && hipEventRecord(ev_end, stream) != hipSuccess)
                return SPEC_ELAUNCH;
        }
        hipLaunchKernelGGL(k_draw<D>, dim3((unsigned)(nb * nc)), dim3(kThreads), 0, stream, p);
        hipLaunchKernelGGL(k_locate<D>, dim3((unsigned)nb), dim3(kWave), 0, stream, p);
        if (hipGetLastError() != hipSuccess)
            return SPEC_ELAUNCH;
    }
    return SPEC_OK;
}


constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices];  // this device's address of `scratch`, once known

// Device address of `scratch` on the device that owns `stream`.
int scratch_for_stream(hipStream_t stream, void **out)
{
    int cur = -1, dev = -1;
    if (hipGetDevice(&cur) != hipSuccess)
        return SPEC_ELAUNCH;
    if (stream) {
        if (hipStreamGetDevice(stream, &dev) != hipSuccess)
            return SPEC_EINVAL;
    } else {
        dev = cur;
    }
    if (dev < 0 || dev >= kMaxDevices)
        return SPEC_EINVAL;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess)
            return SPEC_ELAUNCH;
        void *p = nullptr;
        const hipError_t rc = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess)
            return SPEC_ELAUNCH;
        if (rc != hipSuccess || !p)
            return SPEC_ELAUNCH;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return SPEC_OK;
}

int verify_entry(const void *target_logits, const void *draft_logits, int32_t dtype,
                 const int32_t *draft_tokens, const int32_t *draft_len, const float *temperature,
                 const int32_t *top_k, const float *top_p, int32_t B, int32_t k, int32_t V,
                 uint64_t seed,
                 uint32_t seq_base, int32_t *out_tokens, int32_t *num_accepted,
                 const spec_verify_aux_t *aux, void *workspace, size_t workspace_bytes,
                 void *stream, bool early_exit, bool use_scratch = false)
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
        (draft_tokens && !aligned(draft_tokens, 4)) || (draft_len && !aligned(draft_len, 4)) ||
        !aligned(top_p, 4) || !aligned(top_k, 4))
        return SPEC_EINVAL;
    if (use_scratch) {
        // allocation-free entry: the static scratch, after every host check
        if (lay.total > (size_t)SPEC_NOALLOC_SCRATCH_BYTES)
            return SPEC_ESCRATCH;
        const int rc = scratch_for_stream(static_cast<hipStream_t>(stream), &workspace);
        if (rc != SPEC_OK)
            return rc;
        workspace_bytes = (size_t)SPEC_NOALLOC_SCRATCH_BYTES;
    }
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
    p.top_p = top_p;
    p.top_k = top_k;
    {
        // fixed-point masses of a row: V elements of at most 2^F each must
        // sum below 2^62
        int lv = 0;
        while (lv < 31 && (1ll << lv) < (int64_t)V)
            ++lv;
        p.fix_bits = std::min(40, 62 - lv);
    }
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
        return launch_all<F32>(p, aux, lay, ws, st, early_exit);
    return launch_all<BF16>(p, aux, lay, ws, st, early_exit);
}

}  // namespace

extern "C" int spec_verify(const void *target_logits, const void *draft_logits, int32_t dtype,
                           const int32_t *draft_tokens, const int32_t *draft_len,
                           const float *temperature, int32_t B, int32_t k, int32_t V,
                           uint64_t seed, uint32_t seq_base, int32_t *out_tokens,
                           int32_t *num_accepted, const spec_verify_aux_t *aux, void *workspace,
                           size_t workspace_bytes, void *stream)
{
    return verify_entry(target_logits, draft_logits, dtype, draft_tokens, draft_len, temperature,
                        nullptr, nullptr, B, k, V, seed, seq_base, out_tokens, num_accepted, aux,
                        workspace, workspace_bytes, stream, false);
}

extern "C" int spec_verify_top_p(const void *target_logits, const void *draft_logits,
                                 int32_t dtype, const int32_t *draft_tokens,
                                 const int32_t *draft_len, const float *temperature,
                                 const float *top_p, int32_t B, int32_t k, int32_t V,
                                 uint64_t seed, uint32_t seq_base, int32_t *out_tokens,
                                 int32_t *num_accepted, const spec_verify_aux_t *aux,
                                 void *workspace, size_t workspace_bytes, void *stream)
{
    if (!top_p && B > 0)
        return SPEC_EINVAL;
    return verify_entry(target_logits, draft_logits, dtype, draft_tokens, draft_len, temperature,
                        nullptr, top_p, B, k, V, seed, seq_base, out_tokens, num_accepted, aux,
                        workspace, workspace_bytes, stream, false);
}

extern "C" int spec_verify_top_k_top_p(const void *target_logits, const void *draft_logits,
                                       int32_t dtype, const int32_t *draft_tokens,
                                       const int32_t *draft_len, const float *temperature,
                                       const int32_t *top_k, const float *top_p, int32_t B,
                                       int32_t k, int32_t V, uint64_t seed, uint32_t seq_base,
                                       int32_t *out_tokens, int32_t *num_accepted,
                                       const spec_verify_aux_t *aux, void *workspace,
                                       size_t workspace_bytes, void *stream)
{
    if (!top_k && !top_p && B > 0)
        return SPEC_EINVAL;
    return verify_entry(target_logits, draft_logits, dtype, draft_tokens, draft_len, temperature,
                        top_k, top_p, B, k, V, seed, seq_base, out_tokens, num_accepted, aux,
                        workspace, workspace_bytes, stream, false);
}

extern "C" int spec_verify_early_exit(const void *target_logits, const void *draft_logits,
                                      int32_t dtype, const int32_t *draft_tokens,
                                      const int32_t *draft_len, const float *temperature,
                                      int32_t B, int32_t k, int32_t V, uint64_t seed,
                                      uint32_t seq_base, int32_t *out_tokens,
                                      int32_t *num_accepted, const spec_verify_aux_t *aux,
                                      void *workspace, size_t workspace_bytes, void *stream)
{
    return verify_entry(target_logits, draft_logits, dtype, draft_tokens, draft_len, temperature,
                        nullptr, nullptr, B, k, V, seed, seq_base, out_tokens, num_accepted, aux,
                        workspace, workspace_bytes, stream, true);
}

extern "C" int spec_verify_noalloc(const void *target_logits, const void *draft_logits,
                                   int32_t dtype, const int32_t *draft_tokens,
                                   const int32_t *draft_len, const float *temperature, int32_t B,
                                   int32_t k, int32_t V, uint64_t seed, uint32_t seq_base,
                                   int32_t *out_tokens, int32_t *num_accepted,
                                   const spec_verify_aux_t *aux, void *stream)
{
    return verify_entry(target_logits, draft_logits, dtype, draft_tokens, draft_len, temperature,
                        nullptr, nullptr, B, k, V, seed, seq_base, out_tokens, num_accepted, aux,
                        nullptr, 0, stream, false, true);
}

extern "C" size_t spec_verify_workspace_size(int32_t B, int32_t k, int32_t V, int32_t dtype)
{
    Layout lay;
    return layout_for(B, k, V, dtype, &lay) ? lay.total : 0;
}

extern "C" const char *spec_verify_strerror(int status)
{
    switch (status) {
    case SPEC_OK: return "success";
    case SPEC_EINVAL: return "invalid argument (null pointer, size, dtype or alignment)";
    case SPEC_EWORKSPACE: return "workspace null, misaligned or smaller than spec_verify_workspace_size()";
    case SPEC_ELAUNCH: return "kernel launch failed";
    case SPEC_ESCRATCH:
        return "sizes need more workspace than spec_verify_noalloc's static scratch "
               "(SPEC_NOALLOC_SCRATCH_BYTES); use spec_verify with a workspace";
    default: return "unknown status";
    }
}

extern "C" int spec_verify_version(void) { return kDeviceVersion; }
