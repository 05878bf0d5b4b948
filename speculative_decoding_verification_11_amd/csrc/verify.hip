// verify.hip -- HIP kernels and C ABI of the speculative-sampling
// verification step on MI355X (gfx950): spec_verify, spec_verify_top_p and
// spec_verify_early_exit.
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
// Three or four launches per call (top-p adds k_nucleus before k_draw),
// stream-ordered, no host synchronisation. Every hand-over between
// workgroups crosses a launch boundary, so no workgroup ever waits for
// another and nothing needs device-scope atomics:
//
//   k_rowstats  one workgroup per 32 KiB chunk of every logit row the step
//               needs (b-major). Each streams its chunk once with 16-byte
//               loads and stores an 8-byte partial: (max logit, sum
//               2^((x - max) * log2(e)/tau)) for sampling rows, (max logit,
//               lowest index of it) for greedy rows. This kernel carries
//               all of the algorithmic HBM traffic and runs at copy speed.
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
//               bonus) over its chunk in fp64, per segment and in all.
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

#include "common.h"

namespace {

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
    float2 *nucleus;      // [B][2k+1]: top-p (threshold logit, kept mass) per row
    int32_t fix_bits;     // top-p: fixed-point fraction bits of the row masses
    int32_t *ee_count;    // [k+2]: early exit: length of each position's list
    int32_t *ee_list;     // [k+1][B]: early exit: sequences to stream at each position
    int32_t *ee_done;     // [k+1][B]: early exit: chunks finished per position
    int32_t decide_in_draw;  // k_draw takes the decisions itself (small batches)
    int32_t *out_tokens, *num_accepted;
    AuxDev aux;
};

struct DrawShared {
    float tr[kWaves][2 * kTiles][kTrStride];  // per-lane group sums, transposed
    double seg[2][kSegs];                       // segment sums of w and p
};
struct LocateShared {
    double cm[kMaxLdsChunks];  // chunk masses (w, p) of one sequence
};

// ===========================================================================
// Decision of one sequence (one wave; `lane` in [0, 64)). Writes the
// accepted prefix, num_accepted, diagnostics and the decision record.
// ===========================================================================
template <class D>
__device__ __forceinline__ Decision decide(const Params &p, int64_t b, int lane, bool write)
{
    using E = typename D::Elem;
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
    } else if (p.top_p && !(p.top_p[b] > 0.f)) {
        status = SPEC_SEQ_BAD_TOP_P;
    } else {
        g = lane < L ? p.draft_tokens[b * k + lane] : -1;
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
                    t[q] = c0 + q < nc ? pp[c0 + q]
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
        if (write && lane <= k)
            out[lane] = lane < j ? g : (lane == j ? tok : -1);
        dec.row = j;
        dec.kind = SPEC_DRAW_GREEDY;
        if (write && lane == 0)
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
                    t[q] = c0 + q < nc ? pp[c0 + q] : make_float2(-INFINITY, 0.f);
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
                    t[q] = c0 + q < nc ? pp[c0 + q] : make_float2(-INFINITY, 0.f);
#pragma unroll
                for (int q = 0; q < kFoldBatch; ++q)
                    ds = soft_merge(ds, Soft{t[q].x, t[q].y}, scale);
            }
        }
        // Top-p: each row keeps its logits >= its threshold, normalised by
        // the kept mass (k_nucleus); otherwise the whole row and Z.
        float tz = ts.z, tth = -INFINITY, dz = ds.z, dth = -INFINITY;
        const bool filtered = (p.top_p && p.top_p[b] < 1.f) ||
                              (p.top_k && p.top_k[b] > 0 && p.top_k[b] < V);
        if (filtered) {
            if (lane <= L) {
                const float2 n = p.nucleus[b * rows + lane];
                tth = n.x;
                tz = n.y;
            }
            if (lane < L) {
                const float2 n = p.nucleus[b * rows + k + 1 + lane];
                dth = n.x;
                dz = n.y;
            }
        }
        if (lane < L) {
            const float xt = D::at(target + (b * (k + 1) + lane) * (int64_t)V, g);
            const float xd = D::at(draft + (b * k + lane) * (int64_t)V, g);
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
    const float et = exp2_fast((xt - dec.mt) * dec.scale) * inv_zt;
    const float pt = xt >= dec.tht ? et : 0.f;  // outside the target's nucleus: 0
    if (!resid)
        return {pt, pt};
    const float ed = exp2_fast((xd - dec.md) * dec.scale) * inv_zd;
    const float pd = xd >= dec.thd ? ed : 0.f;
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
        // kBatch 16-byte loads per row in flight before their arithmetic
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
                lt[u] = in ? stream_load(vt + gi) : u32x4{0u, 0u, 0u, 0u};
                ld[u] = in && r.resid ? stream_load(vd + gi) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                float ft[D::kVec], fd[D::kVec], w[D::kVec], pw[D::kVec];
                D::unpack(lt[u], ft);
                D::unpack(ld[u], fd);
#pragma unroll
                for (int j = 0; j < D::kVec; ++j) {
                    const Weights x = draw_weights(ft[j], fd[j], dec, r.inv_zt, r.inv_zd, r.resid);
                    w[j] = x.w;
                    pw[j] = x.p;
                }
                const bool in = (int64_t)(h + u) * kThreads + tid < sp.ngroups;
                gw[h + u] = in ? pairwise(w) : 0.f;
                gp[h + u] = in ? pairwise(pw) : 0.f;
            }
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
    const Decision dec = p.decisions[b];
    if (dec.kind != SPEC_DRAW_RESIDUAL && dec.kind != SPEC_DRAW_BONUS)
        return;  // greedy or error: the decision wrote everything
    const DrawRows<D> r = draw_rows<D>(p, b, dec);
    const double *mw = reinterpret_cast<const double *>(p.masses + b * (int64_t)nc);
    const bool staged = nc <= kMaxLdsChunks / 2;
    if (staged) {
        for (int q = lane; q < 2 * nc; q += kWave)
            sh.cm[q] = mw[q];
        __syncthreads();
    }

    // Chunk level (every lane runs the same scalar loop over LDS).
    auto mass = [&](int q) { return staged ? sh.cm[q] : mw[q]; };
    double Sw = 0.0, Sp = 0.0;
    for (int c = 0; c < nc; ++c) {
        Sw += mass(2 * c);
        Sp += mass(2 * c + 1);
    }
    int kind = dec.kind;
    bool use_p = !r.resid;
    if (r.resid && !(Sw > 0.0)) {  // residual mass rounded away: draw from p
        use_p = true;
        kind = SPEC_DRAW_RESIDUAL_AS_P;
    }
    const int sel = use_p ? 1 : 0;
    const double S = use_p ? Sp : Sw;
    const double t = (double)dec.v * S;
    double base = 0.0;
    int cs = -1;
    for (int c = 0; c < nc; ++c) {  // first chunk whose cumulative weight exceeds t
        const double m = mass(2 * c + sel);
        if (base + m > t) {
            cs = c;
            break;
        }
        base += m;
    }
    bool fallback = cs < 0;
    if (fallback) {  // no crossing: the last chunk with weight
        cs = nc - 1;
        for (int c = nc - 1; c >= 0; --c)
            if (mass(2 * c + sel) > 0.0) {
                cs = c;
                break;
            }
    }
    const int64_t s = (int64_t)cs * CH, e = min64((int64_t)p.V, s + CH);
    const Span sp = make_span2<D>(r.t, r.d, s, e);

    // Segment level: one segment sum per lane, scanned in order.
    const double *segs = p.segs + (b * (int64_t)nc + cs) * (2 * kSegs) + sel * kSegs;
    const double sv = lane < kSegs ? segs[lane] : 0.0;
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
            const Weights y = draw_weights(ft[j], fd[j], dec, r.inv_zt, r.inv_zd, r.resid);
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
        if (p.aux.resid_mass) p.aux.resid_mass[b] = (float)S;
        if (p.aux.draw_kind) p.aux.draw_kind[b] = kind;
    }
}

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

// Workgroup of the nucleus search: eight waves share one row's table.
constexpr int kNucThreads = 512;
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

// ===========================================================================
// The step.
// ===========================================================================
template <class D>
__global__ __launch_bounds__(kThreads) void k_rowstats(Params p)
{
    using E = typename D::Elem;
    constexpr int64_t CH = chunk_elems<D>();
    __shared__ RowShared sh;
    const int64_t item = blockIdx.x;
    const int k = p.k, nc = p.nc, rows = 2 * k + 1;

    const int c = (int)(item % nc);
    const int64_t rs = item / nc;
    const int slot = (int)(rs % rows);
    const int64_t b = rs / rows;
    const int L = p.draft_len ? p.draft_len[b] : k;
    const float tau = p.temperature[b];
    if (!valid_len(L, k) || !valid_temp(tau))
        return;  // the decision reports the sequence
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
    if (threadIdx.x == 0)
        p.partials[item] = part;
}

// One wave per sequence (large batches: see kFoldDecisionItems).
template <class D>
__global__ __launch_bounds__(kThreads) void k_decide(Params p)
{
    const int64_t b = (int64_t)blockIdx.x * kWaves + threadIdx.x / kWave;
    if (b < p.B)
        decide<D>(p, b, (int)(threadIdx.x % kWave), true);
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
            const Decision d = decide<D>(p, b, (int)threadIdx.x, c == 0);
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
    chunk_weight_sums<D>(p, b, c, dec, sh);
}

// One single-wave workgroup per sequence.
template <class D>
__global__ __launch_bounds__(kWave) void k_locate(Params p)
{
    __shared__ LocateShared sh;
    locate<D>(p, blockIdx.x, (int)threadIdx.x, sh);
}

// ===========================================================================
// Early-exit schedule. Rows after a sequence's first rejection never
// influence its outputs, so positions can be taken one at a time for the
// whole batch, each reading only the rows of the sequences still accepting.
// Decisions, draws and RNG are those of the full step; the diagnostics of
// rows that are never read (p_g, q_g, argmax past the stop) stay NaN / -1.
//
// Position 0 has its own decision launch (which also validates the inputs
// and clears the counters). From position 1 on, the workgroup that finishes
// the last chunk of a sequence's rows at position i takes that sequence's
// decision at once, and a sequence that accepts is appended to the list of
// position i + 1, so each position's launch only streams listed sequences.
// ===========================================================================

// Exchange of partials inside one launch: device-scope (write-through)
// stores and loads, and a writer drains its stores (s_waitcnt) before the
// relaxed device-scope count that tells the last workgroup to read them.
// Agent-scope release/acquire would write back / invalidate the whole L2 of
// the workgroup's XCD each time instead.
__device__ inline void publish_float2(float2 *ptr, float2 v)
{
    const uint64_t bits = (uint64_t)__float_as_uint(v.x) | ((uint64_t)__float_as_uint(v.y) << 32);
    __hip_atomic_store(reinterpret_cast<uint64_t *>(ptr), bits, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float2 fetch_float2(const float2 *ptr)
{
    const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t *>(ptr), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}
__device__ inline void drain_stores() { __builtin_amdgcn_s_waitcnt(0); }
__device__ inline int counter_add(int32_t *ptr, int32_t v)
{
    return __hip_atomic_fetch_add(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Row-statistics chunks of sequence b at position i.
__device__ inline int ee_items(int nc, bool greedy, int i, int L)
{
    return nc * (1 + (!greedy && i < L ? 1 : 0));
}

// Outputs of a sequence that stops at position j (one thread). The first
// pq_set entries of p_g / q_g and the first am_set of argmax were written
// position by position; the rest become NaN / -1. A draw's token is left
// to k_locate.
__device__ inline void ee_stop(const Params &p, int64_t b, int j, int status,
                               const Decision &dec, bool token_here, int token, int pq_set,
                               int am_set)
{
    const int k = p.k;
    int32_t *out = p.out_tokens + b * (k + 1);
    const bool ok = status == SPEC_SEQ_OK;
    for (int x = 0; x <= k; ++x) {
        if (!ok || x > j)
            out[x] = -1;
        else if (x < j)
            out[x] = p.draft_tokens[b * k + x];
        else if (token_here)
            out[x] = token;
    }
    p.num_accepted[b] = ok ? j : 0;
    const AuxDev &aux = p.aux;
    for (int x = ok ? pq_set : 0; x < k; ++x) {
        if (aux.p_g) aux.p_g[b * k + x] = NAN;
        if (aux.q_g) aux.q_g[b * k + x] = NAN;
    }
    if (aux.argmax)
        for (int x = ok ? am_set : 0; x <= k; ++x)
            aux.argmax[b * (k + 1) + x] = -1;
    if (aux.seq_status) aux.seq_status[b] = status;
    if (aux.draw_row) aux.draw_row[b] = ok ? j : -1;
    if (dec.kind != SPEC_DRAW_RESIDUAL && dec.kind != SPEC_DRAW_BONUS) {
        if (aux.draw_kind) aux.draw_kind[b] = dec.kind;
        if (aux.resid_mass) aux.resid_mass[b] = NAN;
    }
    p.decisions[b] = dec;
}

// Decision of sequence b at position i (one thread): the same folds (chunk
// order), gathers, Philox draws and tests as the full step's decision, for
// one position. Returns true when the sequence accepts g_i and goes on to
// position i + 1. `published`: the partials were written in this launch.
template <class D>
__device__ inline bool ee_decide(const Params &p, int64_t b, int i, int L, float tau,
                                 bool published)
{
    using E = typename D::Elem;
    const int k = p.k, V = p.V, nc = p.nc, rows = 2 * k + 1;
    Decision dec = no_decision();
    auto partial = [&](const float2 *q) { return published ? fetch_float2(q) : *q; };

    const E *target = static_cast<const E *>(p.target);
    const E *draft = static_cast<const E *>(p.draft);
    const float2 *pt = p.partials + (b * rows + i) * (int64_t)nc;
    const int g = i < L ? p.draft_tokens[b * k + i] : -1;
    if (tau == 0.f) {
        ArgMax acc{-INFINITY, INT32_MAX};
        for (int c = 0; c < nc; ++c) {
            const float2 t = partial(pt + c);
            acc = argmax_merge(acc, ArgMax{t.x, __float_as_int(t.y)});
        }
        if (p.aux.argmax) p.aux.argmax[b * (k + 1) + i] = acc.i;
        if (i < L && acc.i == g)
            return true;
        dec.row = i;
        dec.kind = SPEC_DRAW_GREEDY;
        ee_stop(p, b, i, SPEC_SEQ_OK, dec, true, acc.i, 0, i + 1);
        return false;
    }
    const float scale = temp_scale(tau);
    Soft ts{-INFINITY, 0.f}, ds{-INFINITY, 0.f};
    for (int c = 0; c < nc; ++c) {
        const float2 t = partial(pt + c);
        ts = soft_merge(ts, Soft{t.x, t.y}, scale);
    }
    const uint4 w = philox4x32_10(make_uint4((uint32_t)i, p.seq_base + (uint32_t)b, 0u, 0u),
                                  p.key0, p.key1);
    const float u = uniform24(w.x), v = uniform24(w.y);
    if (i < L) {
        const float2 *pd = p.partials + (b * rows + k + 1 + i) * (int64_t)nc;
        for (int c = 0; c < nc; ++c) {
            const float2 t = partial(pd + c);
            ds = soft_merge(ds, Soft{t.x, t.y}, scale);
        }
        const float xt = D::at(target + (b * (k + 1) + i) * (int64_t)V, g);
        const float xd = D::at(draft + (b * k + i) * (int64_t)V, g);
        const float pg = exp2_fast((xt - ts.m) * scale) / ts.z;
        const float qg = exp2_fast((xd - ds.m) * scale) / ds.z;
        if (!(qg > 0.f)) {
            ee_stop(p, b, i, SPEC_SEQ_QZERO, dec, false, 0, 0, 0);
            return false;
        }
        if (p.aux.p_g) p.aux.p_g[b * k + i] = pg;
        if (p.aux.q_g) p.aux.q_g[b * k + i] = qg;
        if (u < fminf(1.f, pg / qg))
            return true;
    }
    dec.row = i;
    dec.kind = i < L ? SPEC_DRAW_RESIDUAL : SPEC_DRAW_BONUS;
    dec.v = v;
    dec.scale = scale;
    dec.mt = ts.m;
    dec.zt = ts.z;
    dec.md = ds.m;
    dec.zd = ds.z;
    ee_stop(p, b, i, SPEC_SEQ_OK, dec, false, 0, i < L ? i + 1 : L, 0);
    return false;
}

// Streams one chunk of target row i (slot 0) or draft row i (slot 1) of
// sequence b; thread 0 returns the partial.
template <class D>
__device__ __forceinline__ float2 ee_chunk(const Params &p, int64_t b, int slot, int c, int i,
                                           float tau, RowShared &sh)
{
    using E = typename D::Elem;
    constexpr int64_t CH = chunk_elems<D>();
    const int k = p.k;
    const bool greedy = tau == 0.f;
    const E *row = slot == 0 ? static_cast<const E *>(p.target) + (b * (k + 1) + i) * (int64_t)p.V
                             : static_cast<const E *>(p.draft) + (b * k + i) * (int64_t)p.V;
    const int64_t s = (int64_t)c * CH;
    return chunk_stats<D>(row, s, min64((int64_t)p.V, s + CH), greedy,
                          greedy ? 0.f : temp_scale(tau), sh);
}

// Position 0: every sequence with a valid length and temperature.
template <class D>
__global__ __launch_bounds__(kThreads) void k_ee_rowstats0(Params p)
{
    __shared__ RowShared sh;
    const int64_t item = blockIdx.x;
    const int k = p.k, nc = p.nc, rows = 2 * k + 1;
    if (item == 0 && threadIdx.x == 0)
        p.ee_count[1] = 0;  // position 1's list, filled by k_ee_decide0
    const int c = (int)(item % nc);
    const int64_t rs = item / nc;
    const int slot = (int)(rs % 2);
    const int64_t b = rs / 2;
    const int L = p.draft_len ? p.draft_len[b] : k;
    const float tau = p.temperature[b];
    if (!(valid_len(L, k) && valid_temp(tau)))
        return;
    if (slot == 1 && (tau == 0.f || L == 0))
        return;
    const float2 part = ee_chunk<D>(p, b, slot, c, 0, tau, sh);
    if (threadIdx.x == 0)
        p.partials[(b * rows + (slot == 0 ? 0 : k + 1)) * (int64_t)nc + c] = part;
}

// Appends b to position i's list (one atomic per wave).
__device__ inline void ee_enlist(const Params &p, int64_t b, int i, bool go)
{
    const uint64_t mask = __ballot(go);
    if (!mask)
        return;
    const int lane = threadIdx.x & (kWave - 1);
    const int leader = __ffsll((unsigned long long)mask) - 1;
    int base = 0;
    if (lane == leader)
        base = counter_add(p.ee_count + i, __popcll(mask));
    base = __shfl(base, leader, kWave);
    if (go) {
        const int rank = __popcll(mask & ((1ull << lane) - 1));
        p.ee_list[(int64_t)i * p.B + base + rank] = (int32_t)b;
    }
}

// Position 0's decisions, one thread per sequence; also validates the
// inputs and clears the counters of the later positions.
template <class D>
__global__ __launch_bounds__(kThreads) void k_ee_decide0(Params p)
{
    const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const bool in = b < p.B;
    const int k = p.k, V = p.V;
    if (blockIdx.x == 0 && threadIdx.x > 1 && threadIdx.x <= k + 1)
        p.ee_count[threadIdx.x] = 0;  // positions 2..k (and k + 1, never read)
    bool go = false;
    if (in) {
        for (int i = 1; i <= k; ++i)
            p.ee_done[(int64_t)i * p.B + b] = 0;
        const int L = p.draft_len ? p.draft_len[b] : k;
        const float tau = p.temperature[b];
        int status = SPEC_SEQ_OK;
        if (!valid_len(L, k)) {
            status = SPEC_SEQ_BAD_LEN;
        } else if (!valid_temp(tau)) {
            status = SPEC_SEQ_BAD_TEMP;
        } else {
            for (int x = 0; x < L; ++x) {
                const int g = p.draft_tokens[b * k + x];
                if (g < 0 || g >= V)
                    status = SPEC_SEQ_BAD_TOKEN;
            }
        }
        if (status != SPEC_SEQ_OK) {
            const Decision dec = no_decision();
            ee_stop(p, b, 0, status, dec, false, 0, 0, 0);
        } else {
            go = ee_decide<D>(p, b, 0, L, tau, false);
        }
    }
    ee_enlist(p, b, 1, go);
}

// Position i >= 1: the sequences on position i's list. The workgroup that
// completes a sequence's chunks decides it and lists it for i + 1.
template <class D>
__global__ __launch_bounds__(kThreads) void k_ee_rowstats(Params p, int i)
{
    __shared__ RowShared sh;
    const int64_t item = blockIdx.x;
    const int k = p.k, nc = p.nc, rows = 2 * k + 1;
    const int64_t j = item / (2 * nc);
    if (j >= p.ee_count[i])
        return;
    const int slot = (int)((item / nc) % 2);
    const int c = (int)(item % nc);
    const int64_t b = p.ee_list[(int64_t)i * p.B + j];
    const int L = p.draft_len ? p.draft_len[b] : k;
    const float tau = p.temperature[b];
    if (slot == 1 && (tau == 0.f || i >= L))
        return;
    const float2 part = ee_chunk<D>(p, b, slot, c, i, tau, sh);
    if (threadIdx.x != 0)
        return;
    publish_float2(p.partials + (b * rows + (slot == 0 ? i : k + 1 + i)) * (int64_t)nc + c, part);
    drain_stores();  // the partial is visible before the count
    const int items = ee_items(nc, tau == 0.f, i, L);
    if (counter_add(p.ee_done + (int64_t)i * p.B + b, 1) != items - 1)
        return;
    if (ee_decide<D>(p, b, i, L, tau, true) && i < k) {
        const int at = counter_add(p.ee_count + i + 1, 1);
        p.ee_list[(int64_t)(i + 1) * p.B + at] = (int32_t)b;
    }
}

// Positions P..k in one launch: every remaining row (target rows P..L,
// draft rows P..L-1) of the sequences on position P's list. Once few
// sequences are left, a launch per position costs more than reading the
// rows after a stop that will never be used. The workgroup that completes
// a sequence's chunks decides its positions P, P+1, ... up to the stop.
template <class D>
__global__ __launch_bounds__(kThreads) void k_ee_tail(Params p, int P)
{
    __shared__ RowShared sh;
    const int64_t item = blockIdx.x;
    const int k = p.k, nc = p.nc, rows = 2 * k + 1;
    const int nt = k - P + 1, R = 2 * nt - 1;  // target rows P..k, draft rows P..k-1
    const int64_t j = item / ((int64_t)R * nc);
    if (j >= p.ee_count[P])
        return;
    const int rest = (int)(item % ((int64_t)R * nc));
    const int slot = rest / nc, c = rest % nc;
    const int64_t b = p.ee_list[(int64_t)P * p.B + j];
    const int L = p.draft_len ? p.draft_len[b] : k;
    const float tau = p.temperature[b];
    const bool greedy = tau == 0.f;
    const bool is_target = slot < nt;
    const int i = is_target ? P + slot : P + slot - nt;
    if (is_target ? i > L : (greedy || i >= L))
        return;
    const float2 part = ee_chunk<D>(p, b, is_target ? 0 : 1, c, i, tau, sh);
    if (threadIdx.x != 0)
        return;
    publish_float2(p.partials + (b * rows + (is_target ? i : k + 1 + i)) * (int64_t)nc + c, part);
    drain_stores();  // the partial is visible before the count
    int items = 0;
    for (int x = P; x <= L; ++x)
        items += ee_items(nc, greedy, x, L);
    if (counter_add(p.ee_done + (int64_t)P * p.B + b, 1) != items - 1)
        return;
    for (int x = P; x <= L; ++x)
        if (!ee_decide<D>(p, b, x, L, tau, true))
            break;
}

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
    lay->ee_count = lay->nucleus + align_up(nb * (size_t)(2 * k + 1) * sizeof(float2), 256);
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
        p.nucleus = reinterpret_cast<float2 *>(ws + lay.nucleus) + b0 * rows;
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

        // The events bracket the row statistics (and, for early exit, the
        // per-position decisions) of the first slice only.
        if (ev_begin && b0 == 0 && hipEventRecord(ev_begin, stream) != hipSuccess)
            return SPEC_ELAUNCH;
        if (!early_exit) {
            hipLaunchKernelGGL(k_rowstats<D>, dim3((unsigned)p.n_row_items), dim3(kThreads), 0,
                               stream, p);
            if (ev_end && b0 == 0 && hipEventRecord(ev_end, stream) != hipSuccess)
                return SPEC_ELAUNCH;
            if (p.top_p || p.top_k)
                hipLaunchKernelGGL(k_nucleus<D>, dim3((unsigned)(nb * rows)), dim3(kNucThreads), 0,
                                   stream, p);
            if (nb * nc <= kFoldDecisionItems)
                p.decide_in_draw = 1;
            else
                hipLaunchKernelGGL(k_decide<D>, dim3((unsigned)((nb + kWaves - 1) / kWaves)),
                                   dim3(kThreads), 0, stream, p);
        } else {
            hipLaunchKernelGGL(k_ee_rowstats0<D>, dim3((unsigned)(nb * 2 * nc)), dim3(kThreads),
                               0, stream, p);
            hipLaunchKernelGGL(k_ee_decide0<D>, dim3((unsigned)((nb + kThreads - 1) / kThreads)),
                               dim3(kThreads), 0, stream, p);
            const int P = std::min(k + 1, kEarlyExitSingle);
            for (int i = 1; i < P; ++i)
                hipLaunchKernelGGL(k_ee_rowstats<D>, dim3((unsigned)(nb * 2 * nc)),
                                   dim3(kThreads), 0, stream, p, i);
            if (P <= k)
                hipLaunchKernelGGL(k_ee_tail<D>,
                                   dim3((unsigned)(nb * (2 * (k - P + 1) - 1) * nc)),
                                   dim3(kThreads), 0, stream, p, P);
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


int verify_entry(const void *target_logits, const void *draft_logits, int32_t dtype,
                 const int32_t *draft_tokens, const int32_t *draft_len, const float *temperature,
                 const int32_t *top_k, const float *top_p, int32_t B, int32_t k, int32_t V,
                 uint64_t seed,
                 uint32_t seq_base, int32_t *out_tokens, int32_t *num_accepted,
                 const spec_verify_aux_t *aux, void *workspace, size_t workspace_bytes,
                 void *stream, bool early_exit)
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
    default: return "unknown status";
    }
}

extern "C" int spec_verify_version(void) { return kDeviceVersion; }
