// early_exit.hip -- the early-exit schedule of the verification step on
// MI355X (gfx950): positions taken one at a time for the whole batch, so
// that rows after a sequence's first rejection are never read (kernels
// launched from verify.hip).
#include "verify.h"

namespace spv {

// ===========================================================================
// Early-exit schedule. Rows after a sequence's first rejection never
// influence its outputs, so positions can be taken one at a time for the
// whole batch, each reading only the rows of the sequences still accepting.
// Decisions, draws and RNG are those of the full step; the diagnostics of
// rows that are never read (p_g, q_g, argmax past the stop) stay NaN / -1.
//
// Position 0 has its own decision launch (one wave per sequence; it also
// validates the inputs and clears the counters). From position 1 on, the
// workgroup that finishes the last chunk of a sequence's rows at position i
// takes that sequence's decision at once (its first wave), and a sequence
// that accepts is appended to the list of position i + 1, so each
// position's launch only streams listed sequences.
// ===========================================================================

// Partials are exchanged inside one launch with the agent-coherent accesses
// of verify.h (st_f2<true> / ld_f2<true>, drain_stores, counter_add).
__device__ inline void publish_float2(float2 *ptr, float2 v) { st_f2<true>(ptr, v); }
__device__ inline float2 fetch_float2(const float2 *ptr) { return ld_f2<true>(ptr); }
#ifndef SPEC_EE_FORMAL
#define SPEC_EE_FORMAL 0
#endif
// Count of n published partials; returns the count before the add.
__device__ inline int count_published(int32_t *ctr, int n)
{
#if SPEC_EE_FORMAL
    const int before = __hip_atomic_fetch_add(ctr, n, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
#else
    drain_stores();  // the partials are visible before the count
    const int before = counter_add(ctr, n);
#endif
    return before;
}
// The last arriver, before it reads the others' partials.
__device__ inline void acquire_published()
{
#if SPEC_EE_FORMAL
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#endif
}

// Row-statistics chunks of sequence b at position i.
__device__ inline int ee_items(int nc, bool greedy, int i, int L)
{
    return nc * (1 + (!greedy && i < L ? 1 : 0));
}

// Outputs of a sequence that stops at position j, written by one wave
// (`lane` in [0, 64); k <= SPEC_MAX_K < 64, so lane x owns position x). The
// first pq_set entries of p_g / q_g and the first am_set of argmax were
// written position by position; the rest become NaN / -1. A draw's token is
// left to k_locate.
__device__ inline void ee_stop(const Params &p, int64_t b, int j, int status,
                               const Decision &dec, bool token_here, int token, int pq_set,
                               int am_set, int lane)
{
    const int k = p.k, x = lane;
    const bool ok = status == SPEC_SEQ_OK;
    if (x <= k) {
        int32_t *out = p.out_tokens + b * (k + 1);
        if (!ok || x > j)
            out[x] = -1;
        else if (x < j)
            out[x] = p.draft_tokens[b * k + x];
        else if (token_here)
            out[x] = token;
    }
    const AuxDev &aux = p.aux;
    if (x < k && x >= (ok ? pq_set : 0)) {
        if (aux.p_g) aux.p_g[b * k + x] = NAN;
        if (aux.q_g) aux.q_g[b * k + x] = NAN;
    }
    if (aux.argmax && x <= k && x >= (ok ? am_set : 0))
        aux.argmax[b * (k + 1) + x] = -1;
    if (lane != 0)
        return;
    p.num_accepted[b] = ok ? j : 0;
    if (aux.seq_status) aux.seq_status[b] = status;
    if (aux.draw_row) aux.draw_row[b] = ok ? j : -1;
    if (dec.kind != SPEC_DRAW_RESIDUAL && dec.kind != SPEC_DRAW_BONUS) {
        if (aux.draw_kind) aux.draw_kind[b] = dec.kind;
        if (aux.resid_mass) aux.resid_mass[b] = NAN;
    }
    p.decisions[b] = dec;
}

// Decision of sequence b at position i, by one wave (the result is the same
// in every lane): the same folds (chunk order), gathers, Philox draws and
// tests as the full step's decision, for one position. Lanes load the
// partials, and every lane folds them in chunk order, so the few memory
// round trips overlap. Returns true when the sequence accepts g_i and goes
// on to position i + 1. `published`: the partials were written in this
// launch.
template <class D>
__device__ inline bool ee_decide(const Params &p, int64_t b, int i, int L, float tau,
                                 bool published, int lane)
{
    using E = typename D::Elem;
    const int k = p.k, V = p.V, nc = p.nc, rows = 2 * k + 1;
    Decision dec = no_decision();
    auto partial = [&](const float2 *q) { return published ? fetch_float2(q) : *q; };

    const E *target = static_cast<const E *>(p.target);
    const E *draft = static_cast<const E *>(p.draft);
    const float2 *pt = p.partials + (b * rows + i) * (int64_t)nc;
    const float2 *pd = p.partials + (b * rows + k + 1 + i) * (int64_t)nc;
    const int g = i < L ? p.draft_tokens[b * k + i] : -1;
    if (tau == 0.f) {
        ArgMax acc{-INFINITY, INT32_MAX};
        for (int c0 = 0; c0 < nc; c0 += kWave) {
            const int c = c0 + lane, n = min(kWave, nc - c0);
            const float2 t =
                c < nc ? partial(pt + c) : make_float2(-INFINITY, __int_as_float(INT32_MAX));
            for (int q = 0; q < n; ++q)
                acc = argmax_merge(acc, ArgMax{__shfl(t.x, q, kWave),
                                               __float_as_int(__shfl(t.y, q, kWave))});
        }
        if (lane == 0 && p.aux.argmax)
            p.aux.argmax[b * (k + 1) + i] = acc.i;
        if (i < L && acc.i == g)
            return true;
        dec.row = i;
        dec.kind = SPEC_DRAW_GREEDY;
        ee_stop(p, b, i, SPEC_SEQ_OK, dec, true, acc.i, 0, i + 1, lane);
        return false;
    }
    const float scale = temp_scale(tau);
    const bool drafted = i < L;
    float xt = 0.f, xd = 0.f;  // the two logits of g, loaded with the partials
    if (drafted) {
        xt = D::at(target + (b * (k + 1) + i) * (int64_t)V, g);
        xd = D::at(draft + (b * k + i) * (int64_t)V, g);
    }
    Soft ts{-INFINITY, 0.f}, ds{-INFINITY, 0.f};
    for (int c0 = 0; c0 < nc; c0 += kWave) {
        const int c = c0 + lane, n = min(kWave, nc - c0);
        const float2 t = c < nc ? partial(pt + c) : make_float2(-INFINITY, 0.f);
        const float2 d = drafted && c < nc ? partial(pd + c) : make_float2(-INFINITY, 0.f);
        for (int q = 0; q < n; ++q) {
            ts = soft_merge(ts, Soft{__shfl(t.x, q, kWave), __shfl(t.y, q, kWave)}, scale);
            if (drafted)
                ds = soft_merge(ds, Soft{__shfl(d.x, q, kWave), __shfl(d.y, q, kWave)}, scale);
        }
    }
    const uint4 w = philox4x32_10(make_uint4((uint32_t)i, p.seq_base + (uint32_t)b, 0u, 0u),
                                  p.key0, p.key1);
    const float u = uniform24(w.x), v = uniform24(w.y);
    if (drafted) {
        const float pg = exp2_fast((xt - ts.m) * scale) / ts.z;
        const float qg = exp2_fast((xd - ds.m) * scale) / ds.z;
        if (!(qg > 0.f)) {
            ee_stop(p, b, i, SPEC_SEQ_QZERO, dec, false, 0, 0, 0, lane);
            return false;
        }
        if (lane == 0) {
            if (p.aux.p_g) p.aux.p_g[b * k + i] = pg;
            if (p.aux.q_g) p.aux.q_g[b * k + i] = qg;
        }
        if (u < fminf(1.f, pg / qg))
            return true;
    }
    dec.row = i;
    dec.kind = drafted ? SPEC_DRAW_RESIDUAL : SPEC_DRAW_BONUS;
    dec.v = v;
    dec.scale = scale;
    dec.mt = ts.m;
    dec.zt = ts.z;
    dec.md = ds.m;
    dec.zd = ds.z;
    if (!drafted)  // a bonus draw: its chunk from the row statistics, as in decide()
        bonus_chunk(nc, v, ts.m, ts.z, scale, lane, [&](int c) { return partial(pt + c); },
                    dec.chunk, dec.mass, dec.base, dec.total);
    ee_stop(p, b, i, SPEC_SEQ_OK, dec, false, 0, drafted ? i + 1 : L, 0, lane);
    return false;
}

// Decisions of sequence b at positions P..L at once, by one wave: lane x
// takes position x (its rows' partials folded in chunk order, its gathers
// and Philox draws, as ee_decide does for one position), and the first
// position that rejects (or the bonus at L) ends the round. Bit-identical
// to calling ee_decide for P, P + 1, ... until it stops, in one memory round
// trip for the partials instead of one per position. Requires P <= L.
template <class D>
__device__ inline void ee_decide_range(const Params &p, int64_t b, int P, int L, float tau,
                                       int lane)
{
    using E = typename D::Elem;
    const int k = p.k, V = p.V, nc = p.nc, rows = 2 * k + 1;
    const int x = lane;                       // this lane's position
    const bool mine = x >= P && x <= L;       // a position this call decides
    const bool drafted = mine && x < L;
    const int g = drafted ? p.draft_tokens[b * k + x] : -1;
    const float2 *pt = p.partials + (b * rows + (mine ? x : 0)) * (int64_t)nc;
    const float2 *pd = p.partials + (b * rows + k + 1 + (drafted ? x : 0)) * (int64_t)nc;
    Decision dec = no_decision();
    if (tau == 0.f) {
        ArgMax acc{-INFINITY, INT32_MAX};
        if (mine)
            for (int c = 0; c < nc; ++c) {
                const float2 t = fetch_float2(pt + c);
                acc = argmax_merge(acc, ArgMax{t.x, __float_as_int(t.y)});
            }
        const uint64_t stop = __ballot(mine && !(x < L && acc.i == g));
        const int j = __ffsll((unsigned long long)stop) - 1;  // L stops at the latest
        if (mine && x <= j && p.aux.argmax)
            p.aux.argmax[b * (k + 1) + x] = acc.i;
        dec.row = j;
        dec.kind = SPEC_DRAW_GREEDY;
        ee_stop(p, b, j, SPEC_SEQ_OK, dec, true, __shfl(acc.i, j, kWave), 0, j + 1, lane);
        return;
    }
    const float scale = temp_scale(tau);
    float xt = 0.f, xd = 0.f;
    if (drafted) {
        xt = D::at(static_cast<const E *>(p.target) + (b * (k + 1) + x) * (int64_t)V, g);
        xd = D::at(static_cast<const E *>(p.draft) + (b * k + x) * (int64_t)V, g);
    }
    Soft ts{-INFINITY, 0.f}, ds{-INFINITY, 0.f};
    if (mine)
        for (int c = 0; c < nc; ++c) {
            const float2 t = fetch_float2(pt + c);
            ts = soft_merge(ts, Soft{t.x, t.y}, scale);
            if (drafted) {
                const float2 d = fetch_float2(pd + c);
                ds = soft_merge(ds, Soft{d.x, d.y}, scale);
            }
        }
    const uint4 w = philox4x32_10(make_uint4((uint32_t)x, p.seq_base + (uint32_t)b, 0u, 0u),
                                  p.key0, p.key1);
    const float u = uniform24(w.x), v = uniform24(w.y);
    float pg = 0.f, qg = 0.f;
    if (drafted) {
        pg = exp2_fast((xt - ts.m) * scale) / ts.z;
        qg = exp2_fast((xd - ds.m) * scale) / ds.z;
    }
    const bool qzero = drafted && !(qg > 0.f);
    const bool reject = drafted && !qzero && !(u < fminf(1.f, pg / qg));
    const uint64_t stop = __ballot(mine && (qzero || reject || x == L));
    const int j = __ffsll((unsigned long long)stop) - 1;
    if (__shfl((int)qzero, j, kWave)) {
        ee_stop(p, b, j, SPEC_SEQ_QZERO, dec, false, 0, 0, 0, lane);
        return;
    }
    if (drafted && x <= j) {  // the accepted positions and the one that rejects
        if (p.aux.p_g) p.aux.p_g[b * k + x] = pg;
        if (p.aux.q_g) p.aux.q_g[b * k + x] = qg;
    }
    const bool bonus = j == L;
    dec.row = j;
    dec.kind = bonus ? SPEC_DRAW_BONUS : SPEC_DRAW_RESIDUAL;
    dec.v = __shfl(v, j, kWave);
    dec.scale = scale;
    dec.mt = __shfl(ts.m, j, kWave);
    dec.zt = __shfl(ts.z, j, kWave);
    dec.md = __shfl(ds.m, j, kWave);
    dec.zd = __shfl(ds.z, j, kWave);
    if (bonus) {  // its chunk from the row statistics, as in decide()
        const float2 *pj = p.partials + (b * rows + j) * (int64_t)nc;
        bonus_chunk(nc, dec.v, dec.mt, dec.zt, scale, lane,
                    [&](int c) { return fetch_float2(pj + c); }, dec.chunk, dec.mass, dec.base,
                    dec.total);
    }
    ee_stop(p, b, j, SPEC_SEQ_OK, dec, false, 0, bonus ? L : j + 1, 0, lane);
}

// Chunk c0 (Per == 1), or chunks c0 and c0 + 1 (Per == 2; the second where
// c0 + 1 < nc), of target row i (slot 0) or draft row i (slot 1) of sequence
// b, as in k_rowstats: where both of a pair are single blocks, the second
// one's loads are in flight through the first one's reduction. emit(c,
// partial) runs in thread 0, in chunk order; returns the number of chunks
// streamed.
template <class D, int Per, class Emit>
__device__ __forceinline__ int ee_chunks(const Params &p, int64_t b, int slot, int c0, int i,
                                         float tau, RowShared &sh, Emit emit)
{
    using E = typename D::Elem;
    constexpr int64_t CH = chunk_elems<D>();
    const int k = p.k, nc = p.nc;
    const int64_t V = p.V;
    const bool greedy = tau == 0.f;
    const float scale = greedy ? 0.f : temp_scale(tau);
    const E *row = slot == 0 ? static_cast<const E *>(p.target) + (b * (k + 1) + i) * V
                             : static_cast<const E *>(p.draft) + (b * k + i) * V;
    const int cend = min(nc, c0 + Per);
    if (Per == 2 && chunks_single_blocks<D>(row, V, nc, cend)) {
        chunk_pair_stats<D>(row, V, c0, cend, greedy, scale, sh, (int)threadIdx.x, emit);
    } else {
        for (int c = c0; c < cend; ++c) {
            const int64_t s = (int64_t)c * CH;
            const float2 v = chunk_stats<D>(row, s, min64(V, s + CH), greedy, scale, sh);
            if (threadIdx.x == 0)
                emit(c, v);
        }
    }
    return cend - c0;
}

// Workgroups per row: one per Per chunks.
template <int Per>
__device__ inline int ee_groups(int nc)
{
    return (nc + Per - 1) / Per;
}

// Position 0: every sequence with a valid length and temperature, one
// workgroup per Per chunks of its target and draft row. Pairs of chunks are
// compiled for at least 5 waves per SIMD (96 VGPRs), as in k_rowstats.
template <class D, int Per>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Per == 2 ? 5 : 1, 8))) void
k_ee_rowstats0(Params p)
{
    __shared__ RowShared sh;
    const uint32_t item = blockIdx.x;
    const int k = p.k, nc = p.nc, rows = 2 * k + 1;
    if (item == 0 && threadIdx.x == 0)
        p.ee_count[1] = 0;  // position 1's list, filled by k_ee_decide0
    // 32-bit decode of the grid index (64-bit division is a long scalar
    // sequence every workgroup would run before its first load).
    const uint32_t np = (uint32_t)ee_groups<Per>(nc);
    const int c0 = Per * (int)(item % np);
    const uint32_t rs = item / np;
    const int slot = (int)(rs % 2u);
    const int64_t b = rs / 2u;
    const int L = p.draft_len ? p.draft_len[b] : k;
    const float tau = p.temperature[b];
    if (!(valid_len(L, k) && valid_temp(tau)))
        return;
    if (slot == 1 && (tau == 0.f || L == 0))
        return;
    float2 *out = p.partials + (b * rows + (slot == 0 ? 0 : k + 1)) * (int64_t)nc;
    ee_chunks<D, Per>(p, b, slot, c0, 0, tau, sh, [&](int c, float2 v) { out[c] = v; });
}

// Appends b to position i's list (lane 0 of the deciding wave).
__device__ inline void ee_enlist(const Params &p, int64_t b, int i)
{
    const int at = counter_add(p.ee_count + i, 1);
    p.ee_list[(int64_t)i * p.B + at] = (int32_t)b;
}

// Position 0's decisions, one wave per sequence; also validates the inputs
// and clears the counters of the later positions. The sequences that accept
// are listed for position 1 with one counter add per workgroup (one per
// sequence would queue up to B device-scope adds on one address).
template <class D>
__global__ __launch_bounds__(kThreads) void k_ee_decide0(Params p)
{
    __shared__ int accepted[kWaves];
    __shared__ int list_at;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int64_t b = (int64_t)blockIdx.x * kWaves + wave;
    const int k = p.k, V = p.V;
    if (blockIdx.x == 0 && threadIdx.x > 1 && threadIdx.x <= k + 1)
        p.ee_count[threadIdx.x] = 0;  // positions 2..k (and k + 1, never read)
    bool accept = false;
    if (b < p.B) {  // no early return: every wave reaches the barriers below
        if (lane >= 1 && lane <= k)
            p.ee_done[(int64_t)lane * p.B + b] = 0;
        const int L = p.draft_len ? p.draft_len[b] : k;
        const float tau = p.temperature[b];
        int status = SPEC_SEQ_OK;
        if (!valid_len(L, k)) {
            status = SPEC_SEQ_BAD_LEN;
        } else if (!valid_temp(tau)) {
            status = SPEC_SEQ_BAD_TEMP;
        } else {
            const int g = lane < L ? p.draft_tokens[b * k + lane] : 0;
            if (__any(lane < L && (g < 0 || g >= V)))
                status = SPEC_SEQ_BAD_TOKEN;
        }
        if (status != SPEC_SEQ_OK)
            ee_stop(p, b, 0, status, no_decision(), false, 0, 0, 0, lane);
        else
            accept = ee_decide<D>(p, b, 0, L, tau, false, lane);
    }
    if (lane == 0)
        accepted[wave] = accept ? 1 : 0;
    __syncthreads();
    if (threadIdx.x == 0) {
        int n = 0;
        for (int w = 0; w < kWaves; ++w)
            n += accepted[w];
        list_at = n ? counter_add(p.ee_count + 1, n) : 0;
    }
    __syncthreads();
    if (lane == 0 && accept) {
        int at = list_at;
        for (int w = 0; w < wave; ++w)
            at += accepted[w];
        p.ee_list[p.B + at] = (int32_t)b;  // position 1's list
    }
}

// Position i >= 1: the sequences on position i's list, one workgroup per
// Per chunks. The workgroup that completes a sequence's chunks decides it
// and lists it for i + 1.
template <class D, int Per>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Per == 2 ? 5 : 1, 8))) void
k_ee_rowstats(Params p, int i)
{
    __shared__ RowShared sh;
    const uint32_t item = blockIdx.x;  // 32-bit decode, as in k_ee_rowstats0
    const int k = p.k, nc = p.nc, rows = 2 * k + 1;
    const uint32_t np = (uint32_t)ee_groups<Per>(nc);
    const int64_t j = item / (2u * np);
    if (j >= p.ee_count[i])
        return;
    const int slot = (int)((item / np) % 2u);
    const int c0 = Per * (int)(item % np);
    const int64_t b = p.ee_list[(int64_t)i * p.B + j];
    const int L = p.draft_len ? p.draft_len[b] : k;
    const float tau = p.temperature[b];
    if (slot == 1 && (tau == 0.f || i >= L))
        return;
    float2 *out = p.partials + (b * rows + (slot == 0 ? i : k + 1 + i)) * (int64_t)nc;
    const int n = ee_chunks<D, Per>(p, b, slot, c0, i, tau, sh,
                                    [&](int c, float2 v) { publish_float2(out + c, v); });
    if (threadIdx.x >= kWave)
        return;
    const int lane = threadIdx.x;
    int last = 0;
    if (lane == 0) {
        const int items = ee_items(nc, tau == 0.f, i, L);
        last = count_published(p.ee_done + (int64_t)i * p.B + b, n) + n == items;
    }
    if (!__shfl(last, 0, kWave))
        return;
    acquire_published();
    // The last chunk of the sequence's rows: the first wave decides.
    if (ee_decide<D>(p, b, i, L, tau, true, lane) && i < k && lane == 0)
        ee_enlist(p, b, i + 1);
}

// Positions P..k in one launch: every remaining row (target rows P..L,
// draft rows P..L-1) of the sequences on position P's list, one workgroup
// per Per chunks. Once few sequences are left, a launch per position costs
// more than reading the rows after a stop that will never be used. The
// workgroup that completes a sequence's chunks decides its positions P,
// P+1, ... up to the stop.
template <class D, int Per>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Per == 2 ? 5 : 1, 8))) void
k_ee_tail(Params p, int P)
{
    __shared__ RowShared sh;
    const uint32_t item = blockIdx.x;  // 32-bit decode, as in k_ee_rowstats0
    const int k = p.k, nc = p.nc, rows = 2 * k + 1;
    const int nt = k - P + 1, R = 2 * nt - 1;  // target rows P..k, draft rows P..k-1
    const uint32_t np = (uint32_t)ee_groups<Per>(nc);
    const uint32_t per_seq = (uint32_t)R * np;
    const int64_t j = item / per_seq;
    if (j >= p.ee_count[P])
        return;
    const uint32_t rest = item % per_seq;
    const int slot = (int)(rest / np), c0 = Per * (int)(rest % np);
    const int64_t b = p.ee_list[(int64_t)P * p.B + j];
    const int L = p.draft_len ? p.draft_len[b] : k;
    const float tau = p.temperature[b];
    const bool greedy = tau == 0.f;
    const bool is_target = slot < nt;
    const int i = is_target ? P + slot : P + slot - nt;
    if (is_target ? i > L : (greedy || i >= L))
        return;
    float2 *out = p.partials + (b * rows + (is_target ? i : k + 1 + i)) * (int64_t)nc;
    const int n = ee_chunks<D, Per>(p, b, is_target ? 0 : 1, c0, i, tau, sh,
                                    [&](int c, float2 v) { publish_float2(out + c, v); });
    if (threadIdx.x >= kWave)
        return;
    const int lane = threadIdx.x;
    int last = 0;
    if (lane == 0) {
        int items = 0;
        for (int x = P; x <= L; ++x)
            items += ee_items(nc, greedy, x, L);
        last = count_published(p.ee_done + (int64_t)P * p.B + b, n) + n == items;
    }
    if (!__shfl(last, 0, kWave))
        return;
    acquire_published();
    // The last chunk of the sequence's rows: the first wave decides
    // positions P, P + 1, ... up to the stop, all at once.
    ee_decide_range<D>(p, b, P, L, tau, lane);
}

template __global__ void k_ee_rowstats0<F32, 1>(Params p);
template __global__ void k_ee_rowstats0<F32, 2>(Params p);
template __global__ void k_ee_rowstats0<BF16, 1>(Params p);
template __global__ void k_ee_rowstats0<BF16, 2>(Params p);
template __global__ void k_ee_decide0<F32>(Params p);
template __global__ void k_ee_decide0<BF16>(Params p);
template __global__ void k_ee_rowstats<F32, 1>(Params p, int i);
template __global__ void k_ee_rowstats<F32, 2>(Params p, int i);
template __global__ void k_ee_rowstats<BF16, 1>(Params p, int i);
template __global__ void k_ee_rowstats<BF16, 2>(Params p, int i);
template __global__ void k_ee_tail<F32, 1>(Params p, int P);
template __global__ void k_ee_tail<F32, 2>(Params p, int P);
template __global__ void k_ee_tail<BF16, 1>(Params p, int P);
template __global__ void k_ee_tail<BF16, 2>(Params p, int P);

}  // namespace spv
