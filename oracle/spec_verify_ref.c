/*
 * spec_verify_ref.c -- plain fp64 CPU oracle for the speculative-sampling
 * verification step.
 *
 * TEST INFRASTRUCTURE ONLY. This is the reference the HIP library is checked
 * against. Only the test suite, the smoke check and the benchmark's CPU
 * baseline load it; the product path never does. It shares no code, header,
 * table or helper with the HIP library.
 *
 * It is deliberately slow and literal: every probability row is widened to
 * fp64, normalised in full, and every decision is taken in the order the
 * pages describe. No blocking, no fusion, no reordering.
 *
 * Sources (cited below by the short tag in brackets):
 *   [ART] "Speculative Decoding and the Art of Fast LLM Inference"
 *         (mesuvash.github.io blog), sections "The Algorithm, Step by Step"
 *         and "Why It Stays Exact".
 *   [TLS] thelatentsource.com article "speculative-decoding-llm-speed",
 *         section "The correction that keeps the target in charge"
 *         (P_accept, the accept_token snippet, r(x), the red/blue example).
 *   [TAI] techaiinterview.com, "How does speculative decoding work, why is it
 *         lossless, and how much does it speed things up?", sections
 *         "Core explanation" (algorithm, steps 1-4) and "Deep dive:
 *         correctness and speedup" (greedy rule).
 *   [PHX] J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel
 *         Random Numbers: As Easy as 1, 2, 3", SC'11 -- Philox4x32, 10 rounds.
 *
 * Readings taken where the pages leave a step open (each one is listed with
 * its reason in the design notes of the repository):
 *   R1  temperature: p = softmax(logits / tau) for target and draft alike,
 *       one tau per sequence; tau == 0 selects the greedy rule.
 *   R2  random draws: Philox4x32-10, key = seed, counter = (position, global
 *       sequence index, 0, 0); word 0 -> acceptance uniform, word 1 -> the
 *       residual/bonus uniform; uniform = (word >> 8) * 2^-24 in [0, 1).
 *   R3  acceptance: accept iff u < min(1, p(g)/q(g)), strict.
 *   R4  inverse CDF: ascending token id, C(x) = sum_{y<=x} w(y) summed
 *       sequentially, pick the smallest x with C(x) > v*S.
 *   R5  greedy: accept g_i iff it equals the target argmax at i (lowest id
 *       on ties); the correction/bonus is that argmax.
 *   R6  row alignment: target row i and draft row i score draft position i
 *       (0-based); the bonus is target row L (L = the sequence's draft length).
 *   T1  candidate trees: greedy acceptance only (the pages give no sampling
 *       rule for trees). Node 0 is the root; node n >= 1 holds a drafted
 *       token and a parent with a smaller index; the target row of node n
 *       scores the token that follows node n's path.
 *   T2  a tree round keeps the deepest accepted node, the lowest node index
 *       among equally deep ones.
 *   TP1 top-p ([ART] "Why It Stays Exact", key limitation: verification
 *       must use the target's own sampling parameters, temperature and
 *       top-p): after the temperature softmax, keep whole probability
 *       levels -- tokens of equal logit -- from the top until their mass
 *       reaches top_p times the row's mass; ties at the boundary are all
 *       kept. The kept tokens are renormalised and the rest get 0. The
 *       draft row is filtered with the same top_p. top_p >= 1 keeps all.
 *   TK1 top-k (the same key limitation, for the other common sampling
 *       parameter): keep whole levels from the top until they hold at
 *       least top_k tokens -- every token tied with the top_k-th largest
 *       logit is kept -- and renormalise; top_k <= 0 or >= V keeps all.
 *       With both parameters the row is filtered by top-k first and the
 *       nucleus is then taken on the result (the usual order of sampling
 *       pipelines; the pages give no order).
 *   P1  prompt lookup: n-gram sizes are tried from n_max down to n_min; for
 *       a size n the match is the most recent occurrence of the context's
 *       last n tokens that ends before the last token; the proposal is the
 *       (up to k) tokens that followed it, cut at the end of the context.
 *       No match at any size proposes nothing.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { REF_F32 = 0, REF_BF16 = 1 };

enum {
    REF_SEQ_OK = 0,
    REF_SEQ_BAD_TOKEN = 1,
    REF_SEQ_BAD_LEN = 2,
    REF_SEQ_BAD_TEMP = 3,
    REF_SEQ_QZERO = 4,
    REF_SEQ_BAD_TREE = 5, /* a parent index outside [0, n) for node n */
    REF_SEQ_BAD_TOP_P = 6 /* top_p NaN or not positive                */
};

enum {
    REF_DRAW_NONE = 0,           /* sequence rejected by a status check      */
    REF_DRAW_GREEDY = 1,         /* greedy correction / bonus (argmax)       */
    REF_DRAW_RESIDUAL = 2,       /* sample from norm(max(0, p - q))          */
    REF_DRAW_BONUS = 3,          /* sample from p at row L                   */
    REF_DRAW_RESIDUAL_AS_P = 4   /* residual mass rounded to 0: sample p     */
};

/* ------------------------------------------------------------------ */
/* Input widening (exact): fp32 -> fp64; bf16 -> fp32 -> fp64.          */
/* ------------------------------------------------------------------ */
static double ref_logit(const void *buf, int dtype, size_t idx)
{
    if (dtype == REF_F32)
        return (double)((const float *)buf)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)buf)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------ */
/* Softmax of one logit row at temperature tau (reading R1).            */
/* [ART] "Verify in parallel": the target returns a distribution p_i at */
/* each position; [ART] "Why It Stays Exact", key limitation: draft and */
/* target must use the same sampling parameters (temperature).          */
/* p(x) = exp(x/tau - max_y y/tau) / sum_z exp(z/tau - max_y y/tau).    */
/* ------------------------------------------------------------------ */
void ref_softmax_row(const void *row, int dtype, int64_t V, double tau, double *p)
{
    double mx = -INFINITY;
    for (int64_t x = 0; x < V; x++) {
        double s = ref_logit(row, dtype, (size_t)x) / tau;
        if (s > mx)
            mx = s;
    }
    double z = 0.0;
    for (int64_t x = 0; x < V; x++) {
        p[x] = exp(ref_logit(row, dtype, (size_t)x) / tau - mx);
        z += p[x];
    }
    for (int64_t x = 0; x < V; x++)
        p[x] /= z;
}

/* Lowest token id holding the row maximum (reading R5). */
int64_t ref_argmax_row(const void *row, int dtype, int64_t V)
{
    int64_t best = 0;
    double bv = ref_logit(row, dtype, 0);
    for (int64_t x = 1; x < V; x++) {
        double s = ref_logit(row, dtype, (size_t)x);
        if (s > bv) {
            bv = s;
            best = x;
        }
    }
    return best;
}

/* ------------------------------------------------------------------ */
/* Nucleus (top-p) filter of one probability row (reading TP1).          */
/*   row: the logits (for the levels), p: the row's softmax, filtered    */
/*   in place. Levels are visited from the largest logit down; each      */
/*   level's mass is added to the running total until it reaches        */
/*   top_p * (sum of p); that level and all above it are kept.           */
/* Returns the kept mass before renormalisation; *thr = the boundary     */
/* logit (keep x >= *thr); *margin = distance of top_p * total to the    */
/* running mass just before and just after the boundary level, relative */
/* to total (small: the boundary is a near tie).                        */
/* ------------------------------------------------------------------ */
typedef struct {
    double x;
    int64_t i;
} ref_level_item;

static int ref_level_desc(const void *a, const void *b)
{
    const ref_level_item *u = a, *v = b;
    if (u->x != v->x)
        return u->x > v->x ? -1 : 1;
    return u->i < v->i ? -1 : (u->i > v->i);
}

double ref_nucleus_row(const void *row, int dtype, int64_t V, double top_p, double *p, double *thr,
                       double *margin)
{
    double total = 0.0;
    for (int64_t x = 0; x < V; x++)
        total += p[x];
    *thr = -INFINITY;
    *margin = NAN;
    if (!(top_p < 1.0))
        return total;
    ref_level_item *it = malloc(sizeof(ref_level_item) * (size_t)V);
    if (!it)
        return NAN;
    for (int64_t x = 0; x < V; x++) {
        it[x].x = ref_logit(row, dtype, (size_t)x);
        if (it[x].x == 0.0)
            it[x].x = 0.0; /* -0 and +0 are one level */
        it[x].i = x;
    }
    qsort(it, (size_t)V, sizeof(ref_level_item), ref_level_desc);
    const double target = top_p * total;
    double cum = 0.0, kept = total;
    for (int64_t a = 0; a < V;) {
        int64_t b = a;
        double level = 0.0;
        while (b < V && it[b].x == it[a].x)
            level += p[it[b++].i];
        const double before = cum;
        cum += level;
        if (cum >= target) {
            *thr = it[a].x;
            kept = cum;
            const double m1 = (cum - target) / total, m2 = (target - before) / total;
            *margin = m1 < m2 ? m1 : m2;
            break;
        }
        a = b;
    }
    free(it);
    for (int64_t x = 0; x < V; x++) {
        double lx = ref_logit(row, dtype, (size_t)x);
        p[x] = lx >= *thr ? p[x] / kept : 0.0;
    }
    return kept;
}

/* ------------------------------------------------------------------ */
/* Top-k filter of one probability row (reading TK1): levels are visited */
/* from the largest logit down and kept until they hold at least top_k  */
/* tokens; that level and all above it are kept, the rest get 0, and    */
/* the kept tokens are renormalised in place. Returns the kept mass     */
/* before renormalisation; *thr = the boundary logit (keep x >= *thr).  */
/* top_k <= 0 or >= V keeps everything (*thr = -inf).                    */
/* ------------------------------------------------------------------ */
double ref_topk_row(const void *row, int dtype, int64_t V, int64_t top_k, double *p, double *thr)
{
    double total = 0.0;
    for (int64_t x = 0; x < V; x++)
        total += p[x];
    *thr = -INFINITY;
    if (top_k <= 0 || top_k >= V)
        return total;
    ref_level_item *it = malloc(sizeof(ref_level_item) * (size_t)V);
    if (!it)
        return NAN;
    for (int64_t x = 0; x < V; x++) {
        it[x].x = ref_logit(row, dtype, (size_t)x);
        if (it[x].x == 0.0)
            it[x].x = 0.0; /* -0 and +0 are one level */
        it[x].i = x;
    }
    qsort(it, (size_t)V, sizeof(ref_level_item), ref_level_desc);
    int64_t count = 0;
    for (int64_t a = 0; a < V;) {
        int64_t b = a;
        while (b < V && it[b].x == it[a].x)
            b++;
        count += b - a;
        if (count >= top_k) {
            *thr = it[a].x;
            break;
        }
        a = b;
    }
    free(it);
    double kept = 0.0;
    for (int64_t x = 0; x < V; x++)
        if (ref_logit(row, dtype, (size_t)x) >= *thr)
            kept += p[x];
    for (int64_t x = 0; x < V; x++) {
        double lx = ref_logit(row, dtype, (size_t)x);
        p[x] = lx >= *thr ? p[x] / kept : 0.0;
    }
    return kept;
}

/* ------------------------------------------------------------------ */
/* Philox4x32-10 [PHX] (reading R2).                                    */
/* Each round multiplies counter words 0 and 2 by the two Philox        */
/* multipliers, keeps both halves of each 64-bit product, and mixes the */
/* high halves with the two other counter words and the round key; the */
/* key advances by the two Weyl constants between rounds.               */
/* ------------------------------------------------------------------ */
void ref_philox4x32_10(const uint32_t ctr[4], uint64_t seed, uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    for (int round = 0; round < 10; round++) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        uint64_t prod0 = (uint64_t)M0 * c0;
        uint64_t prod1 = (uint64_t)M1 * c2;
        uint32_t n0 = (uint32_t)(prod1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)prod1;
        uint32_t n2 = (uint32_t)(prod0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)prod0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/* 24 high bits of a word as a uniform in [0, 1): exact in fp32 and fp64. */
double ref_uniform24(uint32_t word)
{
    return (double)(word >> 8) * (1.0 / 16777216.0);
}

/* The two uniforms of draft position `pos` of global sequence `seq`. */
void ref_position_uniforms(uint64_t seed, uint32_t seq, uint32_t pos, double *u, double *v)
{
    uint32_t ctr[4] = {pos, seq, 0u, 0u};
    uint32_t w[4];
    ref_philox4x32_10(ctr, seed, w);
    *u = ref_uniform24(w[0]);
    *v = ref_uniform24(w[1]);
}

/* ------------------------------------------------------------------ */
/* Inverse-CDF draw from non-negative weights w[0..V-1] (reading R4).   */
/* S = sum of w (sequential, so S equals C(V-1)); returns the smallest  */
/* x with C(x) > v*S. A zero-weight id is never returned. If rounding   */
/* left no such x, the largest id with w > 0 is returned and *fallback  */
/* is set. Returns -1 when S <= 0. *margin = distance of v to the       */
/* nearer CDF boundary of the chosen id, in units of S.                 */
/* ------------------------------------------------------------------ */
int64_t ref_draw_inverse_cdf(const double *w, int64_t V, double v, double *S_out,
                             double *margin, int *fallback)
{
    double S = 0.0;
    for (int64_t x = 0; x < V; x++)
        S += w[x];
    *S_out = S;
    *fallback = 0;
    *margin = NAN;
    if (!(S > 0.0))
        return -1;
    double t = v * S;
    double c = 0.0;
    for (int64_t x = 0; x < V; x++) {
        double before = c;
        c += w[x];
        if (c > t) {
            double lo = fabs(v - before / S), hi = fabs(c / S - v);
            *margin = lo < hi ? lo : hi;
            return x;
        }
    }
    *fallback = 1;
    for (int64_t x = V - 1; x >= 0; x--)
        if (w[x] > 0.0) {
            *margin = 0.0;
            return x;
        }
    return -1;
}

/* ------------------------------------------------------------------ */
/* The ids an inverse-CDF draw could return if its uniform were moved by */
/* at most `band` (reading R4, with the flagging rule of the parity      */
/* protocol: a draw whose uniform lies within `band` of a CDF boundary   */
/* may legitimately land on the neighbouring id when the weights are     */
/* rounded differently). Id x, of weight w(x) > 0, owns the uniforms in  */
/* [C(x-1)/S, C(x)/S) with the same sequential C and S as               */
/* ref_draw_inverse_cdf; *lo and *hi are the smallest and largest such x */
/* whose interval meets [v - band, v + band]. Both are -1 when S <= 0.   */
/* ------------------------------------------------------------------ */
void ref_draw_window(const double *w, int64_t V, double v, double band, int64_t *lo, int64_t *hi)
{
    double S = 0.0;
    for (int64_t x = 0; x < V; x++)
        S += w[x];
    *lo = -1;
    *hi = -1;
    if (!(S > 0.0))
        return;
    double c = 0.0;
    for (int64_t x = 0; x < V; x++) {
        double from = c / S;
        c += w[x];
        if (w[x] > 0.0 && c / S > v - band && from <= v + band) {
            if (*lo < 0)
                *lo = x;
            *hi = x;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Flag band of a final draw (parity protocol, not the method). The     */
/* kernel forms each draw weight in fp32 from p(x) and, for a residual, */
/* q(x): a few roundings of relative size 2^-24 of the larger of the    */
/* two. Relative to S the CDF it scans is then uncertain by about       */
/* 2^-24 sqrt(sum_x m(x)^2) / S for independent roundings, with m(x) =  */
/* max(p(x), q(x)) (p(x) alone when q is NULL). A uniform within 8 times */
/* that of a CDF boundary is as undecided in fp32 as one within `band`; */
/* the larger of the two is returned. Where two nearly equal rows put   */
/* almost all their mass on one token, S is tiny against that token's   */
/* weight and the band exceeds 1: the draw is not resolved in fp32.     */
/* ------------------------------------------------------------------ */
double ref_draw_band(const double *p, const double *q, int64_t V, double S, double band)
{
    if (!(S > 0.0))
        return band;
    double m2 = 0.0;
    for (int64_t x = 0; x < V; x++) {
        const double m = q && q[x] > p[x] ? q[x] : p[x];
        m2 += m * m;
    }
    const double e = 8.0 * 0x1p-24 * sqrt(m2) / S;
    return e > band ? e : band;
}

/* ------------------------------------------------------------------ */
/* One sampling round for one sequence, given the probability rows and  */
/* the uniforms ([ART] steps "Accept or reject, left to right", "Stop   */
/* at the first rejection", "Bonus token"; [TLS] P_accept, the          */
/* accept_token rule and r(x); [TAI] algorithm steps 3-4).              */
/*                                                                      */
/*   p : (L+1) x V target probabilities; row L is the bonus position    */
/*   q : L x V draft probabilities                                      */
/*   g : L drafted tokens                                               */
/*   u : L acceptance uniforms;  v : L+1 draw uniforms (row i uses v[i])*/
/*   w : V doubles of scratch                                           */
/* Outputs: out[0..n] (n = accepted count, out[n] = correction/bonus),  */
/* *S (mass of the weights drawn from), *row = n, *kind, margins.       */
/* Returns n, or -1 with *status = REF_SEQ_QZERO when a drafted token   */
/* has no draft probability ([TLS] accept_token raises in that case).   */
/* ------------------------------------------------------------------ */
int ref_round_sampling(const double *p, const double *q, const int32_t *g, int L, int64_t V,
                       const double *u, const double *v, double *w, int32_t *out, double *S,
                       int *row, int *kind, double *margin_accept, double *margin_draw,
                       int *status)
{
    *status = REF_SEQ_OK;
    for (int i = 0; i < L; i++) {
        const double *pi = p + (size_t)i * V;
        const double *qi = q + (size_t)i * V;
        double pg = pi[g[i]], qg = qi[g[i]];
        if (!(qg > 0.0)) {
            *status = REF_SEQ_QZERO;
            return -1;
        }
        double ratio = pg / qg;
        double thr = ratio < 1.0 ? ratio : 1.0;
        margin_accept[i] = fabs(u[i] - thr);
        if (u[i] < thr) {
            out[i] = g[i];
            continue;
        }
        /* First rejection: discard g_i and everything after it, and draw
         * the correction from max(0, p_i - q_i), renormalised. */
        for (int64_t x = 0; x < V; x++) {
            double d = pi[x] - qi[x];
            w[x] = d > 0.0 ? d : 0.0;
        }
        int fb = 0;
        int64_t x = ref_draw_inverse_cdf(w, V, v[i], S, margin_draw, &fb);
        *kind = REF_DRAW_RESIDUAL;
        if (x < 0) {
            /* Only reachable through rounding: exactly, a rejection implies
             * sum max(0, p - q) >= q(g) - p(g) > 0. */
            x = ref_draw_inverse_cdf(pi, V, v[i], S, margin_draw, &fb);
            *kind = REF_DRAW_RESIDUAL_AS_P;
        }
        out[i] = (int32_t)x;
        *row = i;
        return i;
    }
    /* Every draft accepted: one more token from the bonus position. */
    int fb = 0;
    int64_t x = ref_draw_inverse_cdf(p + (size_t)L * V, V, v[L], S, margin_draw, &fb);
    out[L] = (int32_t)x;
    *row = L;
    *kind = REF_DRAW_BONUS;
    return L;
}

/* One greedy round: accept while the target argmax equals the drafted token
 * ([TAI] "Deep dive", greedy remark; reading R5). amax has L+1 entries. */
int ref_round_greedy(const int64_t *amax, const int32_t *g, int L, int32_t *out)
{
    for (int i = 0; i < L; i++) {
        if (amax[i] == g[i]) {
            out[i] = g[i];
            continue;
        }
        out[i] = (int32_t)amax[i];
        return i;
    }
    out[L] = (int32_t)amax[L];
    return L;
}

/* ------------------------------------------------------------------ */
/* The whole step for a batch of B sequences.                           */
/*                                                                      */
/* target: [B, k+1, V], draft: [B, k, V] (dtype REF_F32 or REF_BF16 as  */
/* raw bits); draft_tokens [B, k]; draft_len [B] or NULL (= k);          */
/* temperature [B] fp32. Sequence b draws with global index seq_base+b. */
/*                                                                      */
/* Outputs (all caller-allocated; optional ones may be NULL):           */
/*   out_tokens [B, k+1]: accepted prefix, then the correction or bonus,*/
/*                        then -1;  num_accepted [B];  seq_status [B]    */
/*   p_g, q_g [B, k]: p_i(g_i), q_i(g_i) for sampling rows i < L, NaN   */
/*                    elsewhere                                          */
/*   argmax [B, k+1]: target argmax of rows 0..L of greedy sequences, -1 */
/*   resid_mass [B]: mass S of the weights of the final draw (NaN for   */
/*                   greedy)                                             */
/*   margin_accept [B, k]: |u - min(1, p/q)| per acceptance test, NaN   */
/*   margin_draw [B]: CDF-boundary distance of the final draw, NaN      */
/*   draw_row [B], draw_kind [B]: row of the final token and REF_DRAW_*  */
/* Returns 0, or -1 if a scratch allocation failed.                     */
/* ------------------------------------------------------------------ */
static int verify_batch(const void *target, const void *draft, int dtype,
                        const int32_t *draft_tokens, const int32_t *draft_len,
                        const float *temperature, const int32_t *top_k, const float *top_p,
                        int32_t B, int32_t k,
                        int64_t V, uint64_t seed, uint32_t seq_base, int32_t *out_tokens,
                        int32_t *num_accepted, int32_t *seq_status, double *p_g, double *q_g,
                        int32_t *argmax, double *resid_mass, double *margin_accept,
                        double *margin_draw, double *margin_nucleus, int32_t *draw_row,
                        int32_t *draw_kind, double band, int32_t *draw_window,
                        double *band_draw)
{
    const size_t esz = dtype == REF_F32 ? 4 : 2;
    double *p = malloc(sizeof(double) * (size_t)(k + 1) * (size_t)V);
    double *q = malloc(sizeof(double) * (size_t)(k > 0 ? k : 1) * (size_t)V);
    double *w = malloc(sizeof(double) * (size_t)V);
    double *u = malloc(sizeof(double) * (size_t)(k + 1));
    double *v = malloc(sizeof(double) * (size_t)(k + 1));
    int64_t *amax = malloc(sizeof(int64_t) * (size_t)(k + 1));
    double *macc = malloc(sizeof(double) * (size_t)(k + 1));
    if (!p || !q || !w || !u || !v || !amax || !macc) {
        free(p), free(q), free(w), free(u), free(v), free(amax), free(macc);
        return -1;
    }

    for (int32_t b = 0; b < B; b++) {
        int32_t *out = out_tokens + (size_t)b * (k + 1);
        const int32_t *g = draft_tokens + (size_t)b * k;
        const char *trow0 = (const char *)target + (size_t)b * (k + 1) * V * esz;
        const char *drow0 = (const char *)draft + (size_t)b * k * V * esz;
        int L = draft_len ? draft_len[b] : k;
        double tau = (double)temperature[b];

        for (int i = 0; i <= k; i++)
            out[i] = -1;
        for (int i = 0; i < k; i++) {
            if (p_g) p_g[(size_t)b * k + i] = NAN;
            if (q_g) q_g[(size_t)b * k + i] = NAN;
            if (margin_accept) margin_accept[(size_t)b * k + i] = NAN;
        }
        for (int i = 0; i <= k; i++)
            if (argmax) argmax[(size_t)b * (k + 1) + i] = -1;
        for (int i = 0; i < 2 * k + 1; i++)
            if (margin_nucleus) margin_nucleus[(size_t)b * (2 * k + 1) + i] = NAN;
        if (resid_mass) resid_mass[b] = NAN;
        if (margin_draw) margin_draw[b] = NAN;
        if (draw_row) draw_row[b] = -1;
        if (draw_kind) draw_kind[b] = REF_DRAW_NONE;
        if (draw_window) draw_window[2 * (size_t)b] = draw_window[2 * (size_t)b + 1] = -1;
        if (band_draw) band_draw[b] = NAN;
        num_accepted[b] = 0;

        /* Input checks, in this order: length, temperature, top-p, tokens.
         * A temperature must be 0 (greedy) or a normal positive fp32. */
        int status = REF_SEQ_OK;
        if (L < 0 || L > k)
            status = REF_SEQ_BAD_LEN;
        else if (!(tau == 0.0 || (tau >= (double)1.17549435e-38f && isfinite(tau))))
            status = REF_SEQ_BAD_TEMP;
        else if (top_p && !(top_p[b] > 0.0f))
            status = REF_SEQ_BAD_TOP_P;
        else
            for (int i = 0; i < L; i++)
                if (g[i] < 0 || (int64_t)g[i] >= V)
                    status = REF_SEQ_BAD_TOKEN;
        if (status != REF_SEQ_OK) {
            if (seq_status) seq_status[b] = status;
            continue;
        }

        int n;
        if (tau == 0.0) {
            for (int i = 0; i <= L; i++) {
                amax[i] = ref_argmax_row(trow0 + (size_t)i * V * esz, dtype, V);
                if (argmax) argmax[(size_t)b * (k + 1) + i] = (int32_t)amax[i];
            }
            n = ref_round_greedy(amax, g, L, out);
            if (draw_row) draw_row[b] = n;
            if (draw_kind) draw_kind[b] = REF_DRAW_GREEDY;
        } else {
            for (int i = 0; i <= L; i++)
                ref_softmax_row(trow0 + (size_t)i * V * esz, dtype, V, tau, p + (size_t)i * V);
            for (int i = 0; i < L; i++)
                ref_softmax_row(drow0 + (size_t)i * V * esz, dtype, V, tau, q + (size_t)i * V);
            if (top_k && top_k[b] > 0 && (int64_t)top_k[b] < V) {
                /* top-k first (TK1), on every target and draft row */
                double thr;
                for (int i = 0; i <= L; i++)
                    ref_topk_row(trow0 + (size_t)i * V * esz, dtype, V, top_k[b],
                                 p + (size_t)i * V, &thr);
                for (int i = 0; i < L; i++)
                    ref_topk_row(drow0 + (size_t)i * V * esz, dtype, V, top_k[b],
                                 q + (size_t)i * V, &thr);
            }
            if (top_p && top_p[b] < 1.0f) {
                /* the same nucleus rule on every target and draft row */
                const double tp = (double)top_p[b];
                double thr, mg;
                for (int i = 0; i <= L; i++) {
                    ref_nucleus_row(trow0 + (size_t)i * V * esz, dtype, V, tp, p + (size_t)i * V,
                                    &thr, &mg);
                    if (margin_nucleus) margin_nucleus[(size_t)b * (2 * k + 1) + i] = mg;
                }
                for (int i = 0; i < L; i++) {
                    ref_nucleus_row(drow0 + (size_t)i * V * esz, dtype, V, tp, q + (size_t)i * V,
                                    &thr, &mg);
                    if (margin_nucleus) margin_nucleus[(size_t)b * (2 * k + 1) + k + 1 + i] = mg;
                }
            }
            for (int i = 0; i < L; i++) {
                if (p_g) p_g[(size_t)b * k + i] = p[(size_t)i * V + g[i]];
                if (q_g) q_g[(size_t)b * k + i] = q[(size_t)i * V + g[i]];
            }
            for (int i = 0; i <= L; i++)
                ref_position_uniforms(seed, seq_base + (uint32_t)b, (uint32_t)i, &u[i], &v[i]);
            for (int i = 0; i <= L; i++)
                macc[i] = NAN;
            double S = NAN, mdraw = NAN;
            int row = -1, kind = REF_DRAW_NONE;
            n = ref_round_sampling(p, q, g, L, V, u, v, w, out, &S, &row, &kind, macc, &mdraw,
                                   &status);
            if (status != REF_SEQ_OK) {
                for (int i = 0; i <= k; i++)
                    out[i] = -1;
                if (seq_status) seq_status[b] = status;
                continue;
            }
            for (int i = 0; i < L; i++)
                if (margin_accept) margin_accept[(size_t)b * k + i] = macc[i];
            if (resid_mass) resid_mass[b] = S;
            if (margin_draw) margin_draw[b] = mdraw;
            if (draw_row) draw_row[b] = row;
            if (draw_kind) draw_kind[b] = kind;
            if (draw_window || band_draw) {
                /* the weights of the final draw: the residual (still in the
                 * scratch row w), or p at the draw row; the window is taken
                 * over the draw's own flag band */
                const int resid = kind == REF_DRAW_RESIDUAL;
                const double *wd = resid ? w : p + (size_t)row * V;
                const double be = ref_draw_band(p + (size_t)row * V,
                                                resid ? q + (size_t)row * V : NULL, V, S, band);
                if (band_draw) band_draw[b] = be;
                if (draw_window) {
                    int64_t lo, hi;
                    ref_draw_window(wd, V, v[row], be, &lo, &hi);
                    draw_window[2 * (size_t)b] = (int32_t)lo;
                    draw_window[2 * (size_t)b + 1] = (int32_t)hi;
                }
            }
        }
        num_accepted[b] = n;
        if (seq_status) seq_status[b] = REF_SEQ_OK;
    }

    free(p), free(q), free(w), free(u), free(v), free(amax), free(macc);
    return 0;
}

int spec_verify_ref(const void *target, const void *draft, int dtype,
                    const int32_t *draft_tokens, const int32_t *draft_len,
                    const float *temperature, int32_t B, int32_t k, int64_t V, uint64_t seed,
                    uint32_t seq_base, int32_t *out_tokens, int32_t *num_accepted,
                    int32_t *seq_status, double *p_g, double *q_g, int32_t *argmax,
                    double *resid_mass, double *margin_accept, double *margin_draw,
                    int32_t *draw_row, int32_t *draw_kind)
{
    return verify_batch(target, draft, dtype, draft_tokens, draft_len, temperature, NULL, NULL, B,
                        k, V, seed, seq_base, out_tokens, num_accepted, seq_status, p_g, q_g,
                        argmax, resid_mass, margin_accept, margin_draw, NULL, draw_row,
                        draw_kind, 0.0, NULL, NULL);
}

/* The whole step with nucleus filtering (reading TP1): top_p [B] fp32, 1  */
/* or more (or a greedy sequence) filters nothing. margin_nucleus          */
/* [B, 2k+1] (may be NULL): the nucleus margin of target row i (index i)   */
/* and draft row i (index k+1+i), NaN where no filter was applied.         */
int spec_verify_topp_ref(const void *target, const void *draft, int dtype,
                         const int32_t *draft_tokens, const int32_t *draft_len,
                         const float *temperature, const float *top_p, int32_t B, int32_t k,
                         int64_t V, uint64_t seed, uint32_t seq_base, int32_t *out_tokens,
                         int32_t *num_accepted, int32_t *seq_status, double *p_g, double *q_g,
                         int32_t *argmax, double *resid_mass, double *margin_accept,
                         double *margin_draw, double *margin_nucleus, int32_t *draw_row,
                         int32_t *draw_kind)
{
    return verify_batch(target, draft, dtype, draft_tokens, draft_len, temperature, NULL, top_p,
                        B, k, V, seed, seq_base, out_tokens, num_accepted, seq_status, p_g, q_g,
                        argmax, resid_mass, margin_accept, margin_draw, margin_nucleus,
                        draw_row, draw_kind, 0.0, NULL, NULL);
}

/* The whole step with top-k and nucleus filtering (TK1 then TP1): top_k */
/* [B] int32 (may be NULL: no top-k), top_p [B] fp32 (may be NULL: no    */
/* top-p). The top-p checks and margins are those of spec_verify_topp_ref */
/* (the nucleus margin is taken on the top-k-filtered row).               */
int spec_verify_filter_ref(const void *target, const void *draft, int dtype,
                           const int32_t *draft_tokens, const int32_t *draft_len,
                           const float *temperature, const int32_t *top_k, const float *top_p,
                           int32_t B, int32_t k, int64_t V, uint64_t seed, uint32_t seq_base,
                           int32_t *out_tokens, int32_t *num_accepted, int32_t *seq_status,
                           double *p_g, double *q_g, int32_t *argmax, double *resid_mass,
                           double *margin_accept, double *margin_draw, double *margin_nucleus,
                           int32_t *draw_row, int32_t *draw_kind)
{
    return verify_batch(target, draft, dtype, draft_tokens, draft_len, temperature, top_k, top_p,
                        B, k, V, seed, seq_base, out_tokens, num_accepted, seq_status, p_g, q_g,
                        argmax, resid_mass, margin_accept, margin_draw, margin_nucleus,
                        draw_row, draw_kind, 0.0, NULL, NULL);
}

/* Every option at once: spec_verify_filter_ref (top_k and top_p may be  */
/* NULL) plus, for the final draw of a sampling sequence, band_draw [B]  */
/* (may be NULL): its flag band (ref_draw_band: `band`, or wider where   */
/* fp32 weights cannot resolve the draw; NaN where there was no sampled  */
/* draw), and draw_window [B, 2] (may be NULL): the smallest and largest */
/* token ids a shift of its uniform by at most that band could select    */
/* (ref_draw_window); -1 where there was no sampled draw.                */
int spec_verify_full_ref(const void *target, const void *draft, int dtype,
                         const int32_t *draft_tokens, const int32_t *draft_len,
                         const float *temperature, const int32_t *top_k, const float *top_p,
                         int32_t B, int32_t k, int64_t V, uint64_t seed, uint32_t seq_base,
                         int32_t *out_tokens, int32_t *num_accepted, int32_t *seq_status,
                         double *p_g, double *q_g, int32_t *argmax, double *resid_mass,
                         double *margin_accept, double *margin_draw, double *margin_nucleus,
                         int32_t *draw_row, int32_t *draw_kind, double band,
                         int32_t *draw_window, double *band_draw)
{
    return verify_batch(target, draft, dtype, draft_tokens, draft_len, temperature, top_k, top_p,
                        B, k, V, seed, seq_base, out_tokens, num_accepted, seq_status, p_g, q_g,
                        argmax, resid_mass, margin_accept, margin_draw, margin_nucleus,
                        draw_row, draw_kind, band, draw_window, band_draw);
}

/* ------------------------------------------------------------------ */
/* Greedy verification of one candidate tree ([ART] "EAGLE: drafting in */
/* feature space": a tree of candidate continuations verified together; */
/* [TAI] "Drafts and limits": tree verification checks several          */
/* candidate continuations in one target pass; readings T1, T2, R5).    */
/*                                                                      */
/*   amax[n]: target argmax of node n's row (n < n_nodes)               */
/*   par[n], tok[n]: parent and drafted token of node n >= 1            */
/* Node 0 (the root) is accepted; node n >= 1 is accepted iff its parent */
/* is accepted and tok[n] equals the parent's argmax -- the linear      */
/* greedy rule applied along every branch. The round keeps the deepest  */
/* accepted node b, emits the tokens on the path root -> b and then     */
/* amax[b]. out[0..d-1] = path tokens, out[d] = amax[b],                */
/* path[0..d-1] = path nodes (root excluded). Returns d.                */
/* ------------------------------------------------------------------ */
int ref_tree_greedy(const int64_t *amax, const int32_t *par, const int32_t *tok, int n_nodes,
                    int32_t *out, int32_t *path)
{
    char *acc = malloc((size_t)n_nodes);
    int *depth = malloc(sizeof(int) * (size_t)n_nodes);
    if (!acc || !depth) {
        free(acc), free(depth);
        return -1;
    }
    acc[0] = 1;
    depth[0] = 0;
    for (int n = 1; n < n_nodes; n++) {
        acc[n] = acc[par[n]] && (int64_t)tok[n] == amax[par[n]];
        depth[n] = depth[par[n]] + 1;
    }
    int best = 0;
    for (int n = 1; n < n_nodes; n++)  /* ascending: the first of the deepest wins */
        if (acc[n] && depth[n] > depth[best])
            best = n;
    const int d = depth[best];
    int x = best;
    for (int j = d - 1; j >= 0; j--) {
        path[j] = x;
        out[j] = tok[x];
        x = par[x];
    }
    out[d] = (int32_t)amax[best];
    free(acc), free(depth);
    return d;
}

/* ------------------------------------------------------------------ */
/* Greedy tree verification for a batch of B sequences.                 */
/*                                                                      */
/* target [B, N, V] (dtype REF_F32 or REF_BF16 as raw bits): row n of    */
/* sequence b is scored at node n. parents [B, N], tokens [B, N] (entry */
/* 0 of each is ignored), n_nodes [B] in [1, N].                        */
/* Outputs: out_tokens [B, N]: path tokens, then the bonus, then -1;    */
/* path_nodes [B, N]: path nodes, then -1; num_accepted [B];            */
/* seq_status [B] (REF_SEQ_BAD_LEN: n_nodes outside [1, N];             */
/* REF_SEQ_BAD_TREE: a parent outside [0, n); REF_SEQ_BAD_TOKEN: a token */
/* outside [0, V)); argmax [B, N] (may be NULL): argmax of the rows of  */
/* nodes < n_nodes, -1 elsewhere. Returns 0, or -1 on allocation failure.*/
/* ------------------------------------------------------------------ */
int spec_tree_ref(const void *target, int dtype, const int32_t *parents, const int32_t *tokens,
                  const int32_t *n_nodes, int32_t B, int32_t N, int64_t V, int32_t *out_tokens,
                  int32_t *path_nodes, int32_t *num_accepted, int32_t *seq_status,
                  int32_t *argmax)
{
    const size_t esz = dtype == REF_F32 ? 4 : 2;
    int64_t *amax = malloc(sizeof(int64_t) * (size_t)N);
    if (!amax)
        return -1;
    for (int32_t b = 0; b < B; b++) {
        int32_t *out = out_tokens + (size_t)b * N;
        int32_t *path = path_nodes + (size_t)b * N;
        const int32_t *par = parents + (size_t)b * N;
        const int32_t *tok = tokens + (size_t)b * N;
        const int nn = n_nodes[b];
        for (int n = 0; n < N; n++) {
            out[n] = -1;
            path[n] = -1;
            if (argmax) argmax[(size_t)b * N + n] = -1;
        }
        num_accepted[b] = 0;
        int status = REF_SEQ_OK;
        if (nn < 1 || nn > N) {
            status = REF_SEQ_BAD_LEN;
        } else {
            for (int n = 1; n < nn; n++)
                if (par[n] < 0 || par[n] >= n)
                    status = REF_SEQ_BAD_TREE;
            if (status == REF_SEQ_OK)
                for (int n = 1; n < nn; n++)
                    if (tok[n] < 0 || (int64_t)tok[n] >= V)
                        status = REF_SEQ_BAD_TOKEN;
        }
        seq_status[b] = status;
        if (status != REF_SEQ_OK)
            continue;
        const char *rows = (const char *)target + (size_t)b * N * V * esz;
        for (int n = 0; n < nn; n++) {
            amax[n] = ref_argmax_row(rows + (size_t)n * V * esz, dtype, V);
            if (argmax) argmax[(size_t)b * N + n] = (int32_t)amax[n];
        }
        const int d = ref_tree_greedy(amax, par, tok, nn, out, path);
        if (d < 0) {
            free(amax);
            return -1;
        }
        num_accepted[b] = d;
    }
    free(amax);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Prompt-lookup drafting for one context ([ART] "n-gram and prompt     */
/* lookup: no model at all": search the existing context for a recent   */
/* matching n-gram and propose the tokens that followed it last time;   */
/* [TAI] "Drafts and limits", n-gram / prompt lookup; reading P1).      */
/*                                                                      */
/*   ctx[0..T-1]: the context. For n = n_max down to n_min, and for     */
/*   start s = T-n-1 down to 0 (latest first), the window ctx[s..s+n-1] */
/*   matches if it equals the last n tokens ctx[T-n..T-1]; the first    */
/*   match proposes ctx[s+n .. min(s+n+k, T) - 1].                      */
/* Writes the proposal to draft[0..len-1] and returns len (0 if none);  */
/* *match_n and *match_s get the n-gram size and start (0 and -1 when   */
/* nothing matched).                                                    */
/* ------------------------------------------------------------------ */
int ref_prompt_lookup(const int32_t *ctx, int T, int n_min, int n_max, int k, int32_t *draft,
                      int *match_n, int *match_s)
{
    *match_n = 0;
    *match_s = -1;
    for (int n = n_max; n >= n_min; n--) {
        if (n > T - 1)
            continue;  /* no window of this size ends before the last token */
        for (int s = T - n - 1; s >= 0; s--) {
            int same = 1;
            for (int j = 0; j < n; j++)
                if (ctx[s + j] != ctx[T - n + j]) {
                    same = 0;
                    break;
                }
            if (!same)
                continue;
            int len = 0;
            for (int j = s + n; j < T && len < k; j++)
                draft[len++] = ctx[j];
            *match_n = n;
            *match_s = s;
            return len;
        }
    }
    return 0;
}

/* Prompt lookup for a batch: contexts [B, T_max] (row b holds ctx_len[b]  */
/* tokens; a length outside [0, T_max] proposes nothing); draft_tokens    */
/* [B, k] (-1 after the proposal), draft_len [B], match_n [B],            */
/* match_s [B] (may be NULL).                                            */
void spec_prompt_lookup_ref(const int32_t *contexts, const int32_t *ctx_len, int32_t B,
                            int32_t T_max, int32_t n_min, int32_t n_max, int32_t k,
                            int32_t *draft_tokens, int32_t *draft_len, int32_t *match_n,
                            int32_t *match_s)
{
    for (int32_t b = 0; b < B; b++) {
        int32_t *d = draft_tokens + (size_t)b * k;
        for (int j = 0; j < k; j++)
            d[j] = -1;
        const int T = ctx_len[b];
        int mn = 0, ms = -1, len = 0;
        if (T >= 0 && T <= T_max)
            len = ref_prompt_lookup(contexts + (size_t)b * T_max, T, n_min, n_max, k, d, &mn,
                                    &ms);
        draft_len[b] = len;
        if (match_n) match_n[b] = mn;
        if (match_s) match_s[b] = ms;
    }
}
