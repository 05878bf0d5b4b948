/*
 * oracle_runner.c -- runs every entry of the C oracle (oracle/spec_verify_ref.c)
 * on small seeded batches, for builds with AddressSanitizer and
 * UndefinedBehaviorSanitizer, or ThreadSanitizer (`threads` > 1: disjoint
 * slices of each batch on parallel threads, as the Python wrapper does).
 *
 * Test infrastructure only. Inputs come from a plain 64-bit LCG; nothing of
 * the verification's arithmetic is here. Exits non-zero if an entry reports
 * an allocation failure or an output leaves its documented range; the
 * sanitizers abort on their own findings.
 *
 *   oracle_runner [threads]
 */
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int spec_verify_full_ref(const void *target, const void *draft, int dtype,
                         const int32_t *draft_tokens, const int32_t *draft_len,
                         const float *temperature, const int32_t *top_k, const float *top_p,
                         int32_t B, int32_t k, int64_t V, uint64_t seed, uint32_t seq_base,
                         int32_t *out_tokens, int32_t *num_accepted, int32_t *seq_status,
                         double *p_g, double *q_g, int32_t *argmax, double *resid_mass,
                         double *margin_accept, double *margin_draw, double *margin_nucleus,
                         int32_t *draw_row, int32_t *draw_kind, double band,
                         int32_t *draw_window, double *band_draw);
int spec_tree_ref(const void *target, int dtype, const int32_t *parents, const int32_t *tokens,
                  const int32_t *n_nodes, int32_t B, int32_t N, int64_t V, int32_t *out_tokens,
                  int32_t *path_nodes, int32_t *num_accepted, int32_t *seq_status,
                  int32_t *argmax);
void spec_prompt_lookup_ref(const int32_t *contexts, const int32_t *ctx_len, int32_t B,
                            int32_t T_max, int32_t n_min, int32_t n_max, int32_t k,
                            int32_t *draft_tokens, int32_t *draft_len, int32_t *match_n,
                            int32_t *match_s);

static uint64_t lcg_state;
static uint32_t next_u32(void)
{
    lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(lcg_state >> 32);
}
/* roughly N(0, s^2): a sum of four uniforms, centred */
static float noise(float s)
{
    float a = 0.f;
    for (int i = 0; i < 4; i++)
        a += (float)next_u32() * (1.0f / 4294967296.0f);
    return (a - 2.f) * 1.7f * s;
}
static uint16_t to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16);
}

/* One batch and its outputs. */
typedef struct {
    int dtype, B, k;
    int64_t V;
    void *target, *draft;
    int32_t *tokens, *lens, *top_k;
    float *temp, *top_p;
    int32_t *out, *nacc, *status, *amax, *drow, *dkind, *win;
    double *pg, *qg, *S, *macc, *mdraw, *mnuc;
} batch_t;

static void *xcalloc(size_t n, size_t sz)
{
    void *p = calloc(n ? n : 1, sz);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(3);
    }
    return p;
}

static void make_batch(batch_t *bt, int dtype, int B, int k, int64_t V)
{
    bt->dtype = dtype, bt->B = B, bt->k = k, bt->V = V;
    const size_t nt = (size_t)B * (k + 1) * V, nd = (size_t)B * k * V;
    const size_t esz = dtype == 0 ? 4 : 2;
    bt->target = xcalloc(nt, esz);
    bt->draft = xcalloc(nd, esz);
    for (size_t i = 0; i < nt; i++) {
        const float x = noise(2.f);
        if (dtype == 0) ((float *)bt->target)[i] = x;
        else ((uint16_t *)bt->target)[i] = to_bf16(x);
    }
    for (int b = 0; b < B; b++)
        for (int i = 0; i < k; i++)
            for (int64_t x = 0; x < V; x++) {
                const size_t ti = ((size_t)b * (k + 1) + i) * V + x, di = ((size_t)b * k + i) * V + x;
                if (dtype == 0)
                    ((float *)bt->draft)[di] = ((float *)bt->target)[ti] + noise(0.7f);
                else
                    ((uint16_t *)bt->draft)[di] = to_bf16(noise(2.f));
            }
    bt->tokens = xcalloc((size_t)B * k, 4);
    bt->lens = xcalloc((size_t)B, 4);
    bt->top_k = xcalloc((size_t)B, 4);
    bt->temp = xcalloc((size_t)B, 4);
    bt->top_p = xcalloc((size_t)B, 4);
    static const float taus[] = {0.f, 0.6f, 1.f, 1.7f};
    for (int b = 0; b < B; b++) {
        bt->lens[b] = (int32_t)(next_u32() % (uint32_t)(k + 1));
        bt->temp[b] = taus[b % 4];
        bt->top_k[b] = (int32_t)(next_u32() % (uint32_t)(V + 2)) - 1;
        bt->top_p[b] = (float)(next_u32() % 11) / 10.f;  /* 0 (an input error) .. 1 */
        for (int i = 0; i < k; i++)
            bt->tokens[(size_t)b * k + i] = (int32_t)(next_u32() % (uint32_t)V);
    }
    if (B > 1 && k > 0) bt->tokens[(size_t)k] = (int32_t)V + 3; /* a bad token */
    if (B > 2) bt->lens[2] = k + 1;                          /* a bad length */
    if (B > 3) bt->temp[3] = -1.f;                           /* a bad temperature */
    bt->out = xcalloc((size_t)B * (k + 1), 4);
    bt->nacc = xcalloc((size_t)B, 4);
    bt->status = xcalloc((size_t)B, 4);
    bt->amax = xcalloc((size_t)B * (k + 1), 4);
    bt->drow = xcalloc((size_t)B, 4);
    bt->dkind = xcalloc((size_t)B, 4);
    bt->win = xcalloc((size_t)B * 2, 4);
    bt->pg = xcalloc((size_t)B * k, 8);
    bt->qg = xcalloc((size_t)B * k, 8);
    bt->S = xcalloc((size_t)B, 8);
    bt->macc = xcalloc((size_t)B * k, 8);
    bt->mdraw = xcalloc((size_t)B, 8);
    bt->mnuc = xcalloc((size_t)B * (2 * k + 1), 8);
}

static void free_batch(batch_t *bt)
{
    void *ps[] = {bt->target, bt->draft, bt->tokens, bt->lens, bt->top_k, bt->temp, bt->top_p,
                  bt->out, bt->nacc, bt->status, bt->amax, bt->drow, bt->dkind, bt->win,
                  bt->pg, bt->qg, bt->S, bt->macc, bt->mdraw, bt->mnuc};
    for (size_t i = 0; i < sizeof ps / sizeof ps[0]; i++)
        free(ps[i]);
}

/* filters: 0 none, 1 top-p, 2 top-k then top-p */
typedef struct {
    batch_t *bt;
    int b0, b1, filters;
    int rc;
} slice_t;

static void *run_slice(void *arg)
{
    slice_t *s = arg;
    batch_t *bt = s->bt;
    const int k = bt->k, b0 = s->b0, n = s->b1 - s->b0;
    const int64_t V = bt->V;
    const size_t esz = bt->dtype == 0 ? 4 : 2;
    s->rc = spec_verify_full_ref(
        (const char *)bt->target + (size_t)b0 * (k + 1) * V * esz,
        (const char *)bt->draft + (size_t)b0 * k * V * esz, bt->dtype, bt->tokens + (size_t)b0 * k,
        bt->lens + b0, bt->temp + b0, s->filters == 2 ? bt->top_k + b0 : NULL,
        s->filters >= 1 ? bt->top_p + b0 : NULL, n, k, V, 0x1234567890abcdefull, (uint32_t)b0,
        bt->out + (size_t)b0 * (k + 1), bt->nacc + b0, bt->status + b0, bt->pg + (size_t)b0 * k,
        bt->qg + (size_t)b0 * k, bt->amax + (size_t)b0 * (k + 1), bt->S + b0,
        bt->macc + (size_t)b0 * k, bt->mdraw + b0,
        s->filters >= 1 ? bt->mnuc + (size_t)b0 * (2 * k + 1) : NULL, bt->drow + b0,
        bt->dkind + b0, 1e-6, bt->win + 2 * (size_t)b0, NULL);
    return NULL;
}

static int check_batch(const batch_t *bt)
{
    for (int b = 0; b < bt->B; b++) {
        const int n = bt->nacc[b];
        if (bt->status[b] != 0) {
            if (n != 0) return 1;
            continue;
        }
        if (n < 0 || n > bt->lens[b]) return 1;
        const int32_t tok = bt->out[(size_t)b * (bt->k + 1) + n];
        if (tok < 0 || tok >= bt->V) return 1;
        for (int i = n + 1; i <= bt->k; i++)
            if (bt->out[(size_t)b * (bt->k + 1) + i] != -1) return 1;
    }
    return 0;
}

static int run_verify(int threads)
{
    static const struct { int dtype, B, k; int64_t V; } shapes[] = {
        {0, 9, 3, 257}, {1, 9, 4, 1001}, {0, 6, 0, 17}, {1, 5, 63, 8}, {0, 12, 2, 1},
    };
    int bad = 0;
    for (size_t si = 0; si < sizeof shapes / sizeof shapes[0]; si++) {
        batch_t bt;
        make_batch(&bt, shapes[si].dtype, shapes[si].B, shapes[si].k, shapes[si].V);
        for (int filters = 0; filters < 3; filters++) {
            const int nth = threads < bt.B ? threads : bt.B;
            pthread_t tid[64];
            slice_t sl[64];
            const int step = (bt.B + nth - 1) / nth;
            int used = 0;
            for (int b0 = 0; b0 < bt.B; b0 += step, used++) {
                sl[used] = (slice_t){&bt, b0, b0 + step < bt.B ? b0 + step : bt.B, filters, 0};
                if (nth > 1) pthread_create(&tid[used], NULL, run_slice, &sl[used]);
                else run_slice(&sl[used]);
            }
            for (int t = 0; t < used; t++) {
                if (nth > 1) pthread_join(tid[t], NULL);
                bad |= sl[t].rc != 0;
            }
            bad |= check_batch(&bt);
        }
        free_batch(&bt);
    }
    return bad;
}

static int run_tree_and_lookup(void)
{
    enum { B = 5, N = 12, V = 300, T = 200 };
    uint16_t *target = xcalloc((size_t)B * N * V, 2);
    for (size_t i = 0; i < (size_t)B * N * V; i++)
        target[i] = to_bf16(noise(2.f));
    int32_t par[B * N], tok[B * N], nn[B], out[B * N], path[B * N], nacc[B], st[B], am[B * N];
    for (int b = 0; b < B; b++) {
        nn[b] = 1 + (int)(next_u32() % N);
        for (int n = 0; n < N; n++) {
            par[b * N + n] = n ? (int32_t)(next_u32() % (uint32_t)n) : -1;
            tok[b * N + n] = (int32_t)(next_u32() % V);
        }
    }
    par[2 * N + 3] = 7;  /* a parent after its node: status BAD_TREE */
    int bad = spec_tree_ref(target, 1, par, tok, nn, B, N, V, out, path, nacc, st, am) != 0;
    free(target);

    int32_t ctx[B * T], lens[B], draft[B * 7], dlen[B], mn[B], ms[B];
    for (int b = 0; b < B; b++) {
        lens[b] = (int32_t)(next_u32() % (T + 1));
        for (int t = 0; t < T; t++)
            ctx[b * T + t] = (int32_t)(next_u32() % 6);
    }
    spec_prompt_lookup_ref(ctx, lens, B, T, 1, 4, 7, draft, dlen, mn, ms);
    for (int b = 0; b < B; b++)
        bad |= dlen[b] < 0 || dlen[b] > 7;
    return bad;
}

int main(int argc, char **argv)
{
    const int threads = argc > 1 ? atoi(argv[1]) : 1;
    lcg_state = 0x9e3779b97f4a7c15ull;
    int bad = run_verify(threads < 1 ? 1 : (threads > 64 ? 64 : threads));
    bad |= run_tree_and_lookup();
    printf("oracle runner: %s\n", bad ? "FAILED" : "ok");
    return bad ? 1 : 0;
}
