/*
 * spec_verify.h -- C ABI of the speculative-sampling verification step on
 * AMD Instinct MI355X (gfx950).
 *
 * One call verifies a batch of B drafted continuations. For each sequence b
 * it takes the target model's logits at k+1 positions, the draft model's
 * logits at k positions and the k drafted tokens, and returns the accepted
 * draft prefix followed by exactly one more token:
 *
 *   - sampling (temperature > 0): p_i = softmax(target_i / tau),
 *     q_i = softmax(draft_i / tau); drafted token g_i is accepted iff
 *     u_i < min(1, p_i(g_i) / q_i(g_i)), scanning left to right and stopping
 *     at the first rejection; at a rejection the token is drawn from
 *     norm(max(0, p_i - q_i)); when every draft is accepted a bonus token is
 *     drawn from the target distribution at the position after the last
 *     draft.
 *     ["Speculative Decoding and the Art of Fast LLM Inference",
 *      "The Algorithm, Step by Step", steps 3-5; thelatentsource.com
 *      "speculative-decoding-llm-speed", "The correction that keeps the
 *      target in charge", P_accept and r(x); techaiinterview.com
 *      speculative-decoding question, "Core explanation", steps 3-4.]
 *   - greedy (temperature == 0): accept g_i while it equals the target
 *     argmax at i (lowest token id on ties); the extra token is that argmax.
 *     [techaiinterview.com, "Deep dive: correctness and speedup", greedy
 *      remark.]
 *
 * Random draws. The pages leave the generator open. This library draws, for
 * draft position i of global sequence s = seq_base + b, one Philox4x32-10
 * block (Salmon et al., SC'11) with key = seed (low word first) and counter
 * (i, s, 0, 0). Word 0 gives the acceptance uniform u_i, word 1 the uniform
 * v_i of a correction/bonus draw at row i; a uniform is (word >> 8) * 2^-24.
 * The draw at a row picks the smallest token id x whose cumulative weight
 * C(x) = sum_{y <= x} w(y) exceeds v * sum_y w(y). Outputs are therefore a
 * deterministic function of (inputs, seed, seq_base), and splitting a batch
 * across calls with matching seq_base gives identical results.
 *
 * Memory. Every pointer argument is device memory owned by the caller,
 * except `aux` (a host struct whose members are device pointers). The
 * library allocates nothing and keeps no state between calls (the one
 * exception, spec_verify_noalloc, keeps a static device array per GPU and
 * its address); calls on different streams with different workspaces may
 * run concurrently. Inputs
 * are only read. All work is enqueued on `stream` (a hipStream_t, NULL for
 * the default stream); the call does not synchronise.
 *
 * Errors. Problems visible on the host (null required pointer, bad sizes or
 * dtype, misaligned pointer, workspace too small) return a status at once
 * and enqueue nothing. Problems in device data are reported per sequence in
 * aux->seq_status (SPEC_SEQ_*); such a sequence gets num_accepted = 0 and
 * out_tokens all -1. Logits may be -inf (a masked token: weight 0) as long
 * as every row the call reads holds a finite logit; NaN, +inf or a row of
 * -inf alone give unspecified (but memory-safe) results.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of the logits. */
typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype_t;

/* Host-side return codes. */
typedef enum {
    SPEC_OK = 0,
    SPEC_EINVAL = 1,     /* bad pointer, size, dtype or alignment          */
    SPEC_EWORKSPACE = 2, /* workspace null, misaligned or too small         */
    SPEC_ELAUNCH = 3,    /* a kernel launch failed (see hipGetLastError)    */
    SPEC_ESCRATCH = 4    /* spec_verify_noalloc: the sizes need more than   */
                         /* SPEC_NOALLOC_SCRATCH_BYTES of workspace         */
} spec_status_t;

/* Per-sequence device status codes, written to aux->seq_status. */
enum {
    SPEC_SEQ_OK = 0,
    SPEC_SEQ_BAD_TOKEN = 1, /* a drafted token g_i (i < L) outside [0, V)     */
    SPEC_SEQ_BAD_LEN = 2,   /* draft length outside [0, k]                   */
    SPEC_SEQ_BAD_TEMP = 3,  /* temperature NaN, infinite, negative, or       */
                            /* positive but below FLT_MIN                    */
    SPEC_SEQ_QZERO = 4,     /* the scan reached a drafted token whose fp32   */
                            /* draft probability is 0 (the acceptance ratio  */
                            /* is undefined; thelatentsource.com accept_token */
                            /* raises in this case)                          */
    SPEC_SEQ_BAD_TREE = 5,  /* spec_verify_tree: a parent index outside      */
                            /* [0, n) for node n                             */
    SPEC_SEQ_BAD_TOP_P = 6  /* spec_verify_top_p: top_p NaN or not positive  */
};

/* How the last emitted token of a sequence was produced (aux->draw_kind). */
enum {
    SPEC_DRAW_NONE = 0,           /* sequence failed a status check          */
    SPEC_DRAW_GREEDY = 1,         /* target argmax (greedy correction/bonus) */
    SPEC_DRAW_RESIDUAL = 2,       /* drawn from norm(max(0, p - q))          */
    SPEC_DRAW_BONUS = 3,          /* drawn from p at row L                   */
    SPEC_DRAW_RESIDUAL_AS_P = 4   /* residual mass rounded to 0: drawn from p */
};

/* Largest supported number of drafted positions. */
#define SPEC_MAX_K 63

/* Optional diagnostic outputs. Every member may be NULL. Device pointers,
 * caller-owned, fully overwritten on each call. */
typedef struct {
    float *p_g;          /* [B, k]: p_i(g_i) for i < L of sampling sequences; NaN elsewhere */
    float *q_g;          /* [B, k]: q_i(g_i), same positions                              */
    float *resid_mass;   /* [B]: total weight of the final draw (sum max(0, p-q) at a     */
                         /*      rejection, sum p for a bonus); NaN for greedy or errors   */
    int32_t *argmax;     /* [B, k+1]: target argmax of rows 0..L of greedy sequences; -1   */
    int32_t *seq_status; /* [B]: SPEC_SEQ_*                                                */
    int32_t *draw_row;   /* [B]: row of the last emitted token (= num_accepted), -1 on error */
    int32_t *draw_kind;  /* [B]: SPEC_DRAW_*                                               */
    void *event_begin;   /* hipEvent_t or NULL: recorded on `stream` right before the     */
    void *event_end;     /* row pass (the kernels that read every logit row: the row      */
                         /* statistics, and with a filter the filter pass) and right      */
                         /* after it; when B is split into several launch slices          */
                         /* (B * (2k+1) * ceil(V*e / 32 KiB) > 2^22), around the first    */
                         /* slice's                                                       */
} spec_verify_aux_t;

/* Bytes of scratch device memory one spec_verify or spec_verify_early_exit
 * call with these sizes needs. Returns 0 for invalid sizes. */
size_t spec_verify_workspace_size(int32_t B, int32_t k, int32_t V, int32_t dtype);

/*
 * Verify B drafted continuations.
 *
 *   target_logits [B, k+1, V] row-major, dtype. Row i of sequence b scores
 *                 draft position i; row L_b is the bonus position. Rows
 *                 beyond L_b are never read.
 *   draft_logits  [B, k, V] row-major, dtype. Only rows i < L_b of sampling
 *                 sequences are read (greedy sequences never read it).
 *                 May be NULL when k == 0.
 *   dtype         SPEC_F32 or SPEC_BF16.
 *   draft_tokens  [B, k] int32. Entries at i >= L_b are ignored. May be NULL
 *                 when k == 0.
 *   draft_len     [B] int32, L_b in [0, k]; NULL means every L_b = k.
 *   temperature   [B] fp32; 0 selects the greedy rule for that sequence.
 *   B, k, V       B >= 0 (B == 0 does nothing), 0 <= k <= SPEC_MAX_K,
 *                 1 <= V < 2^31.
 *   seed          Philox key (see above).
 *   seq_base      global index of sequence 0 for the Philox counter.
 *   out_tokens    [B, k+1] int32 out: g_0..g_{n-1}, then the correction or
 *                 bonus token at position n, then -1 up to position k.
 *   num_accepted  [B] int32 out: n in [0, L_b]; the round emits n+1 tokens.
 *   aux           NULL, or optional diagnostics (see spec_verify_aux_t).
 *   workspace     device scratch of at least spec_verify_workspace_size()
 *                 bytes, 256-byte aligned; its contents need no
 *                 initialisation and are clobbered.
 *   stream        hipStream_t (NULL = default stream).
 *
 * Logit pointers must be aligned to their element size; int32 and fp32
 * arrays to 4 bytes. Returns SPEC_OK once all work is enqueued.
 */
int spec_verify(const void *target_logits, const void *draft_logits, int32_t dtype,
                const int32_t *draft_tokens, const int32_t *draft_len,
                const float *temperature, int32_t B, int32_t k, int32_t V, uint64_t seed,
                uint32_t seq_base, int32_t *out_tokens, int32_t *num_accepted,
                const spec_verify_aux_t *aux, void *workspace, size_t workspace_bytes,
                void *stream);

/*
 * Same step with an early-exit schedule: the draft positions are taken one
 * at a time for the whole batch, and position i reads only the target and
 * draft rows of the sequences that accepted every earlier drafted token.
 * A round stops at its first rejection, and nothing after that position
 * affects its outputs ("Speculative Decoding and the Art of Fast LLM
 * Inference", "The Algorithm, Step by Step", step "Stop at the first
 * rejection"; techaiinterview.com, "Core explanation", step 3), so rows past
 * it need not be read at all.
 *
 * Arguments, layouts, ownership, RNG contract and host-side errors are those
 * of spec_verify, and out_tokens, num_accepted, seq_status, draw_row,
 * draw_kind and resid_mass are bit-identical to spec_verify's for the same
 * inputs, seed and seq_base. The diagnostics of rows that are never read
 * differ: p_g and q_g are written only for positions up to the stop (and
 * are NaN after it), argmax only for greedy rows up to the stop (-1 after
 * it). Enqueues at most 8 kernels, whatever k: one row-statistics launch
 * for each of positions 0..3, a decision launch after position 0 (from
 * position 1 on, the workgroup that completes a sequence's rows decides
 * it), one launch for all positions from 4 on (every remaining row of the
 * sequences still accepting at position 4, read even past a later stop),
 * and the draw (two launches). event_begin / event_end bracket the
 * position launches.
 * Pays when rejections come early (few accepted tokens per round): up to
 * position 4 it reads about (1 - a^L) / (1 - a) positions per sequence
 * instead of L + 1, at a per-token acceptance rate a. Each position costs
 * a launch and a decision (roughly 10 us on MI355X whatever its size), so
 * it pays only when the rows it skips outweigh that, which needs large
 * batches: measured on MI355X with bf16 logits, B=1024 k=7 V=128256 at 1.4
 * tokens per round took 0.34 ms against 0.43 ms for spec_verify, while
 * B=256 k=4 V=152064 took 0.12 ms against 0.095 ms and B=64 k=5 V=128256
 * 0.077 ms against 0.049 ms.
 */
int spec_verify_early_exit(const void *target_logits, const void *draft_logits, int32_t dtype,
                           const int32_t *draft_tokens, const int32_t *draft_len,
                           const float *temperature, int32_t B, int32_t k, int32_t V,
                           uint64_t seed, uint32_t seq_base, int32_t *out_tokens,
                           int32_t *num_accepted, const spec_verify_aux_t *aux,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * The step with top-p (nucleus) sampling parameters. Verification must use
 * the target's own sampling parameters, temperature and top-p, for the
 * output to follow the target ("Speculative Decoding and the Art of Fast
 * LLM Inference", "Why It Stays Exact", key limitation). For a sampling
 * sequence with 0 < top_p[b] < 1, every target row i <= L and draft row
 * i < L is filtered after the temperature softmax: whole probability levels
 * (tokens of equal logit) are kept from the largest logit down until their
 * mass reaches top_p of the row's mass (tokens tied at the boundary are all
 * kept), and the kept tokens are renormalised. The acceptance test, the
 * residual max(0, p - q) and the bonus draw then use the filtered p and q;
 * a drafted token outside the draft row's nucleus has q(g) = 0 and gives
 * SPEC_SEQ_QZERO. top_p[b] >= 1 filters nothing; greedy sequences ignore
 * it; NaN or top_p[b] <= 0 gives SPEC_SEQ_BAD_TOP_P (checked after the
 * temperature, before the tokens). top_p is [B] fp32 device memory and
 * must not be NULL; everything else is as for spec_verify, with aux->q_g
 * and p_g the filtered probabilities and resid_mass the filtered mass.
 * The nucleus of a row is found exactly, with the row masses summed in
 * 64-bit fixed point. A filtered bf16 row is read once, by a pass that
 * counts its tokens per bf16 value (in place of the row statistics); an
 * fp32 row, and a bf16 row the counts cannot settle (its crossing among
 * magnitudes below 2^-14 or below -2^18, a value at or above 2^18, a NaN,
 * or more than 2048 nonzero magnitudes below 2^-14), takes a radix select
 * over the logits: two or three more reads.
 */
int spec_verify_top_p(const void *target_logits, const void *draft_logits, int32_t dtype,
                      const int32_t *draft_tokens, const int32_t *draft_len,
                      const float *temperature, const float *top_p, int32_t B, int32_t k,
                      int32_t V, uint64_t seed, uint32_t seq_base, int32_t *out_tokens,
                      int32_t *num_accepted, const spec_verify_aux_t *aux, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * The step with top-k and top-p sampling parameters (the same key
 * limitation: verification uses the target's own sampling parameters).
 * For a sampling sequence with 0 < top_k[b] < V, every target row i <= L
 * and draft row i < L first keeps whole levels from the largest logit down
 * until they hold at least top_k[b] tokens (every token tied with the
 * top_k-th largest logit is kept) and is renormalised; then, if top_p is
 * given and top_p[b] < 1, the nucleus is taken on that result as for
 * spec_verify_top_p. top_k[b] <= 0 or >= V applies no top-k. Either
 * pointer may be NULL (that filter is off) but not both; top_k is [B]
 * int32 and top_p [B] fp32 device memory. Statuses, outputs and
 * diagnostics are those of spec_verify_top_p, on the filtered rows. The
 * top-k threshold is found exactly from the per-value counts of the same
 * single pass (bf16 rows, when the top_k-th token has a magnitude in
 * [2^-14, 2^18)) or by a radix select over the counts.
 */
int spec_verify_top_k_top_p(const void *target_logits, const void *draft_logits, int32_t dtype,
                            const int32_t *draft_tokens, const int32_t *draft_len,
                            const float *temperature, const int32_t *top_k, const float *top_p,
                            int32_t B, int32_t k, int32_t V, uint64_t seed, uint32_t seq_base,
                            int32_t *out_tokens, int32_t *num_accepted,
                            const spec_verify_aux_t *aux, void *workspace, size_t workspace_bytes,
                            void *stream);

/* ------------------------------------------------------------------------
 * Greedy verification of candidate trees.
 *
 * A draft may be a tree of candidate continuations verified in one target
 * pass ("Speculative Decoding and the Art of Fast LLM Inference", "EAGLE:
 * drafting in feature space"; techaiinterview.com, "Drafts and limits",
 * tree verification). Node 0 of a sequence's tree is the root (the last
 * committed position); node n >= 1 holds a drafted token tokens[n] and hangs
 * below parents[n] < n. Target row n scores the token that follows node n's
 * path. The pages give no sampling rule for trees, so the rule is greedy:
 * node n >= 1 is accepted iff its parent is accepted and tokens[n] equals
 * the argmax of the parent's row (lowest token id on ties); the round keeps
 * the deepest accepted node (the lowest node index among equally deep ones)
 * and emits the tokens on its path, then the argmax of its row. A chain tree
 * (parents[n] = n - 1) is exactly spec_verify's greedy rule.
 * ---------------------------------------------------------------------- */

/* Largest supported number of nodes per tree (one wave lane per node). */
#define SPEC_MAX_TREE 64

/* Optional outputs of spec_verify_tree. Every member may be NULL. */
typedef struct {
    int32_t *seq_status; /* [B]: SPEC_SEQ_OK, _BAD_LEN (n_nodes outside [1, N]),          */
                         /*      _BAD_TREE, or _BAD_TOKEN (a token outside [0, V))        */
    int32_t *argmax;     /* [B, N]: argmax of the rows of nodes < n_nodes; -1 elsewhere    */
    void *event_begin;   /* hipEvent_t or NULL: recorded right before and right after the  */
    void *event_end;     /* row kernel (of the first launch slice)                        */
} spec_tree_aux_t;

/* Workspace bytes one spec_verify_tree call needs; 0 for invalid sizes. */
size_t spec_verify_tree_workspace_size(int32_t B, int32_t N, int32_t V, int32_t dtype);

/*
 *   target_logits [B, N, V] row-major, dtype; rows of nodes >= n_nodes[b] are
 *                 never read.
 *   parents, tokens [B, N] int32; entry 0 (the root) of each is ignored.
 *   n_nodes       [B] int32, in [1, N].
 *   B, N, V       B >= 0, 1 <= N <= SPEC_MAX_TREE, V >= 1.
 *   out_tokens    [B, N] out: the d accepted tokens along the path, then the
 *                 argmax after the path, then -1.
 *   path_nodes    [B, N] out: the d node indices of the path (root excluded),
 *                 then -1.
 *   num_accepted  [B] out: d, the depth of the kept node.
 * Memory, errors, alignment and streams as for spec_verify: a sequence with a
 * bad status gets num_accepted = 0 and out_tokens / path_nodes all -1.
 */
int spec_verify_tree(const void *target_logits, int32_t dtype, const int32_t *parents,
                     const int32_t *tokens, const int32_t *n_nodes, int32_t B, int32_t N,
                     int32_t V, int32_t *out_tokens, int32_t *path_nodes, int32_t *num_accepted,
                     const spec_tree_aux_t *aux, void *workspace, size_t workspace_bytes,
                     void *stream);

/* ------------------------------------------------------------------------
 * Prompt-lookup drafting.
 *
 * The model-free drafter that precedes verification on copy-heavy tasks:
 * search the existing context for a recent occurrence of its own last n
 * tokens and propose the tokens that followed it ("Speculative Decoding and
 * the Art of Fast LLM Inference", "n-gram and prompt lookup: no model at
 * all"; techaiinterview.com, "Drafts and limits", n-gram / prompt lookup).
 * Sizes are tried from n_max down to n_min; for a size, the most recent
 * occurrence that ends before the context's last token wins, and up to k of
 * the tokens after it are proposed (fewer if the context ends first). No
 * occurrence at any size proposes nothing.
 * ---------------------------------------------------------------------- */

/* Largest supported n-gram size. */
#define SPEC_MAX_NGRAM 16

/*
 *   contexts      [B, T_max] int32 row-major device memory; row b holds
 *                 context_len[b] tokens (any int32 values), the rest is
 *                 never read.
 *   context_len   [B] int32; a length outside [0, T_max] proposes nothing.
 *   n_min, n_max  1 <= n_min <= n_max <= SPEC_MAX_NGRAM.
 *   k             0 <= k <= SPEC_MAX_K: most tokens proposed.
 *   draft_tokens  [B, k] out: the proposal, then -1 (ready for spec_verify's
 *                 draft_tokens); may be NULL when k == 0.
 *   draft_len     [B] out: proposal length in [0, k] (spec_verify's
 *                 draft_len).
 *   match_n       [B] out or NULL: matched n-gram size, 0 if none.
 *   match_start   [B] out or NULL: start of the matched occurrence, -1 if
 *                 none.
 * One kernel, no workspace; errors and streams as for spec_verify.
 */
int spec_prompt_lookup(const int32_t *contexts, const int32_t *context_len, int32_t B,
                       int32_t T_max, int32_t n_min, int32_t n_max, int32_t k,
                       int32_t *draft_tokens, int32_t *draft_len, int32_t *match_n,
                       int32_t *match_start, void *stream);

/*
 * spec_verify for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, outputs, RNG contract and errors as spec_verify, without
 * the workspace: the library uses a static device array of
 * SPEC_NOALLOC_SCRATCH_BYTES per GPU instead (part of the library's code
 * object, held by every GPU the library runs on until the process ends), and
 * the call allocates nothing -- no hipMalloc or hipFree, no allocating
 * library routine. The first call on a GPU looks up that GPU's address of
 * the array once (hipGetSymbolAddress, with the GPU that owns `stream` made
 * current for the lookup). Sizes whose spec_verify_workspace_size() exceeds
 * SPEC_NOALLOC_SCRATCH_BYTES return SPEC_ESCRATCH and enqueue nothing; the
 * default covers B = 1024, k = 7, V = 128256 bf16 (5.9 MB). Every call on a
 * GPU shares that GPU's array: calls that may overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller.
 * Results are bit-identical to spec_verify's for the same inputs.
 */
#define SPEC_NOALLOC_SCRATCH_BYTES (8u << 20)

int spec_verify_noalloc(const void *target_logits, const void *draft_logits, int32_t dtype,
                        const int32_t *draft_tokens, const int32_t *draft_len,
                        const float *temperature, int32_t B, int32_t k, int32_t V,
                        uint64_t seed, uint32_t seq_base, int32_t *out_tokens,
                        int32_t *num_accepted, const spec_verify_aux_t *aux, void *stream);

/* Static, human-readable text for a spec_status_t value. */
const char *spec_verify_strerror(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int spec_verify_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
