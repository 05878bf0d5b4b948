// tree.hip -- greedy verification of candidate trees on MI355X (gfx950):
// the C ABI spec_verify_tree and its kernels.
#include "common.h"

namespace {

using namespace spv;

// ===========================================================================
// Greedy verification of candidate trees. A tree's node 0 is the root (the
// last committed position); node n >= 1 holds a drafted token and a parent
// with a smaller index; the target row of node n scores the token after
// node n's path ("Speculative Decoding and the Art of Fast LLM Inference",
// "EAGLE: drafting in feature space": a tree of candidate continuations
// verified together; techaiinterview.com, "Drafts and limits"). The pages
// give no sampling rule for trees, so the rule is greedy: a node is
// accepted when its parent is and its token equals the parent's target
// argmax; the round keeps the deepest accepted node (lowest index among
// equals) and emits its path, then its argmax.
// ===========================================================================
struct TreeParams {
    const void *target;
    const int32_t *parents, *tokens, *n_nodes;
    int32_t N, V, nc, B;
    float2 *partials;  // [B][N][nc]: (max logit, lowest index of it)
    int32_t *out_tokens, *path_nodes, *num_accepted, *seq_status, *argmax;
};

// One workgroup per 32 KiB chunk of each node's row.
template <class D>
__global__ __launch_bounds__(kThreads) void k_tree_rowstats(TreeParams p)
{
    using E = typename D::Elem;
    constexpr int64_t CH = chunk_elems<D>();
    __shared__ RowShared sh;
    const uint32_t item = blockIdx.x;  // 32-bit decode: the grid index fits
    const int nc = p.nc, N = p.N;
    const int c = (int)(item % (uint32_t)nc);
    const uint32_t rn = item / (uint32_t)nc;
    const int n = (int)(rn % (uint32_t)N);
    const int64_t b = rn / (uint32_t)N;
    const int nn = p.n_nodes[b];
    if (nn < 1 || nn > N || n >= nn)
        return;  // k_tree_decide reports a bad node count
    const E *row = static_cast<const E *>(p.target) + (b * N + n) * (int64_t)p.V;
    const int64_t s = (int64_t)c * CH;
    const float2 part = chunk_stats<D>(row, s, min64((int64_t)p.V, s + CH), true, 0.f, sh);
    if (threadIdx.x == 0)
        p.partials[item] = part;
}

// One wave per sequence, lane n = node n.
template <class D>
__global__ __launch_bounds__(kThreads) void k_tree_decide(TreeParams p)
{
    const int64_t b = (int64_t)blockIdx.x * kWaves + threadIdx.x / kWave;
    const int lane = (int)(threadIdx.x % kWave);
    if (b >= p.B)
        return;
    const int N = p.N, V = p.V, nc = p.nc;
    const int nn = p.n_nodes[b];
    const bool node = lane < nn && lane < N;
    int status = SPEC_SEQ_OK;
    int par = -1, tok = -1;
    if (nn < 1 || nn > N) {
        status = SPEC_SEQ_BAD_LEN;
    } else {
        if (node && lane > 0) {
            par = p.parents[b * N + lane];
            tok = p.tokens[b * N + lane];
        }
        if (__any(node && lane > 0 && (par < 0 || par >= lane)))
            status = SPEC_SEQ_BAD_TREE;
        else if (__any(node && lane > 0 && (tok < 0 || tok >= V)))
            status = SPEC_SEQ_BAD_TOKEN;
    }
    int amax = -1;
    if (status == SPEC_SEQ_OK && node) {
        const float2 *pp = p.partials + (b * N + lane) * (int64_t)nc;
        ArgMax acc{-INFINITY, INT32_MAX};
        for (int c0 = 0; c0 < nc; c0 += kFoldBatch) {
            float2 t[kFoldBatch];
#pragma unroll
            for (int q = 0; q < kFoldBatch; ++q)
                t[q] = c0 + q < nc ? pp[c0 + q] : make_float2(-INFINITY, __int_as_float(INT32_MAX));
#pragma unroll
            for (int q = 0; q < kFoldBatch; ++q)
                acc = argmax_merge(acc, ArgMax{t[q].x, __float_as_int(t[q].y)});
        }
        amax = acc.i;
    }
    int32_t *out = p.out_tokens + b * N;
    int32_t *path = p.path_nodes + b * N;
    if (status != SPEC_SEQ_OK) {
        if (lane < N) {
            out[lane] = -1;
            path[lane] = -1;
            if (p.argmax) p.argmax[b * N + lane] = -1;
        }
        if (lane == 0) {
            p.num_accepted[b] = 0;
            if (p.seq_status) p.seq_status[b] = status;
        }
        return;
    }
    // Acceptance and depth flow down from the root; a parent's index is
    // smaller than its child's, so nn rounds always settle them.
    // (every lane takes part in each shuffle: a lane that skips one leaves
    // nothing for the lanes that read from it)
    const int pl = par < 0 ? 0 : par;
    const int parent_amax = __shfl(amax, pl, kWave);
    const bool match = node && lane > 0 && tok == parent_amax;
    bool acc = lane == 0;
    int depth = 0;
    for (int r = 1; r < nn; ++r) {
        const bool pa = __shfl((int)acc, pl, kWave) != 0;
        const int pd = __shfl(depth, pl, kWave);
        if (lane > 0 && node) {
            acc = match && pa;
            depth = pd + 1;
        }
    }
    // The deepest accepted node, the lowest index among equals.
    int key = acc ? (depth << 8) | (255 - lane) : -1;
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1)
        key = max(key, __shfl_xor(key, off, kWave));
    const int best = 255 - (key & 255), d = key >> 8;
    // Walk the path from the deepest node up; lane j keeps position j.
    int x = best, mine_tok = -1, mine_node = -1;
    for (int j = d - 1; j >= 0; --j) {
        const int tx = __shfl(tok, x, kWave);
        const int px = __shfl(par, x, kWave);
        if (lane == j) {
            mine_tok = tx;
            mine_node = x;
        }
        x = px;
    }
    const int bonus = __shfl(amax, best, kWave);
    if (lane < N) {
        out[lane] = lane < d ? mine_tok : (lane == d ? bonus : -1);
        path[lane] = lane < d ? mine_node : -1;
        if (p.argmax) p.argmax[b * N + lane] = node ? amax : -1;
    }
    if (lane == 0) {
        p.num_accepted[b] = d;
        if (p.seq_status) p.seq_status[b] = SPEC_SEQ_OK;
    }
}

template <class D>
int launch_tree(const TreeParams &base, const spec_tree_aux_t *aux, char *ws, int nc,
                hipStream_t stream)
{
    const int B = base.B, N = base.N;
    const int64_t per_seq_items = (int64_t)N * nc;
    const int64_t max_items = (int64_t)1 << 22;
    const int64_t slice = std::max<int64_t>(1, max_items / per_seq_items);
    hipEvent_t ev_begin = aux ? static_cast<hipEvent_t>(aux->event_begin) : nullptr;
    hipEvent_t ev_end = aux ? static_cast<hipEvent_t>(aux->event_end) : nullptr;
    for (int64_t b0 = 0; b0 < B; b0 += slice) {
        const int64_t nb = std::min<int64_t>((int64_t)B - b0, slice);
        TreeParams p = base;
        p.B = (int32_t)nb;
        p.nc = nc;
        p.target = static_cast<const typename D::Elem *>(base.target) + b0 * N * (int64_t)base.V;
        p.parents = base.parents + b0 * N;
        p.tokens = base.tokens + b0 * N;
        p.n_nodes = base.n_nodes + b0;
        p.partials = reinterpret_cast<float2 *>(ws);
        p.out_tokens = base.out_tokens + b0 * N;
        p.path_nodes = base.path_nodes + b0 * N;
        p.num_accepted = base.num_accepted + b0;
        if (p.seq_status) p.seq_status += b0;
        if (p.argmax) p.argmax += b0 * N;
        if (ev_begin && b0 == 0 && hipEventRecord(ev_begin, stream) != hipSuccess)
            return SPEC_ELAUNCH;
        hipLaunchKernelGGL(k_tree_rowstats<D>, dim3((unsigned)(nb * per_seq_items)),
                           dim3(kThreads), 0, stream, p);
        if (ev_end && b0 == 0 && hipEventRecord(ev_end, stream) != hipSuccess)
            return SPEC_ELAUNCH;
        hipLaunchKernelGGL(k_tree_decide<D>, dim3((unsigned)((nb + kWaves - 1) / kWaves)),
                           dim3(kThreads), 0, stream, p);
        if (hipGetLastError() != hipSuccess)
            return SPEC_ELAUNCH;
    }
    return SPEC_OK;
}

int tree_nc(int32_t V, int32_t dtype)
{
    const int64_t ch = kChunkBytes / (dtype == SPEC_F32 ? 4 : 2);
    return (int)((V + ch - 1) / ch);
}

bool tree_sizes_ok(int32_t B, int32_t N, int32_t V, int32_t dtype)
{
    return B >= 0 && N >= 1 && N <= SPEC_MAX_TREE && V >= 1 &&
           (dtype == SPEC_F32 || dtype == SPEC_BF16);
}

}  // namespace

extern "C" size_t spec_verify_tree_workspace_size(int32_t B, int32_t N, int32_t V, int32_t dtype)
{
    if (!tree_sizes_ok(B, N, V, dtype))
        return 0;
    const size_t bytes = (size_t)B * (size_t)N * (size_t)tree_nc(V, dtype) * sizeof(float2);
    return bytes == 0 ? 256 : align_up(bytes, 256);
}

extern "C" int spec_verify_tree(const void *target_logits, int32_t dtype, const int32_t *parents,
                                const int32_t *tokens, const int32_t *n_nodes, int32_t B,
                                int32_t N, int32_t V, int32_t *out_tokens, int32_t *path_nodes,
                                int32_t *num_accepted, const spec_tree_aux_t *aux,
                                void *workspace, size_t workspace_bytes, void *stream)
{
    if (!tree_sizes_ok(B, N, V, dtype))
        return SPEC_EINVAL;
    if (B == 0)
        return SPEC_OK;
    const size_t esz = dtype == SPEC_F32 ? 4 : 2;
    if (!target_logits || !parents || !tokens || !n_nodes || !out_tokens || !path_nodes ||
        !num_accepted)
        return SPEC_EINVAL;
    if (!aligned(target_logits, esz) || !aligned(parents, 4) || !aligned(tokens, 4) ||
        !aligned(n_nodes, 4) || !aligned(out_tokens, 4) || !aligned(path_nodes, 4) ||
        !aligned(num_accepted, 4) || (aux && aux->seq_status && !aligned(aux->seq_status, 4)) ||
        (aux && aux->argmax && !aligned(aux->argmax, 4)))
        return SPEC_EINVAL;
    if (!workspace || !aligned(workspace, 256) ||
        workspace_bytes < spec_verify_tree_workspace_size(B, N, V, dtype))
        return SPEC_EWORKSPACE;
    TreeParams p{};
    p.target = target_logits;
    p.parents = parents;
    p.tokens = tokens;
    p.n_nodes = n_nodes;
    p.N = N;
    p.V = V;
    p.B = B;
    p.out_tokens = out_tokens;
    p.path_nodes = path_nodes;
    p.num_accepted = num_accepted;
    p.seq_status = aux ? aux->seq_status : nullptr;
    p.argmax = aux ? aux->argmax : nullptr;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    const int nc = tree_nc(V, dtype);
    if (dtype == SPEC_F32)
        return launch_tree<F32>(p, aux, ws, nc, st);
    return launch_tree<BF16>(p, aux, ws, nc, st);
}

