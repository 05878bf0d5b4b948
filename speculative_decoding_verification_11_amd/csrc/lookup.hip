// lookup.hip -- prompt-lookup drafting on MI355X (gfx950): the C ABI
// spec_prompt_lookup and its kernel.
#include "common.h"

namespace {

using namespace spv;

// ===========================================================================
// Prompt-lookup drafting: search the context for a recent occurrence of its
// own last n tokens and propose the tokens that followed it ("Speculative
// Decoding and the Art of Fast LLM Inference", "n-gram and prompt lookup: no
// model at all"; techaiinterview.com, "Drafts and limits"). Sizes are tried
// from n_max down to n_min; for a size the most recent occurrence ending
// before the last token wins.
//
// One workgroup per context. For every candidate end position e < T - 1 the
// lane finds m(e), the number of tokens ending at e that equal the
// context's last tokens (capped at n_max). The answer is the largest
// (min(m(e), n_max), e) with m(e) >= n_min: the largest size that matches
// anywhere, then its latest end. The candidates are scanned from the end of
// the context in blocks of kLookupBlock ends; once a block holds a match of
// size n_max nothing earlier can win (same size, earlier end), so the scan
// stops there, and a context that repeats itself is read only near its end.
// ===========================================================================
constexpr int kLookupThreads = 512;  // lanes per context
constexpr int kLookupWaves = kLookupThreads / kWave;
constexpr int kLookupUnroll = 8;     // context loads in flight per lane
constexpr int kLookupBlock = kLookupThreads * kLookupUnroll;

__global__ __launch_bounds__(kLookupThreads) void k_prompt_lookup(
    const int32_t *__restrict__ contexts, const int32_t *__restrict__ ctx_len, int32_t T_max,
    int32_t n_min, int32_t n_max, int32_t k, int32_t *__restrict__ draft_tokens,
    int32_t *__restrict__ draft_len, int32_t *__restrict__ match_n,
    int32_t *__restrict__ match_start)
{
    __shared__ uint64_t best_w[kLookupWaves];
    __shared__ int32_t tail[kMaxNgram];  // tail[j] = ctx[T - 1 - j]
    const int64_t b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int T = ctx_len[b];
    const bool valid = T >= 0 && T <= T_max;
    const int32_t *ctx = contexts + b * (int64_t)T_max;

    if (tid < kMaxNgram)
        tail[tid] = valid && tid < n_max && tid < T ? ctx[T - 1 - tid] : 0;
    __syncthreads();
    const int32_t last = tail[0];

    // Candidate ends e in [0, T - 2]; key = (size << 32) | e, 0 = none.
    uint64_t key = 0;
    const int e_end = valid ? T - 1 : 0;
    for (int hi = e_end; hi > 0; hi -= kLookupBlock) {
        const int lo = hi - kLookupBlock;  // ends [max(lo, 0), hi)
        int32_t c[kLookupUnroll];
#pragma unroll
        for (int u = 0; u < kLookupUnroll; ++u) {
            const int e = lo + u * kLookupThreads + tid;
            c[u] = e >= 0 ? ctx[e] : 0;
        }
#pragma unroll
        for (int u = 0; u < kLookupUnroll; ++u) {
            const int e = lo + u * kLookupThreads + tid;
            if (e >= 0 && c[u] == last) {
                int m = 1;
                const int cap = min(n_max, e + 1);
                while (m < cap && ctx[e - m] == tail[m])
                    ++m;
                if (m >= n_min) {
                    const uint64_t kk = ((uint64_t)m << 32) | (uint32_t)e;
                    key = kk > key ? kk : key;
                }
            }
        }
        if (__syncthreads_or((int)(key >> 32) >= n_max))
            break;  // a full-size match: nothing earlier can win
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        const uint64_t o = __shfl_xor(key, off, kWave);
        key = o > key ? o : key;
    }
    if (lane == 0)
        best_w[wave] = key;
    __syncthreads();
    key = best_w[0];
#pragma unroll
    for (int w = 1; w < kLookupWaves; ++w)
        key = best_w[w] > key ? best_w[w] : key;

    int n = (int)(key >> 32);
    const int e = (int)(uint32_t)key;
    if (n < n_min || n > n_max || e < 0 || e >= T - 1)
        n = 0;  // no match (a key only ever holds n in [n_min, n_max], e in [0, T - 2])
    const int len = n > 0 ? min(k, T - 1 - e) : 0;
    for (int j = tid; j < k; j += kLookupThreads)
        draft_tokens[b * (int64_t)k + j] = j < len ? ctx[e + 1 + j] : -1;
    if (tid == 0) {
        draft_len[b] = len;
        if (match_n) match_n[b] = n;
        if (match_start) match_start[b] = n > 0 ? e - n + 1 : -1;
    }
}

}  // namespace

extern "C" int spec_prompt_lookup(const int32_t *contexts, const int32_t *context_len, int32_t B,
                                  int32_t T_max, int32_t n_min, int32_t n_max, int32_t k,
                                  int32_t *draft_tokens, int32_t *draft_len, int32_t *match_n,
                                  int32_t *match_start, void *stream)
{
    if (B < 0 || T_max < 0 || n_min < 1 || n_max < n_min || n_max > SPEC_MAX_NGRAM || k < 0 ||
        k > SPEC_MAX_K || T_max > INT32_MAX - 1)
        return SPEC_EINVAL;
    if (B == 0)
        return SPEC_OK;
    if ((T_max > 0 && !contexts) || !context_len || (k > 0 && !draft_tokens) || !draft_len)
        return SPEC_EINVAL;
    if (!aligned(contexts, 4) || !aligned(context_len, 4) || !aligned(draft_tokens, 4) ||
        !aligned(draft_len, 4) || !aligned(match_n, 4) || !aligned(match_start, 4))
        return SPEC_EINVAL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    for (int64_t b0 = 0; b0 < B; b0 += INT32_MAX / 2) {
        const int64_t nb = std::min<int64_t>((int64_t)B - b0, INT32_MAX / 2);
        hipLaunchKernelGGL(k_prompt_lookup, dim3((unsigned)nb), dim3(kLookupThreads), 0, st,
                           contexts ? contexts + b0 * T_max : nullptr, context_len + b0, T_max,
                           n_min, n_max, k, draft_tokens ? draft_tokens + b0 * k : nullptr,
                           draft_len + b0, match_n ? match_n + b0 : nullptr,
                           match_start ? match_start + b0 : nullptr);
        if (hipGetLastError() != hipSuccess)
            return SPEC_ELAUNCH;
    }
    return SPEC_OK;
}

