"""fp64 CPU oracle for the speculative-sampling verification step.

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package. The HIP library
and its Python binding never import it, and it never imports them: the two
share no code. The arithmetic lives in ``spec_verify_ref.c`` (plain C, fp64,
scalar loops); this module only builds it with gcc and marshals numpy arrays.

Parity status of each function (what pins it is in the tests):
  softmax_row          pinned: scipy/torch fp64 softmax, closed forms
  argmax_row           pinned: numpy.argmax (first occurrence) on planted ties
  philox4x32_10        pinned: rocRAND's Philox4x32-10 engine (compiled host-side)
  draw_inverse_cdf     pinned: brute-force interval membership on small cases
  round_sampling       pinned: red/blue example, exact enumeration, forced rounds
  round_greedy         pinned: worked rounds, argmax agreement by hand
  spec_verify_ref      pinned: chi-square of emitted tokens against p, accepted
                       length against the closed form, worked rounds
  nucleus_row          pinned: brute force over level prefixes, closed forms
                       (uniform and two-level rows), top_p = 1 is the identity,
                       planted mistakes
  tree_greedy          pinned: chain trees equal round_greedy; brute-force path
                       enumeration; a hand-worked tree; planted mistakes
  spec_tree_ref        pinned: argmax_row per node + tree_greedy, statuses
  prompt_lookup        pinned: brute force over all windows, hand-worked
                       contexts, invariants, planted mistakes
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spec_verify_ref.c")
_LIB = os.path.join(_HERE, "_build", "libspecverify_oracle.so")

F32 = 0
BF16 = 1

SEQ_OK, SEQ_BAD_TOKEN, SEQ_BAD_LEN, SEQ_BAD_TEMP, SEQ_QZERO, SEQ_BAD_TREE, SEQ_BAD_TOP_P = range(7)
DRAW_NONE, DRAW_GREEDY, DRAW_RESIDUAL, DRAW_BONUS, DRAW_RESIDUAL_AS_P = range(5)

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.ref_softmax_row.argtypes = [P, ctypes.c_int, ctypes.c_int64, ctypes.c_double, P]
        lib.ref_softmax_row.restype = None
        lib.ref_argmax_row.argtypes = [P, ctypes.c_int, ctypes.c_int64]
        lib.ref_argmax_row.restype = ctypes.c_int64
        lib.ref_philox4x32_10.argtypes = [P, ctypes.c_uint64, P]
        lib.ref_philox4x32_10.restype = None
        lib.ref_uniform24.argtypes = [ctypes.c_uint32]
        lib.ref_uniform24.restype = ctypes.c_double
        lib.ref_draw_inverse_cdf.argtypes = [P, ctypes.c_int64, ctypes.c_double, P, P, P]
        lib.ref_draw_inverse_cdf.restype = ctypes.c_int64
        lib.ref_round_sampling.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int64, P, P, P, P,
                                           P, P, P, P, P, P]
        lib.ref_round_sampling.restype = ctypes.c_int
        lib.ref_round_greedy.argtypes = [P, P, ctypes.c_int, P]
        lib.ref_round_greedy.restype = ctypes.c_int
        lib.spec_verify_ref.argtypes = [P, P, ctypes.c_int, P, P, P, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                        ctypes.c_uint32] + [P] * 11
        lib.spec_verify_ref.restype = ctypes.c_int
        lib.ref_nucleus_row.argtypes = [P, ctypes.c_int, ctypes.c_int64, ctypes.c_double, P, P, P]
        lib.ref_nucleus_row.restype = ctypes.c_double
        lib.spec_verify_topp_ref.argtypes = [P, P, ctypes.c_int, P, P, P, P, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                             ctypes.c_uint32] + [P] * 12
        lib.spec_verify_topp_ref.restype = ctypes.c_int
        lib.ref_topk_row.argtypes = [P, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, P, P]
        lib.ref_topk_row.restype = ctypes.c_double
        lib.spec_verify_filter_ref.argtypes = [P, P, ctypes.c_int, P, P, P, P, P, ctypes.c_int32,
                                               ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                               ctypes.c_uint32] + [P] * 12
        lib.spec_verify_filter_ref.restype = ctypes.c_int
        lib.spec_verify_full_ref.argtypes = [P, P, ctypes.c_int, P, P, P, P, P, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                             ctypes.c_uint32] + [P] * 12 + [ctypes.c_double, P, P]
        lib.spec_verify_full_ref.restype = ctypes.c_int
        lib.ref_draw_band.argtypes = [P, P, ctypes.c_int64, ctypes.c_double, ctypes.c_double]
        lib.ref_draw_band.restype = ctypes.c_double
        lib.ref_draw_window.argtypes = [P, ctypes.c_int64, ctypes.c_double, ctypes.c_double, P, P]
        lib.ref_draw_window.restype = None
        lib.ref_tree_greedy.argtypes = [P, P, P, ctypes.c_int, P, P]
        lib.ref_tree_greedy.restype = ctypes.c_int
        lib.spec_tree_ref.argtypes = [P, ctypes.c_int, P, P, P, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int64, P, P, P, P, P]
        lib.spec_tree_ref.restype = ctypes.c_int
        lib.ref_prompt_lookup.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, P, P, P]
        lib.ref_prompt_lookup.restype = ctypes.c_int
        lib.spec_prompt_lookup_ref.argtypes = [P, P, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                               P, P, P, P]
        lib.spec_prompt_lookup_ref.restype = None
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _logits(a: np.ndarray):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError("logits must be float32 or uint16 (bf16 bit patterns)")


def softmax_row(row: np.ndarray, tau: float) -> np.ndarray:
    row, dt = _logits(row)
    out = np.empty(row.shape[-1], dtype=np.float64)
    _load().ref_softmax_row(_ptr(row), dt, row.shape[-1], float(tau), _ptr(out))
    return out


def argmax_row(row: np.ndarray) -> int:
    row, dt = _logits(row)
    return int(_load().ref_argmax_row(_ptr(row), dt, row.shape[-1]))


def philox4x32_10(counter, seed: int) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(counter, dtype=np.uint32).reshape(4))
    out = np.empty(4, dtype=np.uint32)
    _load().ref_philox4x32_10(_ptr(c), ctypes.c_uint64(seed & (2**64 - 1)), _ptr(out))
    return out


def uniform24(word: int) -> float:
    return float(_load().ref_uniform24(ctypes.c_uint32(word)))


def draw_inverse_cdf(w: np.ndarray, v: float):
    """Returns (token, S, margin, fallback)."""
    w = np.ascontiguousarray(w, dtype=np.float64)
    S = np.zeros(1)
    m = np.zeros(1)
    fb = np.zeros(1, dtype=np.int32)
    x = _load().ref_draw_inverse_cdf(_ptr(w), w.shape[0], float(v), _ptr(S), _ptr(m), _ptr(fb))
    return int(x), float(S[0]), float(m[0]), bool(fb[0])


def draw_window(w: np.ndarray, v: float, band: float):
    """Smallest and largest ids an inverse-CDF draw from weights ``w`` could
    return with its uniform moved by at most ``band`` (-1, -1 if sum w <= 0)."""
    w = np.ascontiguousarray(w, dtype=np.float64)
    lo = ctypes.c_int64(0)
    hi = ctypes.c_int64(0)
    _load().ref_draw_window(_ptr(w), w.shape[0], float(v), float(band), ctypes.byref(lo),
                            ctypes.byref(hi))
    return int(lo.value), int(hi.value)


def draw_band(p: np.ndarray, q, S: float, band: float) -> float:
    """Flag band of a draw from max(0, p - q) (q None: from p) of mass S:
    ``band``, or 8 * 2^-24 * sqrt(sum max(p, q)^2) / S where that is larger
    (the fp32 resolution of the draw's CDF)."""
    p = np.ascontiguousarray(p, dtype=np.float64)
    qq = None if q is None else np.ascontiguousarray(q, dtype=np.float64)
    return float(_load().ref_draw_band(_ptr(p), None if qq is None else _ptr(qq), p.shape[0],
                                       float(S), float(band)))


def nucleus_row(row: np.ndarray, p: np.ndarray, top_p: float):
    """Nucleus filter of one row (reading TP1). row: the logits; p: their
    softmax. Returns (filtered p, kept mass, threshold logit, margin)."""
    row, dt = _logits(row)
    q = np.ascontiguousarray(np.asarray(p, dtype=np.float64)).copy()
    thr = np.zeros(1)
    mg = np.zeros(1)
    kept = _load().ref_nucleus_row(_ptr(row), dt, row.shape[-1], float(top_p), _ptr(q), _ptr(thr),
                                   _ptr(mg))
    return q, float(kept), float(thr[0]), float(mg[0])


def topk_row(row: np.ndarray, p: np.ndarray, top_k: int):
    """Top-k filter of one row (reading TK1). row: the logits; p: their
    softmax (or an already filtered row). Returns (filtered p, kept mass,
    threshold logit)."""
    row, dt = _logits(row)
    q = np.ascontiguousarray(np.asarray(p, dtype=np.float64)).copy()
    thr = np.zeros(1)
    kept = _load().ref_topk_row(_ptr(row), dt, row.shape[-1], int(top_k), _ptr(q), _ptr(thr))
    return q, float(kept), float(thr[0])


def round_sampling(p: np.ndarray, q: np.ndarray, g, u, v):
    """One sampling round from explicit probabilities and uniforms.

    p: [L+1, V], q: [L, V], g: [L], u: [L], v: [L+1].
    Returns dict(n, out, S, row, kind, margin_accept, margin_draw, status).
    """
    p = np.ascontiguousarray(p, dtype=np.float64)
    L = p.shape[0] - 1
    V = p.shape[1]
    n_pad = max(L, 1)  # C side never reads q, g, u when L == 0
    qa = np.zeros((n_pad, V))
    ga = np.zeros(n_pad, dtype=np.int32)
    ua = np.zeros(n_pad)
    if L:
        qa[:L] = np.asarray(q, dtype=np.float64).reshape(L, V)
        ga[:L] = np.asarray(g, dtype=np.int32).reshape(L)
        ua[:L] = np.asarray(u, dtype=np.float64).reshape(L)
    q, g, u = qa, ga, ua
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float64).reshape(L + 1))
    w = np.empty(V)
    out = np.full(L + 1, -1, dtype=np.int32)
    S = np.full(1, np.nan)
    row = np.full(1, -1, dtype=np.int32)
    kind = np.zeros(1, dtype=np.int32)
    macc = np.full(n_pad, np.nan)
    mdraw = np.full(1, np.nan)
    status = np.zeros(1, dtype=np.int32)
    n = _load().ref_round_sampling(_ptr(p), _ptr(q), _ptr(g), L, V, _ptr(u), _ptr(v), _ptr(w),
                                   _ptr(out), _ptr(S), _ptr(row), _ptr(kind), _ptr(macc),
                                   _ptr(mdraw), _ptr(status))
    return dict(n=int(n), out=out, S=float(S[0]), row=int(row[0]), kind=int(kind[0]),
                margin_accept=macc[:L], margin_draw=float(mdraw[0]), status=int(status[0]))


def round_greedy(amax, g):
    amax = np.ascontiguousarray(np.asarray(amax, dtype=np.int64))
    L = amax.shape[0] - 1
    ga = np.zeros(max(L, 1), dtype=np.int32)
    if L:
        ga[:L] = np.asarray(g, dtype=np.int32).reshape(L)
    g = ga
    out = np.full(L + 1, -1, dtype=np.int32)
    n = _load().ref_round_greedy(_ptr(amax), _ptr(g), L, _ptr(out))
    return int(n), out


def spec_verify_ref(target: np.ndarray, draft: np.ndarray, draft_tokens: np.ndarray,
                    draft_len, temperature, seed: int, seq_base: int = 0,
                    nthreads: int = 1, top_p=None, top_k=None, band: float = 1e-6) -> dict:
    """The whole step on host arrays (see spec_verify_ref.c for the contract).

    target [B, k+1, V] and draft [B, k, V] are float32 or uint16 (bf16 bits).
    ``nthreads`` > 1 runs disjoint slices of sequences in parallel threads;
    each slice keeps its global sequence index, so results do not change.
    ``top_p`` (fp32) and ``top_k`` (int32), scalars or [B], filter every
    sampling row (readings TP1, TK1); ``margin_nucleus`` is returned with
    ``top_p``. ``band_draw`` [B]: the final draw's flag band, ``band`` or
    wider where fp32 weights cannot resolve the draw (ref_draw_band; NaN
    where no token was sampled). ``draw_window`` [B, 2]: the token ids the
    final draw could select with its uniform moved by at most that band (-1
    where no token was sampled).
    """
    target, dt = _logits(target)
    draft, dt2 = _logits(draft)
    assert dt == dt2, "target and draft must share a dtype"
    B, k1, V = target.shape
    k = k1 - 1
    assert draft.shape == (B, k, V), (draft.shape, (B, k, V))
    tokens = np.ascontiguousarray(np.asarray(draft_tokens, dtype=np.int32).reshape(B, k))
    if draft_len is None:
        lens = None
    else:
        lens = np.ascontiguousarray(np.asarray(draft_len, dtype=np.int32).reshape(B))
    temp = np.asarray(temperature, dtype=np.float32)
    temp = np.ascontiguousarray(np.broadcast_to(temp, (B,)).copy())
    tp = None
    if top_p is not None:
        tp = np.ascontiguousarray(np.broadcast_to(np.asarray(top_p, dtype=np.float32), (B,)).copy())
    tk = None
    if top_k is not None:
        tk = np.ascontiguousarray(np.broadcast_to(np.asarray(top_k, dtype=np.int32), (B,)).copy())

    res = dict(
        out_tokens=np.full((B, k + 1), -1, dtype=np.int32),
        num_accepted=np.zeros(B, dtype=np.int32),
        seq_status=np.zeros(B, dtype=np.int32),
        p_g=np.full((B, k), np.nan),
        q_g=np.full((B, k), np.nan),
        argmax=np.full((B, k + 1), -1, dtype=np.int32),
        resid_mass=np.full(B, np.nan),
        margin_accept=np.full((B, k), np.nan),
        margin_draw=np.full(B, np.nan),
        draw_row=np.full(B, -1, dtype=np.int32),
        draw_kind=np.zeros(B, dtype=np.int32),
        draw_window=np.full((B, 2), -1, dtype=np.int32),
        band_draw=np.full(B, np.nan),
    )
    if tp is not None:
        res["margin_nucleus"] = np.full((B, 2 * k + 1), np.nan)
    lib = _load()

    def run(b0: int, b1: int) -> int:
        if b1 <= b0:
            return 0
        sl = slice(b0, b1)
        mn = res["margin_nucleus"][sl] if tp is not None else None
        outs = [res[n][sl] for n in ("out_tokens", "num_accepted", "seq_status", "p_g", "q_g",
                                     "argmax", "resid_mass", "margin_accept", "margin_draw")]
        return lib.spec_verify_full_ref(
            _ptr(target[sl]), _ptr(draft[sl]), dt, _ptr(tokens[sl]),
            _ptr(lens[sl]) if lens is not None else None, _ptr(temp[sl]),
            _ptr(tk[sl]) if tk is not None else None, _ptr(tp[sl]) if tp is not None else None,
            b1 - b0, k, V, ctypes.c_uint64(seed & (2**64 - 1)),
            ctypes.c_uint32((seq_base + b0) & 0xFFFFFFFF), *[_ptr(o) for o in outs],
            _ptr(mn) if mn is not None else None, _ptr(res["draw_row"][sl]),
            _ptr(res["draw_kind"][sl]), float(band), _ptr(res["draw_window"][sl]),
            _ptr(res["band_draw"][sl]))

    if nthreads <= 1 or B <= 1:
        rc = run(0, B)
        if rc != 0:
            raise MemoryError("oracle scratch allocation failed")
    else:
        step = (B + nthreads - 1) // nthreads
        with ThreadPoolExecutor(max_workers=nthreads) as ex:
            rcs = list(ex.map(lambda b0: run(b0, min(B, b0 + step)), range(0, B, step)))
        if any(rcs):
            raise MemoryError("oracle scratch allocation failed")
    return res


def tree_greedy(amax, parents, tokens):
    """Greedy verification of one candidate tree from per-node argmaxes.
    Returns (d, out[0..d], path[0..d-1])."""
    amax = np.ascontiguousarray(np.asarray(amax, dtype=np.int64))
    n = amax.shape[0]
    par = np.ascontiguousarray(np.asarray(parents, dtype=np.int32).reshape(n))
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(n))
    out = np.full(n, -1, dtype=np.int32)
    path = np.full(n, -1, dtype=np.int32)
    d = _load().ref_tree_greedy(_ptr(amax), _ptr(par), _ptr(tok), n, _ptr(out), _ptr(path))
    if d < 0:
        raise MemoryError("oracle scratch allocation failed")
    return int(d), out[:d + 1].copy(), path[:d].copy()


def spec_tree_ref(target: np.ndarray, parents: np.ndarray, tokens: np.ndarray, n_nodes,
                  nthreads: int = 1) -> dict:
    """Greedy tree verification of a batch on host arrays (see spec_tree_ref
    in spec_verify_ref.c). target [B, N, V] float32 or uint16 (bf16 bits)."""
    target, dt = _logits(target)
    B, N, V = target.shape
    par = np.ascontiguousarray(np.asarray(parents, dtype=np.int32).reshape(B, N))
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(B, N))
    nn = np.ascontiguousarray(np.asarray(n_nodes, dtype=np.int32).reshape(B))
    res = dict(out_tokens=np.full((B, N), -1, dtype=np.int32),
               path_nodes=np.full((B, N), -1, dtype=np.int32),
               num_accepted=np.zeros(B, dtype=np.int32),
               seq_status=np.zeros(B, dtype=np.int32),
               argmax=np.full((B, N), -1, dtype=np.int32))
    lib = _load()

    def run(b0: int, b1: int) -> int:
        if b1 <= b0:
            return 0
        sl = slice(b0, b1)
        return lib.spec_tree_ref(_ptr(target[sl]), dt, _ptr(par[sl]), _ptr(tok[sl]), _ptr(nn[sl]),
                                 b1 - b0, N, V, *[_ptr(res[k][sl]) for k in (
                                     "out_tokens", "path_nodes", "num_accepted", "seq_status",
                                     "argmax")])

    step = max(1, (B + max(1, nthreads) - 1) // max(1, nthreads))
    with ThreadPoolExecutor(max_workers=max(1, nthreads)) as ex:
        rcs = list(ex.map(lambda b0: run(b0, min(B, b0 + step)), range(0, B, step)))
    if any(rcs):
        raise MemoryError("oracle scratch allocation failed")
    return res


def prompt_lookup(ctx, n_min: int, n_max: int, k: int):
    """Prompt-lookup proposal for one context. Returns (tokens, match_n, match_s)."""
    c = np.ascontiguousarray(np.asarray(ctx, dtype=np.int32).reshape(-1))
    T = c.shape[0]
    buf = c if T else np.zeros(1, dtype=np.int32)
    d = np.full(max(k, 1), -1, dtype=np.int32)
    mn = ctypes.c_int(0)
    ms = ctypes.c_int(-1)
    n = _load().ref_prompt_lookup(_ptr(buf), T, n_min, n_max, k, _ptr(d), ctypes.byref(mn),
                                  ctypes.byref(ms))
    return d[:n].copy(), int(mn.value), int(ms.value)


def spec_prompt_lookup_ref(contexts: np.ndarray, ctx_len, n_min: int, n_max: int, k: int) -> dict:
    """Prompt lookup for a batch: contexts [B, T_max] int32, ctx_len [B]."""
    c = np.ascontiguousarray(np.asarray(contexts, dtype=np.int32))
    B, T_max = c.shape
    lens = np.ascontiguousarray(np.asarray(ctx_len, dtype=np.int32).reshape(B))
    res = dict(draft_tokens=np.full((B, max(k, 0)), -1, dtype=np.int32),
               draft_len=np.zeros(B, dtype=np.int32), match_n=np.zeros(B, dtype=np.int32),
               match_s=np.full(B, -1, dtype=np.int32))
    if B == 0:
        return res
    dt = res["draft_tokens"] if k > 0 else np.zeros((B, 1), dtype=np.int32)
    _load().spec_prompt_lookup_ref(_ptr(c), _ptr(lens), B, T_max, n_min, n_max, k, _ptr(dt),
                                   _ptr(res["draft_len"]), _ptr(res["match_n"]),
                                   _ptr(res["match_s"]))
    return res
