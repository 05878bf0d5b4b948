"""Pins of the top-k filter of the oracle, alone and followed by top-p.

Verification has to use the target's own sampling parameters ("Speculative
Decoding and the Art of Fast LLM Inference", "Why It Stays Exact", key
limitation). Reading TK1 (oracle header): keep whole levels (tokens of
equal logit) from the top until they hold at least top_k tokens, so every
token tied with the top_k-th largest logit is kept; renormalise; the draft
row gets the same rule; top_k <= 0 or >= V keeps all; with top-p as well,
top-k comes first and the nucleus is taken on its result. Pinned against:

  - the identity cases and a closed form (top_k = 1 keeps exactly the tied
    maxima);
  - the defining properties, which fix the kept set uniquely (upward closed
    in the logit, at least top_k tokens, dropping its lowest level leaves
    fewer), on random rows with many ties, and brute force over all level
    prefixes;
  - the whole oracle with top_k (and top_k with top_p) against the sampling
    round on rows filtered here, by sorting, from the definitions;
  - losslessness for a top-k-filtered pair, by exact enumeration;
  - planted mistakes.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest
import scipy.special

from conftest import ROOT, bf16_bits, bf16_to_f32

import oracle  # noqa: E402


def _softmax(x, tau=1.0):
    return scipy.special.softmax(np.asarray(x, np.float64) / tau)


def _levels_desc(x):
    return sorted(set(np.asarray(x, np.float64).tolist()), reverse=True)


def _topk_by_sorting(x, p, K):
    """Kept set and filtered row from the definition: the shortest run of
    levels from the top holding at least K tokens."""
    xs = np.asarray(x, np.float64)
    xs = np.where(xs == 0.0, 0.0, xs)
    if K <= 0 or K >= len(xs):
        return np.ones(len(xs), bool), p / p.sum()
    count = 0
    for lv in _levels_desc(xs):
        count += int((xs == lv).sum())
        if count >= K:
            keep = xs >= lv
            return keep, np.where(keep, p, 0.0) / p[keep].sum()
    raise AssertionError("unreachable")


def _nucleus_by_sorting(x, p, tp):
    """The nucleus of an already normalised (possibly filtered) row."""
    xs = np.asarray(x, np.float64)
    xs = np.where(xs == 0.0, 0.0, xs)
    if tp >= 1.0:
        return p
    total, cum = p.sum(), 0.0
    for lv in _levels_desc(xs):
        cum += p[xs == lv].sum()
        if cum >= tp * total:
            keep = xs >= lv
            return np.where(keep, p, 0.0) / p[keep].sum()
    raise AssertionError("unreachable")


def test_identity_cases():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(300).astype(np.float32)
    p = _softmax(x)
    for K in (0, -3, 300, 301, 10**6):
        q, kept, thr = oracle.topk_row(x, p, K)
        assert np.array_equal(q, p) and thr == -np.inf and kept == pytest.approx(1.0, abs=1e-14)


def test_top1_keeps_the_tied_maxima():
    rng = np.random.default_rng(2)
    for trial in range(50):
        V = int(rng.integers(2, 300))
        x = rng.integers(-4, 3, size=V).astype(np.float32)
        nmax = int((x == x.max()).sum())
        p = _softmax(x, 0.9)
        q, kept, thr = oracle.topk_row(x, p, 1)
        assert thr == x.max()
        assert int((q > 0).sum()) == nmax
        np.testing.assert_allclose(q[x == x.max()], 1.0 / nmax, rtol=1e-13)


def test_defining_properties_on_tied_rows():
    rng = np.random.default_rng(3)
    for trial in range(400):
        V = int(rng.integers(1, 250))
        vals = rng.standard_normal(int(rng.integers(1, 15))) * 2
        x = rng.choice(vals, size=V).astype(np.float32)
        p = _softmax(x, float(rng.choice([0.5, 1.0, 1.6])))
        K = int(rng.integers(1, V + 1))
        q, kept, thr = oracle.topk_row(x, p, K)
        keep = q > 0
        xs = x.astype(np.float64)
        if K >= V:
            assert keep.all()
            continue
        assert keep.sum() >= K
        lowest = xs[keep].min()
        assert (keep & (xs > lowest)).sum() < K  # the lowest kept level is needed
        assert all(keep[i] for i in range(V) if xs[i] >= lowest)  # upward closed
        np.testing.assert_allclose(q[keep], p[keep] / p[keep].sum(), rtol=1e-12)
        assert kept == pytest.approx(p[keep].sum(), rel=1e-13)


def test_brute_force_over_level_prefixes():
    rng = np.random.default_rng(4)
    for trial in range(300):
        V = int(rng.integers(1, 40))
        x = rng.integers(-3, 4, size=V).astype(np.float32)
        p = _softmax(x, 0.7)
        K = int(rng.integers(0, V + 2))
        keep, _ = _topk_by_sorting(x, p, K)
        q, _, _ = oracle.topk_row(x, p, K)
        assert np.array_equal(q > 0, keep), (x, K)


def test_whole_oracle_filters_every_row():
    """spec_verify_ref with top_k (and with top_k then top_p) against the
    sampling round on rows filtered here from the definitions."""
    rng = np.random.default_rng(5)
    B, k, V = 6, 3, 96
    t = bf16_bits((rng.standard_normal((B, k + 1, V)) * 2).astype(np.float32))
    d = bf16_bits(bf16_to_f32(t[:, :k]) + rng.standard_normal((B, k, V)).astype(np.float32))
    tv, dv = bf16_to_f32(t), bf16_to_f32(d)
    tau = np.array([0.8, 1.0, 0.6, 1.3, 0.9, 1.1], np.float32)
    top_k = np.array([1, 5, 0, 40, 96, 12], np.int32)
    L = np.array([3, 2, 3, 1, 0, 3], np.int32)
    g = np.zeros((B, k), np.int32)
    for b in range(B):
        for i in range(L[b]):
            g[b, i] = int(np.argmax(dv[b, i]))  # inside every filter of the draft row
    seed = 0x4321
    for top_p in (None, np.array([0.9, 0.5, 0.7, 1.0, 0.8, 0.95], np.float32)):
        res = oracle.spec_verify_ref(t, d, g, L, tau, seed, top_k=top_k, top_p=top_p)
        for b in range(B):
            Lb = int(L[b])

            def filt(x, tau_b):
                pr = _softmax(x, tau_b)
                _, pr = _topk_by_sorting(x, pr, int(top_k[b]))
                if top_p is not None:
                    pr = _nucleus_by_sorting(x, pr, float(top_p[b]))
                return pr

            P = np.stack([filt(tv[b, i], tau[b]) for i in range(Lb + 1)])
            Q = np.stack([filt(dv[b, i], tau[b]) for i in range(Lb)]) if Lb else np.zeros((0, V))
            u = np.zeros(max(Lb, 1))
            v = np.zeros(Lb + 1)
            for i in range(Lb + 1):
                w = oracle.philox4x32_10([i, b, 0, 0], seed)
                if i < Lb:
                    u[i] = oracle.uniform24(int(w[0]))
                v[i] = oracle.uniform24(int(w[1]))
            rr = oracle.round_sampling(P, Q, g[b, :Lb], u[:Lb], v)
            assert res["seq_status"][b] == 0
            assert res["num_accepted"][b] == rr["n"]
            assert list(res["out_tokens"][b, :rr["n"] + 1]) == list(rr["out"][:rr["n"] + 1])
            for i in range(Lb):
                assert res["p_g"][b, i] == pytest.approx(P[i, g[b, i]], rel=1e-12)
                assert res["q_g"][b, i] == pytest.approx(Q[i, g[b, i]], rel=1e-12)


def test_losslessness_for_a_top_k_pair():
    """Speculative sampling with the top-k-filtered pair emits the filtered
    target exactly (enumerated over a uniform grid of (u, v))."""
    from test_oracle_pins import _emitted_by_enumeration

    x = np.array([1.5, 1.5, 0.5, 0.0, -1.0, -2.0], np.float32)
    y = np.array([0.5, 1.8, 1.2, 0.3, -0.5, -2.0], np.float32)
    pf = oracle.topk_row(x, _softmax(x), 3)[0]
    qf = oracle.topk_row(y, _softmax(y), 3)[0]
    assert (pf > 0).sum() == 3 and (qf > 0).sum() == 3
    emitted, _ = _emitted_by_enumeration(oracle, pf, qf, 2**12)
    np.testing.assert_allclose(emitted, pf, atol=2e-3)
    assert emitted[np.where(pf == 0)].sum() == 0


TOPK_MUTATIONS = {
    "strict_count": ("        if (count >= top_k) {", "        if (count > top_k) {"),
    "keeps_next_level": ("        if (count >= top_k) {\n            *thr = it[a].x;",
                         "        if (count >= top_k) {\n            *thr = b < V ? it[b].x : it[a].x;"),
    "not_renormalised": ("        if (ref_logit(row, dtype, (size_t)x) >= *thr)\n            kept += p[x];",
                         "        if (ref_logit(row, dtype, (size_t)x) >= *thr)\n            kept += 0.0 * p[x] + 1.0 / (double)V;"),
    "off_by_one_disable": ("    if (top_k <= 0 || top_k >= V)\n        return total;",
                           "    if (top_k <= 1 || top_k >= V)\n        return total;"),
}


@pytest.mark.parametrize("name", sorted(TOPK_MUTATIONS))
def test_planted_top_k_mistakes_are_caught(tmp_path, name, monkeypatch):
    old, new = TOPK_MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "spec_verify_ref.c")).read()
    assert src.count(old) == 1
    path = tmp_path / "spec_verify_ref.c"
    path.write_text(src.replace(old, new))
    so = str(tmp_path / "lib.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-o", so,
                    str(path), "-lm"], check=True)
    real = oracle._load()
    mut = ctypes.CDLL(so)
    mut.ref_topk_row.argtypes = real.ref_topk_row.argtypes
    mut.ref_topk_row.restype = real.ref_topk_row.restype
    monkeypatch.setattr(oracle, "_lib", mut)
    caught = False
    try:
        test_top1_keeps_the_tied_maxima()
        test_defining_properties_on_tied_rows()
        test_brute_force_over_level_prefixes()
    except AssertionError:
        caught = True
    assert caught, f"mutation {name} was not detected"
