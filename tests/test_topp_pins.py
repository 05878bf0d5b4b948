"""Pins of the top-p (nucleus) filter of the oracle.

The pages only require that verification use the target's own sampling
parameters, temperature and top-p ("Speculative Decoding and the Art of Fast
LLM Inference", "Why It Stays Exact", key limitation). Reading TP1 (oracle
header): keep whole probability levels (tokens of equal logit) from the top
until their mass reaches top_p of the row, renormalise, apply the same rule
to the draft row. Pinned against:

  - top_p = 1: the identity;
  - closed forms: a uniform row is one level (always kept whole); a
    two-level row keeps the top level alone iff its mass reaches top_p;
  - the defining properties, which fix the kept set uniquely: upward
    closed in the logit, mass >= top_p, and dropping its lowest level falls
    below top_p -- checked on random rows with many ties, and by brute force
    over all level prefixes;
  - the whole oracle with top_p against the sampling round run on the
    explicitly filtered rows;
  - losslessness for the filtered pair: exact enumeration of the emitted
    distribution equals the filtered target;
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


def test_top_p_one_is_the_identity():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(300).astype(np.float32)
    p = _softmax(x)
    q, kept, thr, mg = oracle.nucleus_row(x, p, 1.0)
    assert np.array_equal(q, p) and thr == -np.inf and np.isnan(mg)


def test_closed_forms():
    # uniform row: a single level, kept whole for every top_p
    x = np.full(50, 0.25, np.float32)
    p = _softmax(x)
    for tp in (1e-6, 0.3, 0.999):
        q, kept, thr, _ = oracle.nucleus_row(x, p, tp)
        np.testing.assert_allclose(q, np.full(50, 1 / 50), rtol=1e-14)
        assert thr == np.float32(0.25)
    # two levels: a tokens at ln 4, b tokens at 0 -> top level mass 4a/(4a+b)
    a, b = 3, 9
    x = np.array([np.log(4)] * a + [0.0] * b, np.float32)
    p = _softmax(x)
    m_top = p[:a].sum()
    q, kept, thr, mg = oracle.nucleus_row(x, p, m_top * (1 - 1e-9))
    np.testing.assert_allclose(q[:a], 1 / a, rtol=1e-12)
    assert (q[a:] == 0).all() and kept == pytest.approx(m_top, rel=1e-15)
    q, kept, thr, mg = oracle.nucleus_row(x, p, m_top * (1 + 1e-9))
    np.testing.assert_allclose(q, p / p.sum(), rtol=1e-12)
    assert thr == 0.0
    # a level that reaches top_p exactly (dyadic masses) ends the nucleus
    x = np.array([2.0, 1.0, 0.0], np.float32)
    q, kept, thr, mg = oracle.nucleus_row(x, np.array([0.5, 0.25, 0.25]), 0.75)
    assert list(q) == [2 / 3, 1 / 3, 0.0] and kept == 0.75 and thr == 1.0 and mg == 0.0


def _check_properties(x, p, tp, q, thr):
    xs = x.astype(np.float64)
    kept = xs >= thr
    total = p.sum()
    mass = p[kept].sum()
    assert mass >= tp * total * (1 - 1e-12)
    lowest = xs[kept].min()
    assert p[kept & (xs > lowest)].sum() < tp * total * (1 + 1e-12)
    # upward closed; proportional to p; normalised
    assert all(kept[i] for i in range(len(xs)) if xs[i] > lowest)
    np.testing.assert_allclose(q[kept], p[kept] / mass, rtol=1e-12)
    assert (q[~kept] == 0).all()
    assert q.sum() == pytest.approx(1.0, abs=1e-12)


def test_defining_properties_on_tied_rows():
    rng = np.random.default_rng(2)
    for trial in range(400):
        V = int(rng.integers(1, 200))
        vals = rng.standard_normal(int(rng.integers(1, 12))) * 2
        x = rng.choice(vals, size=V).astype(np.float32)
        tau = float(rng.choice([0.5, 1.0, 1.7]))
        p = _softmax(x, tau)
        tp = float(rng.uniform(0.01, 0.999))
        q, kept, thr, mg = oracle.nucleus_row(x, p, tp)
        _check_properties(x, p, tp, q, thr)


def test_brute_force_over_level_prefixes():
    rng = np.random.default_rng(3)
    for trial in range(300):
        V = int(rng.integers(1, 40))
        x = rng.integers(-3, 4, size=V).astype(np.float32)
        p = _softmax(x, 0.7)
        tp = float(rng.uniform(0.05, 0.99))
        levels = sorted(set(x.tolist()), reverse=True)
        best = None
        for cut in range(1, len(levels) + 1):  # shortest prefix of levels reaching tp
            sel = np.isin(x, levels[:cut])
            if p[sel].sum() >= tp * p.sum():
                best = sel
                break
        q, kept, thr, mg = oracle.nucleus_row(x, p, tp)
        assert np.array_equal(q > 0, best)


def test_whole_oracle_filters_every_row():
    rng = np.random.default_rng(4)
    B, k, V = 5, 3, 64
    t = bf16_bits((rng.standard_normal((B, k + 1, V)) * 2).astype(np.float32))
    d = bf16_bits(bf16_to_f32(t[:, :k]) + rng.standard_normal((B, k, V)).astype(np.float32))
    tv, dv = bf16_to_f32(t), bf16_to_f32(d)
    tau = np.array([0.8, 1.0, 0.6, 1.3, 0.9], np.float32)
    top_p = np.array([0.9, 0.5, 1.0, 0.75, 0.95], np.float32)
    L = np.array([3, 2, 3, 1, 0], np.int32)
    g = np.zeros((B, k), np.int32)
    for b in range(B):
        for i in range(L[b]):
            g[b, i] = int(np.argmax(dv[b, i]))  # the draft's top token is in its nucleus
    seed = 0x1234
    res = oracle.spec_verify_ref(t, d, g, L, tau, seed, top_p=top_p)
    for b in range(B):
        Lb = int(L[b])
        P = np.stack([oracle.nucleus_row(t[b, i], oracle.softmax_row(t[b, i], tau[b]),
                                         top_p[b])[0] for i in range(Lb + 1)])
        Q = np.stack([oracle.nucleus_row(d[b, i], oracle.softmax_row(d[b, i], tau[b]),
                                         top_p[b])[0] for i in range(Lb)]) if Lb else np.zeros((0, V))
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
            assert res["p_g"][b, i] == P[i, g[b, i]] and res["q_g"][b, i] == Q[i, g[b, i]]
        filtered = top_p[b] < 1
        assert np.isnan(res["margin_nucleus"][b, 0]) != filtered


def test_losslessness_for_a_filtered_pair():
    """Speculative sampling with the filtered pair emits the filtered target
    exactly (enumerated over a uniform grid of (u, v))."""
    from test_oracle_pins import _emitted_by_enumeration

    x = np.array([1.5, 1.5, 0.5, 0.0, -1.0, -2.0], np.float32)
    y = np.array([0.5, 1.8, 1.2, 0.3, -0.5, -2.0], np.float32)
    pf = oracle.nucleus_row(x, _softmax(x), 0.8)[0]
    qf = oracle.nucleus_row(y, _softmax(y), 0.8)[0]
    emitted, _ = _emitted_by_enumeration(oracle, pf, qf, 2**12)
    np.testing.assert_allclose(emitted, pf, atol=2e-3)
    assert emitted[np.where(pf == 0)].sum() == 0


TOPP_MUTATIONS = {
    "strict_crossing": ("if (cum >= target) {", "if (cum > target) {"),
    "not_renormalised": ("    free(it);\n    for (int64_t x = 0; x < V; x++) {\n"
                         "        double lx = ref_logit(row, dtype, (size_t)x);\n"
                         "        p[x] = lx >= *thr ? p[x] / kept : 0.0;",
                         "    free(it);\n    for (int64_t x = 0; x < V; x++) {\n"
                         "        double lx = ref_logit(row, dtype, (size_t)x);\n"
                         "        p[x] = lx >= *thr ? p[x] : 0.0;"),
    "ties_cut": ("        while (b < V && it[b].x == it[a].x)\n            level += p[it[b++].i];",
                 "        while (b < V && b == a)\n            level += p[it[b++].i];"),
    "lowest_first": ("return u->x > v->x ? -1 : 1;", "return u->x < v->x ? -1 : 1;"),
}


@pytest.mark.parametrize("name", sorted(TOPP_MUTATIONS))
def test_planted_top_p_mistakes_are_caught(tmp_path, name, monkeypatch):
    old, new = TOPP_MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "spec_verify_ref.c")).read()
    assert src.count(old) == 1
    path = tmp_path / "spec_verify_ref.c"
    path.write_text(src.replace(old, new))
    so = str(tmp_path / "lib.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-o", so,
                    str(path), "-lm"], check=True)
    real = oracle._load()
    mut = ctypes.CDLL(so)
    mut.ref_nucleus_row.argtypes = real.ref_nucleus_row.argtypes
    mut.ref_nucleus_row.restype = real.ref_nucleus_row.restype
    monkeypatch.setattr(oracle, "_lib", mut)
    caught = False
    try:
        test_closed_forms()
        test_defining_properties_on_tied_rows()
        test_brute_force_over_level_prefixes()
    except AssertionError:
        caught = True
    assert caught, f"mutation {name} was not detected"
