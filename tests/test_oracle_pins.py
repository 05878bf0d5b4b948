"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each check is a library routine
(scipy / torch softmax, numpy argmax, rocRAND's Philox), a closed form or
invariant, exact enumeration over a grid of uniforms, a value printed on the
pages (tests/golden), or a mutation that a correct test must catch.
"""
import ctypes
import os
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

from conftest import ROOT, bf16_bits, bf16_to_f32, load_golden

# --------------------------------------------------------------------------
# Softmax at temperature (reading: p = softmax(logits / tau)).
# --------------------------------------------------------------------------


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("tau", [0.6, 0.7, 1.0, 2.5])
def test_softmax_matches_library_routines(oracle_lib, dtype, tau):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(4099) * 3.0 - 1.5).astype(np.float32)
    if dtype == "bf16":
        arg = bf16_bits(x)
        xf = bf16_to_f32(arg)
    else:
        arg = x
        xf = x
    tau32 = float(np.float32(tau))
    p = oracle_lib.softmax_row(arg, tau32)
    ref_scipy = scipy.special.softmax(xf.astype(np.float64) / tau32)
    ref_torch = torch.softmax(torch.from_numpy(xf.astype(np.float64)) / tau32, dim=0).numpy()
    np.testing.assert_allclose(p, ref_scipy, rtol=1e-13, atol=0)
    np.testing.assert_allclose(p, ref_torch, rtol=1e-13, atol=0)
    assert abs(p.sum() - 1.0) < 1e-12


def test_softmax_closed_forms_and_invariants(oracle_lib):
    # Equal logits: exactly uniform.
    p = oracle_lib.softmax_row(np.full(1000, 3.25, np.float32), 0.7)
    np.testing.assert_allclose(p, 1.0 / 1000, rtol=1e-15)
    # Two tokens, logits (0, 1) at temperature 1/2: e^2 / (1 + e^2).
    p = oracle_lib.softmax_row(np.array([0.0, 1.0], np.float32), 0.5)
    assert abs(p[1] - 0.8807970779778823) < 1e-15 and abs(p[0] - 0.11920292202211755) < 1e-15
    # Shift invariance and the power-of-two temperature/scale identity.
    rng = np.random.default_rng(5)
    # logits on a 2^-10 grid, so that the shift and the scaling below are exact in fp32
    x = (np.round(rng.standard_normal(257) * 2 * 1024) / 1024).astype(np.float32)
    a = oracle_lib.softmax_row(x, 0.75)
    b = oracle_lib.softmax_row((x + np.float32(16.0)).astype(np.float32), 0.75)
    c = oracle_lib.softmax_row((x * np.float32(4.0)).astype(np.float32), 3.0)
    np.testing.assert_allclose(a, b, rtol=1e-12)
    np.testing.assert_allclose(a, c, rtol=1e-12)
    # Dividing by tau (not multiplying): a lower temperature sharpens.
    hot = oracle_lib.softmax_row(x, 2.0)
    cold = oracle_lib.softmax_row(x, 0.5)
    assert cold.max() > a.max() > hot.max()


# --------------------------------------------------------------------------
# Greedy argmax: lowest token id among ties.
# --------------------------------------------------------------------------


def test_argmax_first_occurrence_with_planted_bf16_ties(oracle_lib):
    rng = np.random.default_rng(3)
    for trial in range(40):
        V = int(rng.choice([7, 1024, 32001, 152064]))
        x = (rng.standard_normal(V) * 3).astype(np.float32)
        bits = bf16_bits(x)
        vals = bf16_to_f32(bits)
        if trial % 2 == 0:
            # plant a tie of the maximum at 2-4 random positions
            top = bits[int(np.argmax(vals))]
            for pos in rng.choice(V, size=min(V, int(rng.integers(2, 5))), replace=False):
                bits[pos] = top
            vals = bf16_to_f32(bits)
        assert oracle_lib.argmax_row(bits) == int(np.argmax(vals))
        assert oracle_lib.argmax_row(vals) == int(np.argmax(vals))


# --------------------------------------------------------------------------
# Philox4x32-10 against rocRAND's engine compiled host-side.
# --------------------------------------------------------------------------


@pytest.fixture(scope="session")
def rocrand_philox(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available: Philox left unpinned against rocRAND here")
    out = str(tmp_path_factory.mktemp("philox_pin") / "pin.so")
    src = os.path.join(ROOT, "tests", "philox_pin", "rocrand_philox_host.cpp")
    subprocess.run([hipcc, "-x", "hip", "--cuda-host-only", "-O1", "-fPIC", "-shared", "-o", out,
                    src], check=True, capture_output=True)
    lib = ctypes.CDLL(out)
    lib.pin_philox4x32_10.argtypes = [ctypes.c_ulonglong, ctypes.c_void_p, ctypes.c_void_p]
    lib.pin_philox4x32_10.restype = None

    def philox(ctr, seed):
        c = np.ascontiguousarray(np.asarray(ctr, np.uint32))
        o = np.zeros(4, np.uint32)
        lib.pin_philox4x32_10(ctypes.c_ulonglong(seed), c.ctypes.data, o.ctypes.data)
        return o

    return philox


def test_philox_matches_rocrand(oracle_lib, rocrand_philox):
    rng = np.random.default_rng(2024)
    cases = [([0, 0, 0, 0], 0), ([0xFFFFFFFF] * 4, 0xFFFFFFFFFFFFFFFF), ([1, 0, 0, 0], 0),
             ([0, 1, 0, 0], 0), ([0, 0, 1, 0], 0), ([0, 0, 0, 1], 0), ([0, 0, 0, 0], 1),
             ([0, 0, 0, 0], 1 << 32), ([7, 1023, 0, 0], 0xC0FFEE05)]
    for _ in range(3000):
        cases.append((rng.integers(0, 2**32, size=4, dtype=np.uint64).astype(np.uint32),
                      int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))))
    for ctr, seed in cases:
        a = oracle_lib.philox4x32_10(ctr, seed)
        b = rocrand_philox(ctr, seed)
        assert np.array_equal(a, b), (ctr, hex(seed), a, b)


def test_uniform24_is_exact_and_in_unit_interval(oracle_lib):
    assert oracle_lib.uniform24(0) == 0.0
    assert oracle_lib.uniform24(0x000000FF) == 0.0
    assert oracle_lib.uniform24(0x80000000) == 0.5
    assert oracle_lib.uniform24(0xFFFFFFFF) == 1.0 - 2.0**-24
    assert oracle_lib.uniform24(0x00000100) == 2.0**-24


# --------------------------------------------------------------------------
# Inverse CDF: brute force with exact (dyadic) weights.
# --------------------------------------------------------------------------


def test_inverse_cdf_brute_force(oracle_lib):
    rng = np.random.default_rng(9)
    for _ in range(60):
        V = int(rng.integers(1, 9))
        num = rng.integers(0, 5, size=V)
        if num.sum() == 0:
            num[int(rng.integers(V))] = 1
        w = num / 64.0  # exact dyadic weights: every partial sum is exact
        S = Fraction(int(num.sum()), 64)
        for j in range(0, 256, 3):
            v = j / 256.0
            x, S_got, margin, fb = oracle_lib.draw_inverse_cdf(w, v)
            assert not fb and Fraction(S_got) == S
            t = Fraction(v) * S
            cum = Fraction(0)
            expect = None
            for idx in range(V):
                lo = cum
                cum += Fraction(int(num[idx]), 64)
                if lo <= t < cum:
                    expect = idx
                    exp_margin = min(abs(Fraction(v) - lo / S), abs(cum / S - Fraction(v)))
                    break
            assert x == expect
            assert num[x] > 0
            assert abs(margin - float(exp_margin)) < 1e-15
    x, S, _, _ = oracle_lib.draw_inverse_cdf(np.zeros(4), 0.3)
    assert x == -1 and S == 0.0


def test_draw_window_is_every_reachable_id(oracle_lib):
    """ref_draw_window against brute force through the inverse CDF: with
    exact dyadic weights, the ids returned for every uniform in [v - band,
    v + band] (its ends, and both sides of every CDF boundary inside it) are
    exactly the ids from lo to hi that carry weight."""
    rng = np.random.default_rng(19)
    for _ in range(80):
        V = int(rng.integers(1, 10))
        num = rng.integers(0, 5, size=V)
        if num.sum() == 0:
            num[int(rng.integers(V))] = 1
        w = num / 64.0
        S = float(num.sum()) / 64.0
        cdf = np.cumsum(num) / num.sum()  # exact: dyadic over a small integer
        for v in (0.0, 0.25, 0.5, float(rng.uniform(0, 1)), float(cdf[0]), 0.999):
            for band in (1e-9, 1.0 / 64, 0.2):
                lo, hi = oracle_lib.draw_window(w, v, band)
                probes = [min(max(v - band, 0.0), 1 - 2**-30), min(v + band, 1 - 2**-30), v]
                for c in cdf:
                    for eps in (-2**-40, 0.0, 2**-40):
                        u = float(c) + eps
                        if v - band <= u <= v + band and 0.0 <= u < 1.0:
                            probes.append(u)
                seen = {oracle_lib.draw_inverse_cdf(w, u)[0] for u in probes}
                seen.discard(-1)
                assert lo == min(seen) and hi == max(seen), (num, v, band, lo, hi, seen)
                assert all(num[x] > 0 for x in seen)
    assert oracle_lib.draw_window(np.zeros(3), 0.5, 0.1) == (-1, -1)
    assert S > 0


# --------------------------------------------------------------------------
# One sampling round, with the uniforms supplied (exact enumeration).
# --------------------------------------------------------------------------


def _emitted_by_enumeration(oracle_lib, p, q, n_grid):
    """Distribution of the token emitted at a single drafted position.

    The drafted token g runs over q's support with weight q(g); u and v run
    over the grid j / n_grid, which is exactly what the 24-bit uniform hits
    when n_grid divides 2^24.
    """
    V = len(p)
    pp = np.vstack([p, p])  # row 1 = bonus row, unused when L = 1 rejects
    emitted = np.zeros(V)
    accept = {}
    for g in range(V):
        if q[g] <= 0:
            continue
        n_acc = 0
        for j in range(n_grid):
            r = oracle_lib.round_sampling(pp, q[None, :], [g], [j / n_grid], [0.0, 0.0])
            n_acc += r["n"] == 1
        a = n_acc / n_grid
        accept[g] = a
        emitted[g] += q[g] * a
        if n_acc < n_grid:
            # rejected: enumerate the residual draw with u forced to reject
            counts = np.zeros(V)
            for j in range(n_grid):
                r = oracle_lib.round_sampling(pp, q[None, :], [g], [1.0 - 2.0**-24],
                                              [j / n_grid, 0.0])
                assert r["n"] == 0 and r["kind"] in (2, 4)
                counts[r["out"][0]] += 1
            emitted += q[g] * (1 - a) * counts / n_grid
    return emitted, accept


def test_red_blue_example_exactly(oracle_lib):
    gold = load_golden("red_blue.json")
    q = np.array(gold["draft_q"])
    p = np.array(gold["target_p"])
    n_grid = 2**12  # 0.625 = 2560/4096 exactly, and u = 0.625 itself is on the grid
    emitted, accept = _emitted_by_enumeration(oracle_lib, p, q, n_grid)
    assert accept[0] == gold["accept_probability"]["red"]  # 40960 / 65536 exactly
    assert accept[1] == gold["accept_probability"]["blue"]
    assert q[0] * accept[0] == pytest.approx(gold["accepted_mass"]["red"], abs=1e-15)
    assert q[1] * accept[1] == pytest.approx(gold["accepted_mass"]["blue"], abs=1e-15)
    assert q[0] * (1 - accept[0]) == pytest.approx(gold["rejected_mass"], abs=1e-15)
    np.testing.assert_allclose(emitted, gold["emitted"], atol=1e-15)
    # residual is one-hot on blue
    r = oracle_lib.round_sampling(np.vstack([p, p]), q[None, :], [0], [0.99], [0.0, 0.0])
    assert r["out"][0] == 1 and r["S"] == pytest.approx(0.3, abs=1e-15)


def test_emitted_distribution_equals_target_by_enumeration(oracle_lib):
    """min(q,p) + max(0,p-q) = p, summed over every draft token and uniform."""
    rng = np.random.default_rng(17)
    n_grid = 1024
    for trial in range(6):
        V = int(rng.integers(3, 7))
        p = rng.dirichlet(np.ones(V))
        q = rng.dirichlet(np.ones(V))
        if trial == 0:
            p[0] = 0.0  # target gives no mass to a token the draft likes
            p /= p.sum()
        if trial == 1:
            q[1] = 0.0  # draft never proposes a token the target likes
            q /= q.sum()
        emitted, _ = _emitted_by_enumeration(oracle_lib, p, q, n_grid)
        # each grid fraction is off by at most 1/n_grid
        assert np.max(np.abs(emitted - p)) <= 2.0 / n_grid + 1e-12, (p, q, emitted)
        # the identity behind it, element by element
        np.testing.assert_allclose(np.minimum(q, p) + np.maximum(0.0, p - q), p, rtol=0, atol=1e-16)
        assert abs(np.maximum(0, p - q).sum() - (1 - np.minimum(p, q).sum())) < 1e-12


def test_bonus_draw_follows_bonus_row(oracle_lib):
    rng = np.random.default_rng(23)
    V, L = 5, 3
    q = rng.dirichlet(np.ones(V), size=L)
    p = np.vstack([q, rng.dirichlet(np.ones(V))])  # rows 0..L-1 equal q: always accept
    n_grid = 4096
    counts = np.zeros(V)
    for j in range(n_grid):
        r = oracle_lib.round_sampling(p, q, [0, 1, 2], [0.999999] * L, [0.5] * L + [j / n_grid])
        assert r["n"] == L and r["kind"] == 3 and r["row"] == L
        counts[r["out"][L]] += 1
    assert np.max(np.abs(counts / n_grid - p[L])) <= 1.0 / n_grid + 1e-12


def test_forced_accept_and_forced_reject(oracle_lib):
    rng = np.random.default_rng(29)
    V = 6
    for _ in range(50):
        L = int(rng.integers(1, 6))
        rows = rng.dirichlet(np.ones(V), size=L + 1)
        g = rng.integers(0, V, size=L)
        u = rng.random(L) * (1 - 1e-9)
        # identical target and draft rows: every draft accepted, bonus drawn
        r = oracle_lib.round_sampling(rows, rows[:L], g, u, rng.random(L + 1))
        assert r["n"] == L and r["kind"] == 3
        assert list(r["out"][:L]) == list(g)
        # target gives the drafted token zero probability at position j: reject there
        j = int(rng.integers(0, L))
        p = rows.copy()
        p[j, g[j]] = 0.0
        p[j] /= p[j].sum()
        r = oracle_lib.round_sampling(p, rows[:L], g, np.zeros(L), rng.random(L + 1))
        assert r["n"] == j and r["kind"] == 2 and r["out"][j] != g[j]
        assert all(r["out"][j + 1:] == -1)


def test_zero_draft_probability_is_an_error(oracle_lib):
    p = np.array([[0.5, 0.5], [0.5, 0.5]])
    q = np.array([[1.0, 0.0]])
    r = oracle_lib.round_sampling(p, q, [1], [0.5], [0.5, 0.5])
    assert r["n"] == -1 and r["status"] == 4


def test_greedy_round(oracle_lib):
    n, out = oracle_lib.round_greedy([3, 4, 9, 2], [3, 4, 5])
    assert n == 2 and list(out) == [3, 4, 9, -1]
    n, out = oracle_lib.round_greedy([3, 4, 5, 2], [3, 4, 5])
    assert n == 3 and list(out) == [3, 4, 5, 2]
    n, out = oracle_lib.round_greedy([1], [])
    assert n == 0 and list(out) == [1]


# --------------------------------------------------------------------------
# Mutations: each planted mistake must make one of the checks above fail.
# --------------------------------------------------------------------------

MUTATIONS = {
    "resample_from_target": ("w[x] = d > 0.0 ? d : 0.0;", "w[x] = pi[x];"),
    "ratio_inverted": ("double ratio = pg / qg;", "double ratio = qg / pg;"),
    "non_strict_accept": ("if (u[i] < thr) {", "if (u[i] <= thr) {"),
    "residual_sign": ("double d = pi[x] - qi[x];", "double d = qi[x] - pi[x];"),
    "cdf_not_strict": ("if (c > t) {", "if (c >= t) {"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(oracle_lib, tmp_path, name, monkeypatch):
    old, new = MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "spec_verify_ref.c")).read()
    assert src.count(old) == 1
    mdir = tmp_path / "oracle_mut"
    mdir.mkdir()
    (mdir / "spec_verify_ref.c").write_text(src.replace(old, new))
    so = str(mdir / "lib.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-o", so,
                    str(mdir / "spec_verify_ref.c"), "-lm"], check=True)
    import oracle as oracle_pkg

    real_lib = oracle_pkg._load()
    mut = ctypes.CDLL(so)
    for fn in ("ref_round_sampling", "ref_draw_inverse_cdf"):
        getattr(mut, fn).argtypes = getattr(real_lib, fn).argtypes
        getattr(mut, fn).restype = getattr(real_lib, fn).restype
    monkeypatch.setattr(oracle_pkg, "_lib", mut)
    gold = load_golden("red_blue.json")
    q = np.array(gold["draft_q"])
    p = np.array(gold["target_p"])
    caught = []
    try:
        emitted, accept = _emitted_by_enumeration(oracle_pkg, p, q, 2**12)
        caught.append(not np.allclose(emitted, gold["emitted"], atol=1e-15)
                      or accept.get(0) != gold["accept_probability"]["red"])
        if name == "resample_from_target":
            assert emitted[0] == pytest.approx(gold["mutation_resample_from_p_emitted_red"])
        if not any(caught):
            # inverse-CDF boundary: exact dyadic weights, v exactly on a boundary
            x, _, _, _ = oracle_pkg.draw_inverse_cdf(np.array([0.25, 0.25, 0.5]), 0.5)
            caught.append(x != 2)
    except (AssertionError, IndexError, ValueError):
        caught.append(True)
    assert any(caught), f"mutation {name} was not detected"


# --------------------------------------------------------------------------
# Worked rounds printed on the pages, through the whole oracle on logits.
# --------------------------------------------------------------------------


def _forced_round_logits(n_drafts, accepted, vocab, drafts, correction):
    """Logits that force `accepted` acceptances, a rejection, and the correction.

    Accepted positions: target row == draft row (p(g) = q(g): accepted for any
    u < 1). Rejected position: the target gives g probability 0 and all of its
    mass to the correction; the draft puts its mass on g, so the residual
    max(0, p - q) is one-hot on the correction.
    """
    V = len(vocab)
    k = n_drafts
    NEG = np.float32(-1e4)
    target = np.full((1, k + 1, V), NEG, np.float32)
    draft = np.full((1, k, V), NEG, np.float32)
    ids = [vocab.index(t) for t in drafts]
    for i in range(k):
        draft[0, i, ids[i]] = 0.0
        if i < accepted:
            target[0, i, ids[i]] = 0.0
    target[0, accepted, :] = NEG
    target[0, accepted, vocab.index(correction)] = 0.0
    for i in range(accepted + 1, k + 1):
        target[0, i, :] = 0.0  # irrelevant rows after the rejection
    return target, draft, np.array([ids], np.int32)


def test_worked_rounds_from_the_pages(oracle_lib):
    gold = load_golden("worked_rounds.json")
    for rnd in gold["rounds"]:
        vocab = sorted(set(rnd["drafts"]) | {rnd["correction"]} | {"<other>"})
        k = len(rnd["drafts"])
        target, draft, g = _forced_round_logits(k, rnd["accepted"], vocab, rnd["drafts"],
                                                rnd["correction"])
        for seed in (0, 1, 0xC0FFEE01, 2**63 + 5):
            res = oracle_lib.spec_verify_ref(target, draft, g, [k], [1.0], seed)
            n = int(res["num_accepted"][0])
            out = res["out_tokens"][0]
            assert n == rnd["accepted"]
            assert n + 1 == rnd["emitted"]
            assert [vocab[t] for t in out[:n]] == rnd["drafts"][:n]
            assert vocab[out[n]] == rnd["correction"]
            assert all(out[n + 1:] == -1)


# --------------------------------------------------------------------------
# Whole-step statistics: 10^6 seeded trials.
# --------------------------------------------------------------------------

TRIALS = 1_000_000
CHUNK = 200_000


def _run_trials(oracle_lib, target_rows, draft_rows, tau, seed, L, rng, trials=TRIALS):
    """Repeat one round over `trials` sequences sharing the same logit rows.

    Drafted tokens are sampled from the draft distribution (scipy softmax of
    the stored fp32 logits) with numpy's generator, independently per trial.
    """
    k = draft_rows.shape[0]
    V = draft_rows.shape[1]
    q = scipy.special.softmax(draft_rows.astype(np.float64) / np.float32(tau), axis=1)
    outs, ns = [], []
    for b0 in range(0, trials, CHUNK):
        nb = min(CHUNK, trials - b0)
        g = np.stack([rng.choice(V, size=nb, p=q[i]) for i in range(k)], axis=1).astype(np.int32)
        tgt = np.broadcast_to(target_rows, (nb,) + target_rows.shape)
        dft = np.broadcast_to(draft_rows, (nb,) + draft_rows.shape)
        res = oracle_lib.spec_verify_ref(np.ascontiguousarray(tgt), np.ascontiguousarray(dft), g,
                                         np.full(nb, L, np.int32), np.full(nb, tau, np.float32),
                                         seed, seq_base=b0, nthreads=4)
        assert (res["seq_status"] == 0).all()
        outs.append(res["out_tokens"])
        ns.append(res["num_accepted"])
    return np.concatenate(outs), np.concatenate(ns)


def _chi2_pvalue(counts, probs):
    from scipy.stats import chisquare

    probs = np.asarray(probs, np.float64)
    n = counts.sum()
    exp = probs * n
    keep = exp >= 20
    obs = np.append(counts[keep], counts[~keep].sum())
    ex = np.append(exp[keep], exp[~keep].sum())
    if ex[-1] == 0:
        obs, ex = obs[:-1], ex[:-1]
    return chisquare(obs, ex * obs.sum() / ex.sum()).pvalue


@pytest.mark.slow
@pytest.mark.parametrize("V,k,tau", [(2, 1, 1.0), (8, 4, 0.7), (16, 4, 1.0)])
def test_emitted_tokens_follow_target_chi_square(oracle_lib, V, k, tau):
    rng = np.random.default_rng(1000 + V)
    target_rows = (rng.standard_normal((k + 1, V)) * 1.2).astype(np.float32)
    draft_rows = (target_rows[:k] + rng.standard_normal((k, V)) * 0.8).astype(np.float32)
    p = scipy.special.softmax(target_rows.astype(np.float64) / np.float32(tau), axis=1)
    out, n = _run_trials(oracle_lib, target_rows, draft_rows, tau, 0xC0FFEE00 + V, k, rng)
    for i in range(k + 1):
        reached = n >= i
        counts = np.bincount(out[reached, i], minlength=V)
        pv = _chi2_pvalue(counts, p[i])
        assert pv > 1e-4, (i, pv, counts / counts.sum(), p[i])


@pytest.mark.slow
def test_emitted_tokens_chi_square_detects_a_biased_sampler(oracle_lib):
    """Power check of the chi-square: samples from q instead of p must fail."""
    rng = np.random.default_rng(99)
    V = 8
    p = scipy.special.softmax(rng.standard_normal(V) * 1.2)
    q = scipy.special.softmax(np.log(p) + rng.standard_normal(V) * 0.8)
    counts = np.bincount(rng.choice(V, size=TRIALS, p=q), minlength=V)
    assert _chi2_pvalue(counts, p) < 1e-10


def _alpha_pair_logits(alpha):
    # p = (1/2, 1/2); q = (1/2 + d, 1/2 - d) gives sum min(p, q) = 1 - d.
    d = 1.0 - alpha
    t = np.array([0.0, 0.0], np.float32)
    dr = np.log(np.array([0.5 + d, 0.5 - d])).astype(np.float32)
    return t, dr


@pytest.mark.slow
@pytest.mark.parametrize("case", range(5))
def test_accepted_length_matches_printed_expectation(oracle_lib, case):
    gold = load_golden("expected_tokens.json")["cases"][case]
    alpha, k = gold["alpha"], gold["k"]
    rng = np.random.default_rng(77 + case)
    if alpha == 1.0:
        t = np.array([0.3, -0.2], np.float32)
        dr = t.copy()
    else:
        t, dr = _alpha_pair_logits(alpha)
    target_rows = np.tile(t, (k + 1, 1))
    draft_rows = np.tile(dr, (k, 1))
    # realised alpha from the stored fp32 logits (library softmax)
    p = scipy.special.softmax(t.astype(np.float64))
    q = scipy.special.softmax(dr.astype(np.float64))
    a = float(np.minimum(p, q).sum())
    closed = float(sum(a**j for j in range(k + 1)))
    nominal = float(sum(alpha**j for j in range(k + 1)))
    # the printed value is the closed form at the nominal alpha, to its printed precision
    assert abs(nominal - gold["printed"]) <= gold["tol"] + 1e-12
    assert abs(closed - nominal) < 1e-6
    _, n = _run_trials(oracle_lib, target_rows, draft_rows, 1.0, 0xC0FFEE10 + case, k, rng)
    emitted = n.astype(np.float64) + 1
    if alpha == 1.0:
        assert (n == k).all()
        return
    probs = np.array([a**j * (1 - a) for j in range(k)] + [a**k])
    var = float((probs * (np.arange(k + 1) + 1) ** 2).sum() - closed**2)
    se = np.sqrt(var / len(n))
    assert abs(emitted.mean() - closed) < 5 * se, (emitted.mean(), closed, se)
    assert _chi2_pvalue(np.bincount(n, minlength=k + 1), probs) > 1e-4


@pytest.mark.slow
def test_accepted_length_dirichlet_alpha_pair(oracle_lib):
    """V=16: q = p with 0.2 of mass moved between two tokens, so sum min = 0.8."""
    rng = np.random.default_rng(4242)
    V, k = 16, 5
    while True:
        p = rng.dirichlet(np.ones(V))
        if p.max() > 0.25:
            break
    b = int(np.argmax(p))
    a_ = (b + 1) % V
    q = p.copy()
    q[b] -= 0.2
    q[a_] += 0.2
    t = np.log(p).astype(np.float32)
    dr = np.log(q).astype(np.float32)
    pr = scipy.special.softmax(t.astype(np.float64))
    qr = scipy.special.softmax(dr.astype(np.float64))
    a = float(np.minimum(pr, qr).sum())
    assert abs(a - 0.8) < 1e-6
    _, n = _run_trials(oracle_lib, np.tile(t, (k + 1, 1)), np.tile(dr, (k, 1)), 1.0, 0xC0FFEE33,
                       k, rng)
    closed = sum(a**j for j in range(k + 1))
    probs = np.array([a**j * (1 - a) for j in range(k)] + [a**k])
    var = float((probs * (np.arange(k + 1) + 1) ** 2).sum() - closed**2)
    assert abs((n + 1).mean() - closed) < 5 * np.sqrt(var / len(n))


# --------------------------------------------------------------------------
# Whole-step bookkeeping: statuses, greedy, sharding.
# --------------------------------------------------------------------------


def test_status_codes_and_padding(oracle_lib):
    rng = np.random.default_rng(1)
    B, k, V = 6, 3, 32
    t = rng.standard_normal((B, k + 1, V)).astype(np.float32)
    d = rng.standard_normal((B, k, V)).astype(np.float32)
    g = rng.integers(0, V, size=(B, k)).astype(np.int32)
    L = np.array([3, 4, -1, 2, 3, 3], np.int32)
    tau = np.array([1.0, 1.0, 1.0, np.nan, -0.5, 1e-40], np.float32)
    g[0, 2] = V  # bad token in the valid range
    res = oracle_lib.spec_verify_ref(t, d, g, L, tau, 5)
    assert list(res["seq_status"]) == [1, 2, 2, 3, 3, 3]
    assert (res["out_tokens"] == -1).all() and (res["num_accepted"] == 0).all()
    # a bad token beyond the draft length is ignored
    g2 = g.copy()
    g2[0, 2] = 0
    g2[1, :] = rng.integers(0, V, size=k)
    g2[1, 2] = -7
    res = oracle_lib.spec_verify_ref(t[:2], d[:2], g2[:2], np.array([3, 2], np.int32),
                                     np.array([1.0, 1.0], np.float32), 5)
    assert list(res["seq_status"]) == [0, 0]
    for b in range(2):
        n = res["num_accepted"][b]
        assert 0 <= n <= [3, 2][b]
        assert (res["out_tokens"][b, n + 1:] == -1).all() and res["out_tokens"][b, n] >= 0


def test_greedy_sequences_with_bf16_ties(oracle_lib):
    rng = np.random.default_rng(8)
    B, k, V = 16, 4, 3001
    t = bf16_bits((rng.standard_normal((B, k + 1, V)) * 3).astype(np.float32))
    d = bf16_bits((rng.standard_normal((B, k, V)) * 3).astype(np.float32))
    tv = bf16_to_f32(t)
    for b in range(0, B, 2):  # ties of the row max
        for i in range(k + 1):
            top = t[b, i, int(np.argmax(tv[b, i]))]
            t[b, i, rng.choice(V, 3, replace=False)] = top
    tv = bf16_to_f32(t)
    amax = np.argmax(tv, axis=2)
    g = amax[:, :k].copy().astype(np.int32)
    L = rng.integers(0, k + 1, size=B).astype(np.int32)
    for b in range(B):  # break agreement at a random position for some sequences
        if b % 3 == 0 and L[b] > 0:
            j = int(rng.integers(0, L[b]))
            g[b, j] = (g[b, j] + 1) % V
    res = oracle_lib.spec_verify_ref(t, d, g, L, np.zeros(B, np.float32), 123)
    for b in range(B):
        Lb = int(L[b])
        assert list(res["argmax"][b, :Lb + 1]) == list(amax[b, :Lb + 1])
        agree = [g[b, i] == amax[b, i] for i in range(Lb)] + [False]
        n = agree.index(False)
        assert res["num_accepted"][b] == n
        assert list(res["out_tokens"][b, :n]) == list(g[b, :n])
        assert res["out_tokens"][b, n] == amax[b, n]
        assert (res["out_tokens"][b, n + 1:] == -1).all()
        assert np.isnan(res["p_g"][b]).all()


def test_seq_base_sharding_and_threads_do_not_change_results(oracle_lib):
    rng = np.random.default_rng(31)
    B, k, V = 24, 5, 64
    t = rng.standard_normal((B, k + 1, V)).astype(np.float32)
    d = (t[:, :k] + rng.standard_normal((B, k, V)) * 0.7).astype(np.float32)
    g = rng.integers(0, V, size=(B, k)).astype(np.int32)
    L = rng.integers(0, k + 1, size=B).astype(np.int32)
    tau = np.full(B, 0.9, np.float32)
    whole = oracle_lib.spec_verify_ref(t, d, g, L, tau, 99)
    threaded = oracle_lib.spec_verify_ref(t, d, g, L, tau, 99, nthreads=5)
    parts = [oracle_lib.spec_verify_ref(t[a:b], d[a:b], g[a:b], L[a:b], tau[a:b], 99, seq_base=a)
             for a, b in ((0, 7), (7, 20), (20, 24))]
    for key in ("out_tokens", "num_accepted", "draw_row", "draw_kind"):
        assert np.array_equal(whole[key], threaded[key])
        assert np.array_equal(whole[key], np.concatenate([p[key] for p in parts]))
    # a different seed changes some outcome
    other = oracle_lib.spec_verify_ref(t, d, g, L, tau, 100)
    assert not np.array_equal(whole["out_tokens"], other["out_tokens"])
