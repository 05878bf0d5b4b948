"""Pins of the prompt-lookup oracle.

The pages give prompt lookup in words: search the existing context for a
recent matching n-gram and propose the tokens that followed it last time
("Speculative Decoding and the Art of Fast LLM Inference", "n-gram and
prompt lookup: no model at all"; techaiinterview.com, "Drafts and limits").
Reading taken: sizes from n_max down to n_min, the most recent occurrence
ending before the last token, up to k following tokens. Pinned against a
brute force written differently (every window listed, then filtered),
hand-worked contexts, invariants and planted mistakes.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

from conftest import ROOT

import oracle  # noqa: E402


def _brute_force(ctx, n_min, n_max, k):
    ctx = list(ctx)
    T = len(ctx)
    for n in range(n_max, n_min - 1, -1):
        if n < 1 or n > T:
            continue
        tail = ctx[T - n:]
        hits = [s for s in range(0, T - n + 1) if ctx[s:s + n] == tail and s + n - 1 < T - 1]
        if hits:
            s = max(hits)
            return ctx[s + n:s + n + k], n, s
    return [], 0, -1


def test_hand_worked_contexts():
    # "1 2 3" recurs at 3..5 and at the end: propose what followed it
    d, n, s = oracle.prompt_lookup([5, 6, 7, 1, 2, 3, 9, 1, 2, 3], 1, 3, 4)
    assert (list(d), n, s) == ([9, 1, 2, 3], 3, 3)
    # no earlier "4 1 2"; the 2-gram "1 2" recurs at 0; the proposal stops at the end
    d, n, s = oracle.prompt_lookup([1, 2, 3, 4, 1, 2], 1, 3, 5)
    assert (list(d), n, s) == ([3, 4, 1, 2], 2, 0)
    # overlapping occurrences: the latest one that ends before the last token
    d, n, s = oracle.prompt_lookup([4, 4, 4, 4], 1, 2, 3)
    assert (list(d), n, s) == ([4], 2, 1)
    # nothing recurs
    d, n, s = oracle.prompt_lookup([1, 2, 3], 1, 3, 3)
    assert (list(d), n, s) == ([], 0, -1)
    # the most recent match wins over an older, longer continuation
    d, n, s = oracle.prompt_lookup([7, 8, 1, 2, 3, 7, 8, 5, 7, 8], 2, 2, 3)
    assert (list(d), n, s) == ([5, 7, 8], 2, 5)
    # k = 0 proposes nothing but still reports the match
    d, n, s = oracle.prompt_lookup([7, 8, 1, 7, 8], 2, 2, 0)
    assert (list(d), n, s) == ([], 2, 0)
    # empty and one-token contexts
    assert oracle.prompt_lookup([], 1, 3, 4)[1:] == (0, -1)
    assert oracle.prompt_lookup([3], 1, 3, 4)[1:] == (0, -1)


def test_brute_force_over_random_contexts():
    rng = np.random.default_rng(11)
    for trial in range(3000):
        T = int(rng.integers(0, 40))
        alphabet = int(rng.integers(1, 6))
        ctx = rng.integers(0, alphabet, size=T)
        n_min = int(rng.integers(1, 4))
        n_max = n_min + int(rng.integers(0, 4))
        k = int(rng.integers(0, 8))
        d, n, s = oracle.prompt_lookup(ctx, n_min, n_max, k)
        bd, bn, bs = _brute_force(ctx, n_min, n_max, k)
        assert (list(d), n, s) == (bd, bn, bs), (list(ctx), n_min, n_max, k)


def test_invariants():
    rng = np.random.default_rng(12)
    for trial in range(1000):
        T = int(rng.integers(2, 60))
        ctx = list(rng.integers(0, 3, size=T))
        d, n, s = oracle.prompt_lookup(ctx, 1, 4, 5)
        if n == 0:
            assert all(ctx[T - 1] != ctx[x] for x in range(T - 1))  # not even a 1-gram recurs
            continue
        assert ctx[s:s + n] == ctx[T - n:]
        assert list(d) == ctx[s + n:s + n + 5]
        for later in range(s + 1, T - n):  # no later occurrence of the same size
            assert ctx[later:later + n] != ctx[T - n:]
        for bigger in range(n + 1, 5):  # no occurrence of a longer n-gram
            assert all(ctx[x:x + bigger] != ctx[T - bigger:] for x in range(0, T - bigger))


def test_batch_oracle():
    rng = np.random.default_rng(13)
    B, T_max, k = 7, 30, 4
    ctx = rng.integers(0, 4, size=(B, T_max)).astype(np.int32)
    lens = np.array([30, 10, 0, 1, 31, -1, 25], np.int32)
    res = oracle.spec_prompt_lookup_ref(ctx, lens, 1, 3, k)
    for b in range(B):
        if 0 <= lens[b] <= T_max:
            d, n, s = _brute_force(ctx[b, :lens[b]], 1, 3, k)
        else:
            d, n, s = [], 0, -1
        assert res["draft_len"][b] == len(d)
        assert list(res["draft_tokens"][b, :len(d)]) == d
        assert (res["draft_tokens"][b, len(d):] == -1).all()
        assert (res["match_n"][b], res["match_s"][b]) == (n, s)


LOOKUP_MUTATIONS = {
    "oldest_match": ("for (int s = T - n - 1; s >= 0; s--) {", "for (int s = 0; s <= T - n - 1; s++) {"),
    "shortest_first": ("for (int n = n_max; n >= n_min; n--) {", "for (int n = n_min; n <= n_max; n++) {"),
    "trailing_counts": ("for (int s = T - n - 1; s >= 0; s--) {", "for (int s = T - n; s >= 0; s--) {"),
    "continuation_early": ("for (int j = s + n; j < T && len < k; j++)",
                           "for (int j = s + n - 1; j < T && len < k; j++)"),
}


@pytest.mark.parametrize("name", sorted(LOOKUP_MUTATIONS))
def test_planted_lookup_mistakes_are_caught(tmp_path, name, monkeypatch):
    old, new = LOOKUP_MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "spec_verify_ref.c")).read()
    assert src.count(old) == 1
    path = tmp_path / "spec_verify_ref.c"
    path.write_text(src.replace(old, new))
    so = str(tmp_path / "lib.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-o", so,
                    str(path), "-lm"], check=True)
    real = oracle._load()
    mut = ctypes.CDLL(so)
    mut.ref_prompt_lookup.argtypes = real.ref_prompt_lookup.argtypes
    mut.ref_prompt_lookup.restype = real.ref_prompt_lookup.restype
    monkeypatch.setattr(oracle, "_lib", mut)
    caught = False
    try:
        test_hand_worked_contexts()
        test_brute_force_over_random_contexts()
    except AssertionError:
        caught = True
    assert caught, f"mutation {name} was not detected"
