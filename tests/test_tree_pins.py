"""Pins of the tree oracle (greedy verification of a candidate tree).

The pages describe tree verification only in words: EAGLE-2/3 verify a tree
of candidate continuations together ("Speculative Decoding and the Art of
Fast LLM Inference", "EAGLE: drafting in feature space"; techaiinterview.com,
"Drafts and limits", tree verification), with no sampling rule, so the oracle
applies the linear greedy rule along every branch. It is pinned against:

  - the linear greedy round, itself pinned elsewhere: a chain tree is a
    linear draft;
  - brute force: every root path enumerated and checked edge by edge, the
    deepest valid one kept (lowest end index among equals);
  - a tree worked by hand;
  - planted mistakes, each of which must break one of the pins above.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

from conftest import ROOT, bf16_bits

import oracle  # noqa: E402


def _brute_force(amax, par, tok):
    n = len(amax)
    best, best_path = 0, []
    for end in range(n):
        path = []
        x = end
        while x != 0:
            path.append(x)
            x = par[x]
        path.reverse()
        ok, prev = True, 0
        for node in path:
            if tok[node] != amax[prev]:
                ok = False
                break
            prev = node
        if ok and len(path) > len(best_path):
            best, best_path = end, path
    out = [tok[x] for x in best_path] + [amax[best]]
    return len(best_path), out, best_path


def _random_tree(rng, n, alphabet):
    par = [-1] + [int(rng.integers(0, i)) for i in range(1, n)]
    tok = [0] + [int(rng.integers(0, alphabet)) for _ in range(1, n)]
    amax = [int(rng.integers(0, alphabet)) for _ in range(n)]
    return amax, par, tok


def test_chain_tree_is_the_linear_greedy_round():
    rng = np.random.default_rng(1)
    for trial in range(300):
        L = int(rng.integers(0, 9))
        amax = rng.integers(0, 4, size=L + 1)
        g = np.where(rng.random(L) < 0.7, amax[:L], rng.integers(0, 4, size=L))
        n_lin, out_lin = oracle.round_greedy(amax, g)
        par = [-1] + list(range(L))
        tok = [0] + list(g)
        d, out, path = oracle.tree_greedy(amax, par, tok)
        assert d == n_lin
        assert list(out) == list(out_lin[:n_lin + 1])
        assert list(path) == list(range(1, d + 1))


def test_brute_force_over_random_trees():
    rng = np.random.default_rng(2)
    for trial in range(2000):
        n = int(rng.integers(1, 13))
        amax, par, tok = _random_tree(rng, n, alphabet=int(rng.integers(1, 4)))
        d, out, path = oracle.tree_greedy(amax, par, tok)
        bd, bout, bpath = _brute_force(amax, par, tok)
        assert (d, list(out), list(path)) == (bd, bout, bpath), (amax, par, tok)


def test_hand_worked_tree():
    # root 0 (argmax 7) has children 1 (token 5) and 2 (token 7): 2 matches.
    # node 2 (argmax 2) has child 4 (token 2): matches; node 4 (argmax 4) has
    # child 5 (token 4): matches; node 5's argmax 1 is the bonus. Node 3 hangs
    # below the rejected node 1 and is not reachable although its token 9
    # equals node 1's argmax.
    amax = [7, 9, 2, 0, 4, 1]
    par = [-1, 0, 0, 1, 2, 4]
    tok = [0, 5, 7, 9, 2, 4]
    d, out, path = oracle.tree_greedy(amax, par, tok)
    assert d == 3
    assert list(out) == [7, 2, 4, 1]
    assert list(path) == [2, 4, 5]
    # two equally deep accepted leaves: the lower node index wins
    d, out, path = oracle.tree_greedy([3, 5, 5, 8, 9], [-1, 0, 0, 1, 2], [0, 3, 3, 5, 5])
    assert (d, list(out), list(path)) == (2, [3, 5, 8], [1, 3])
    # a lone root: nothing accepted, the root's argmax is emitted
    d, out, path = oracle.tree_greedy([6], [-1], [0])
    assert (d, list(out), list(path)) == (0, [6], [])


def test_batch_oracle_argmax_per_node_and_statuses():
    rng = np.random.default_rng(3)
    B, N, V = 6, 8, 50
    logits = rng.standard_normal((B, N, V)).astype(np.float32)
    par = np.tile(np.array([-1, 0, 0, 1, 1, 2, 3, 5], np.int32), (B, 1))
    amax = logits.argmax(axis=2)
    tok = np.zeros((B, N), np.int32)
    for b in range(B):
        for n in range(1, N):
            tok[b, n] = amax[b, par[b, n]] if rng.random() < 0.6 else (amax[b, par[b, n]] + 1) % V
    nn = np.array([8, 5, 1, 0, 8, 8], np.int32)
    par[4, 3] = 3  # parent not before the node
    tok[5, 6] = V  # token out of range
    res = oracle.spec_tree_ref(logits, par, tok, nn)
    assert list(res["seq_status"]) == [0, 0, 0, oracle.SEQ_BAD_LEN, oracle.SEQ_BAD_TREE,
                                       oracle.SEQ_BAD_TOKEN]
    for b in range(3):
        n = nn[b]
        assert list(res["argmax"][b, :n]) == list(amax[b, :n])
        assert (res["argmax"][b, n:] == -1).all()
        d, out, path = _brute_force(list(amax[b, :n]), list(par[b, :n]), list(tok[b, :n]))
        assert res["num_accepted"][b] == d
        assert list(res["out_tokens"][b, :d + 1]) == out
        assert (res["out_tokens"][b, d + 1:] == -1).all()
        assert list(res["path_nodes"][b, :d]) == path
    for b in range(3, 6):
        assert (res["out_tokens"][b] == -1).all() and res["num_accepted"][b] == 0
    # bf16 rows: argmax ties go to the lowest id
    t16 = bf16_bits(np.zeros((1, 2, 16), np.float32))
    res = oracle.spec_tree_ref(t16, np.array([[-1, 0]], np.int32), np.array([[0, 0]], np.int32),
                               [2])
    assert list(res["argmax"][0]) == [0, 0] and res["num_accepted"][0] == 1


TREE_MUTATIONS = {
    "parent_not_required": ("acc[n] = acc[par[n]] && (int64_t)tok[n] == amax[par[n]];",
                            "acc[n] = (int64_t)tok[n] == amax[par[n]];"),
    "own_argmax": ("acc[n] = acc[par[n]] && (int64_t)tok[n] == amax[par[n]];",
                   "acc[n] = acc[par[n]] && (int64_t)tok[n] == amax[n];"),
    "last_of_deepest": ("if (acc[n] && depth[n] > depth[best])",
                        "if (acc[n] && depth[n] >= depth[best])"),
    "bonus_from_parent": ("out[d] = (int32_t)amax[best];", "out[d] = (int32_t)amax[par[best]];"),
}


@pytest.mark.parametrize("name", sorted(TREE_MUTATIONS))
def test_planted_tree_mistakes_are_caught(tmp_path, name, monkeypatch):
    old, new = TREE_MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "spec_verify_ref.c")).read()
    assert src.count(old) == 1
    path = tmp_path / "spec_verify_ref.c"
    path.write_text(src.replace(old, new))
    so = str(tmp_path / "lib.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-o", so,
                    str(path), "-lm"], check=True)
    real = oracle._load()
    mut = ctypes.CDLL(so)
    for fn in ("ref_tree_greedy", "ref_round_greedy"):
        getattr(mut, fn).argtypes = getattr(real, fn).argtypes
        getattr(mut, fn).restype = getattr(real, fn).restype
    monkeypatch.setattr(oracle, "_lib", mut)
    caught = False
    try:
        test_hand_worked_tree()
        test_brute_force_over_random_trees()
        test_chain_tree_is_the_linear_greedy_round()
    except (AssertionError, IndexError):
        caught = True
    assert caught, f"mutation {name} was not detected"
