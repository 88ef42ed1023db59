"""Pins of the best-first tree builder oracle (oracle/tree_build.py), CPU only.

What pins what:
  best_first_tree -- hand-worked fixture (tests/golden/tree_build_handworked.json, scores
                     exact in binary, one case with tied scores); the pages' oracle drafter
                     (the target's token first at every depth with log probability 0,
                     distractors below) gives, with budget 7, the chain of target tokens ("The
                     Capstone Validation", section "What the Test Actually Validated");
                     exhaustive agreement with sorting every rank path by score (the nodes are
                     the top-N paths in score order, each parent its prefix); invariants
                     (parent before child, depth = parent depth + 1, scores non-increasing).
  sensitivity      -- planted mistakes (a sibling scored from the node instead of its prefix;
                     the child pushed before the sibling) each fail a pin.
"""
import heapq
import itertools
import json
import os

import numpy as np
import pytest

from oracle import tree_build

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def fixture_cases():
    with open(os.path.join(GOLDEN, "tree_build_handworked.json")) as fh:
        return json.load(fh)["cases"]


@pytest.mark.parametrize("case", fixture_cases(), ids=lambda c: c["name"])
def test_tree_build_handworked(case):
    lp = np.array([case["logp"]], np.float32)
    cd = np.array([case["cand"]], np.int32)
    par, tok, dep, rk = tree_build.best_first_tree(lp, cd, case["N"])
    assert par[0].tolist() == case["parents"]
    assert tok[0].tolist() == case["tokens"]
    assert dep[0].tolist() == case["depth"]
    assert rk[0].tolist() == case["rank"]


def drafter_logp(rng, B, D, K):
    z = rng.normal(0.0, 2.0, size=(B, D, K))
    lp = np.minimum(z - np.log(np.exp(z).sum(-1, keepdims=True)), 0.0)   # log probabilities are <= 0
    return -np.sort(-lp, axis=-1).astype(np.float32)


def test_pages_oracle_drafter_gives_the_target_chain():
    rng = np.random.default_rng(0)
    D, K = 8, 8
    golden = rng.integers(0, 50000, size=D)
    lp = np.zeros((1, D, K), np.float32)
    lp[0, :, 1:] = -np.arange(1, K, dtype=np.float32)[None, :] * 2.5    # distractors below 0
    cand = np.zeros((1, D, K), np.int32)
    cand[0, :, 0] = golden
    cand[0, :, 1:] = 900000 + rng.integers(0, 1000, size=(D, K - 1))
    par, tok, dep, _ = tree_build.best_first_tree(lp, cand, 7)            # budget 7 (block 8)
    assert par[0].tolist() == [-1, 0, 1, 2, 3, 4, 5]
    assert tok[0].tolist() == golden[:7].tolist()
    assert dep[0].tolist() == list(range(1, 8))


@pytest.mark.parametrize("seed", range(30))
def test_nodes_are_the_top_n_paths_in_score_order(seed):
    rng = np.random.default_rng(seed)
    D, K = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    total = sum(K ** d for d in range(1, D + 1))
    N = int(rng.integers(1, total + 1))
    lp = drafter_logp(rng, 1, D, K)
    cand = rng.integers(0, 1000, size=(1, D, K)).astype(np.int32)
    # every rank path with its fp32 score (prefix score + one log probability per depth)
    paths = {}
    for d in range(1, D + 1):
        for ks in itertools.product(range(K), repeat=d):
            s = np.float32(0.0)
            for j, k in enumerate(ks):
                s = np.float32(s + lp[0, j, k])
            paths[ks] = s
    scores = sorted(paths.values(), reverse=True)
    par, tok, dep, rk = tree_build.best_first_tree(lp, cand, N)
    if len(set(scores[:N + 1])) < min(N + 1, len(scores)):
        # tied scores: which of the tied paths come first depends on push order, so check what
        # is unique -- the chosen nodes' scores are the N best, in order, and every node's
        # prefix is an earlier node
        got = []
        for i in range(N):
            ks, j = [], i
            while j != -1:
                ks.append(int(rk[0, j]))
                j = int(par[0, j])
                assert j < i
            got.append(paths[tuple(reversed(ks))])
            assert dep[0, i] == len(ks)
        assert [float(x) for x in got] == [float(x) for x in scores[:N]]
        return
    top = sorted(paths, key=lambda p: -paths[p])[:N]
    index = {p: i for i, p in enumerate(top)}
    for i, p in enumerate(top):
        assert dep[0, i] == len(p) and rk[0, i] == p[-1]
        assert par[0, i] == (index[p[:-1]] if len(p) > 1 else -1)
        assert tok[0, i] == cand[0, len(p) - 1, p[-1]]


@pytest.mark.parametrize("seed", range(10))
def test_tree_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    B, D, K, N = 4, 8, 8, 64
    lp = drafter_logp(rng, B, D, K)
    cand = rng.integers(0, 1 << 20, size=(B, D, K)).astype(np.int32)
    par, tok, dep, rk = tree_build.best_first_tree(lp, cand, N)
    for b in range(B):
        sc = []
        for i in range(N):
            p = par[b, i]
            assert -1 <= p < i
            assert dep[b, i] == (dep[b, p] + 1 if p >= 0 else 1)
            s = np.float32((sc[p] if p >= 0 else 0.0) + lp[b, dep[b, i] - 1, rk[b, i]])
            sc.append(s)
        assert all(sc[i] >= sc[i + 1] for i in range(N - 1))


def test_short_frontier_pads_with_minus_two():
    lp = np.array([[[-0.5, -1.0]]], np.float32)        # D = 1, K = 2: only two paths
    par, tok, dep, rk = tree_build.best_first_tree(lp, np.array([[[7, 8]]]), 4)
    assert par[0].tolist() == [-1, -1, -2, -2] and tok[0].tolist() == [7, 8, -2, -2]


# ----------------------------------------------------------------------------- sensitivity
def planted(lp, cand, N, sibling_from_node=False, child_first=False):
    lp = np.asarray(lp, np.float32)
    D, K = lp.shape[1:]
    par, sc = [], []
    heap, push = [(-lp[0, 0, 0], 0, -1, 0, 0)], 1
    while heap and len(par) < N:
        neg, _, prefix, d, k = heapq.heappop(heap)
        s = np.float32(-neg)
        i = len(par)
        par.append(prefix)
        sc.append(s)
        todo = []
        if k + 1 < K:
            base = s if sibling_from_node else (sc[prefix] if prefix >= 0 else np.float32(0))
            todo.append((-np.float32(base + lp[0, d, k + 1]), prefix, d, k + 1))
        if d + 1 < D:
            todo.append((-np.float32(s + lp[0, d + 1, 0]), i, d + 1, 0))
        if child_first:
            todo = todo[::-1]
        for t in todo:
            heapq.heappush(heap, (t[0], push, t[1], t[2], t[3]))
            push += 1
    return par


def top_n_parents(lp, N):
    D, K = lp.shape[1:]
    paths = {}
    for d in range(1, D + 1):
        for ks in itertools.product(range(K), repeat=d):
            s = np.float32(0.0)
            for j, k in enumerate(ks):
                s = np.float32(s + lp[0, j, k])
            paths[ks] = s
    top = sorted(paths, key=lambda p: -paths[p])[:N]
    index = {p: i for i, p in enumerate(top)}
    return [index[p[:-1]] if len(p) > 1 else -1 for p in top]


def test_planted_mistakes_fail_a_pin():
    c1 = fixture_cases()[1]
    assert planted(np.array([c1["logp"]]), None, c1["N"], child_first=True) != c1["parents"]
    assert planted(np.array([c1["logp"]]), None, c1["N"]) == c1["parents"]
    # a sibling scored from the node rather than its prefix breaks the top-N pin
    caught = 0
    for seed in range(10):
        lp = drafter_logp(np.random.default_rng(seed), 1, 3, 3)
        caught += planted(lp, None, 12, sibling_from_node=True) != top_n_parents(lp, 12)
    assert caught > 0
