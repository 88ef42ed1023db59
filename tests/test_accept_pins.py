"""Pins of the greedy tree-accept and KV-compaction oracle (oracle/accept.py), CPU only.

What pins what:
  tree_accept -- hand-worked fixture (tests/golden/accept_handworked.json); the pages' own
                 numbers: a drafter that proposes the target's greedy continuation, block 8 /
                 budget 7, commits 8 tokens per verify step and 24 tokens in 3 steps ("The
                 Capstone Validation", sections "What the Test Actually Validated" and
                 "Conclusion"), here with distractor siblings at every depth; exhaustive
                 agreement on random trees with distinct sibling tokens with the deepest node
                 whose whole root path matches (found by enumerating every node's path, not
                 by walking); invariants on trees with repeated sibling tokens (the result is
                 a chain of matches that no child extends, and the bonus follows its end).
  kv_compact  -- element-by-element index arithmetic written out with loops on small
                 inputs; invariants (committed rows untouched, rejected rows absent, lengths).
  sensitivity -- planted mistakes (a node compared with its own prediction instead of its
                 parent's; the bonus taken from the parent of the last accepted node) each
                 fail a pin.
"""
import json
import os

import numpy as np
import pytest

from oracle import accept

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def fixture_cases():
    with open(os.path.join(GOLDEN, "accept_handworked.json")) as fh:
        return json.load(fh)["cases"]


@pytest.mark.parametrize("case", fixture_cases(), ids=lambda c: c["name"])
def test_accept_handworked(case):
    par = np.array([case["parents"]], np.int32)
    tok = np.array([case["tokens"]], np.int32)
    nxt = np.array([case["target_next"]], np.int32)
    path, acc, bonus = accept.tree_accept(par, tok, nxt, np.array([case["root_next"]]))
    want = case["path"]
    assert int(acc[0]) == len(want)
    assert path[0, :len(want)].tolist() == want
    assert (path[0, len(want):] == -1).all()
    assert int(bonus[0]) == case["bonus"]


def golden_step_tree(golden, pos, depth, K, rng):
    """Draft tree of one verify step: the golden continuation at rank 0 of every depth plus
    K - 1 distractor siblings per depth (their own subtrees are not expanded), in best-first
    order -- the golden chain has log-prob 0 and is popped first."""
    parents, tokens = [], []
    prev = -1
    chain = []
    for d in range(depth):
        parents.append(prev)
        tokens.append(golden[pos + d])
        prev = len(parents) - 1
        chain.append(prev)
    for d in range(depth):                       # distractors after the chain nodes
        for k in range(1, K):
            parents.append(chain[d - 1] if d else -1)
            tokens.append(100000 + 17 * d + k + int(rng.integers(0, 7)) * 1000)
    return np.array(parents), np.array(tokens), chain


def test_pages_block8_budget7_commits_24_tokens_in_3_steps():
    rng = np.random.default_rng(5)
    golden = [int(x) for x in rng.integers(0, 50000, size=64)]
    committed = [golden[0]]
    steps = 0
    while len(committed) < 25:                   # the prompt token plus 24 generated ones
        pos = len(committed)
        par, tok, chain = golden_step_tree(golden, pos, depth=7, K=3, rng=rng)
        N = len(par)
        # the target's greedy token after a node: the golden continuation where the node is
        # on the golden path, anything else elsewhere
        nxt = np.array([golden[pos + chain.index(i) + 1] if i in chain else -5 for i in range(N)])
        root_next = golden[pos]                  # the target's token after the context
        path, acc, bonus = accept.tree_accept(par[None], tok[None], nxt[None], np.array([root_next]))
        assert path[0, :acc[0]].tolist() == chain
        committed += [int(tok[j]) for j in path[0, :acc[0]]] + [int(bonus[0])]
        steps += 1
        assert int(acc[0]) + 1 == 8              # 8 tokens per verify step
    assert steps == 3
    assert committed[:25] == golden[:25]


def random_tree(rng, N, distinct_siblings):
    par = np.array([-1] + [int(rng.integers(-1, i)) for i in range(1, N)])
    vocab = 6
    tok = np.zeros(N, np.int64)
    for i in range(N):
        if distinct_siblings:
            used = {int(tok[j]) for j in range(i) if par[j] == par[i]}
            choices = [v for v in range(vocab + N) if v not in used]
            tok[i] = choices[int(rng.integers(0, min(len(choices), vocab)))]
        else:
            tok[i] = int(rng.integers(0, 3))
    return par, tok


def root_path(par, i):
    p = []
    while i != -1:
        p.append(i)
        i = int(par[i])
    return p[::-1]


@pytest.mark.parametrize("seed", range(40))
def test_accept_equals_deepest_matching_path(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 24))
    par, tok = random_tree(rng, N, distinct_siblings=True)
    # predictions mostly hit some child's token so that paths get accepted
    nxt = np.array([int(tok[int(rng.integers(0, N))]) if rng.random() < 0.8 else 999 for _ in range(N)])
    root_next = int(tok[int(rng.integers(0, N))]) if rng.random() < 0.9 else 999
    # exhaustive: every node whose whole root path matches the predictions
    best = []
    for i in range(N):
        p = root_path(par, i)
        want, ok = root_next, True
        for j in p:
            if tok[j] != want:
                ok = False
                break
            want = int(nxt[j])
        if ok and len(p) > len(best):
            best = p
    path, acc, bonus = accept.tree_accept(par[None], tok[None], nxt[None], np.array([root_next]))
    assert path[0, :acc[0]].tolist() == best
    assert int(bonus[0]) == (int(nxt[best[-1]]) if best else root_next)


@pytest.mark.parametrize("seed", range(40))
def test_accept_invariants_with_repeated_tokens(seed):
    rng = np.random.default_rng(1000 + seed)
    B, N = 3, int(rng.integers(1, 20))
    trees = [random_tree(rng, N, distinct_siblings=False) for _ in range(B)]
    par = np.stack([t[0] for t in trees])
    tok = np.stack([t[1] for t in trees])
    nxt = rng.integers(0, 3, size=(B, N))
    root = rng.integers(0, 3, size=B)
    path, acc, bonus = accept.tree_accept(par, tok, nxt, root)
    for b in range(B):
        p = path[b, :acc[b]].tolist()
        want, prev = int(root[b]), -1
        for j in p:                               # a chain of matches from the context
            assert par[b, j] == prev and tok[b, j] == want
            prev, want = j, int(nxt[b, j])
        assert int(bonus[b]) == want
        # no child of the last accepted node carries the bonus token
        assert not any(par[b, j] == prev and tok[b, j] == want for j in range(prev + 1, N))
        # at each step the lowest matching index was taken
        cur, w = -1, int(root[b])
        for j in p:
            assert j == min(k for k in range(cur + 1, N) if par[b, k] == cur and tok[b, k] == w)
            cur, w = j, int(nxt[b, j])


def test_kv_compact_index_arithmetic():
    rng = np.random.default_rng(3)
    B, N, dc, dr = 3, 5, 4, 2
    lens = np.array([3, 0, 2])
    T = int(lens.sum())
    ckv = rng.standard_normal((T, dc))
    krope = rng.standard_normal((T, dr))
    tc = rng.standard_normal((B, N, dc))
    tr = rng.standard_normal((B, N, dr))
    path = np.full((B, N), -1)
    path[0, :2] = [1, 4]
    path[2, :3] = [0, 2, 3]
    acc = np.array([2, 0, 3])
    nc, nr, nl = accept.kv_compact(ckv, krope, lens, tc, tr, path, acc)
    assert nl.tolist() == [5, 0, 5]
    assert nc.shape == (10, dc) and nr.shape == (10, dr)
    # request 0: old rows 0..2 then tree rows 1, 4; request 2: old rows 3..4, tree rows 0, 2, 3
    expect_c = [ckv[0], ckv[1], ckv[2], tc[0, 1], tc[0, 4], ckv[3], ckv[4], tc[2, 0], tc[2, 2], tc[2, 3]]
    expect_r = [krope[0], krope[1], krope[2], tr[0, 1], tr[0, 4], krope[3], krope[4], tr[2, 0], tr[2, 2], tr[2, 3]]
    for r in range(10):
        assert (nc[r] == expect_c[r]).all()
        assert (nr[r] == expect_r[r]).all()


@pytest.mark.parametrize("seed", range(10))
def test_kv_compact_invariants(seed):
    rng = np.random.default_rng(seed)
    B, N, dc, dr = 4, 9, 3, 2
    lens = rng.integers(0, 6, size=B)
    T = int(lens.sum())
    ckv = rng.standard_normal((T, dc))
    krope = rng.standard_normal((T, dr))
    tc = rng.standard_normal((B, N, dc))
    tr = rng.standard_normal((B, N, dr))
    par = np.stack([random_tree(rng, N, True)[0] for _ in range(B)])
    acc = rng.integers(0, 4, size=B)
    path = np.full((B, N), -1)
    for b in range(B):
        path[b, :acc[b]] = np.sort(rng.choice(N, size=acc[b], replace=False))
    nc, nr, nl = accept.kv_compact(ckv, krope, lens, tc, tr, path, acc)
    assert (nl == lens + acc).all() and nc.shape[0] == T + acc.sum()
    off_old = np.concatenate([[0], np.cumsum(lens)])
    off_new = np.concatenate([[0], np.cumsum(nl)])
    for b in range(B):
        # committed rows stay, in order, at the request's new offset
        assert (nc[off_new[b]:off_new[b] + lens[b]] == ckv[off_old[b]:off_old[b] + lens[b]]).all()
        kept = nc[off_new[b] + lens[b]:off_new[b + 1]]
        assert (kept == tc[b, path[b, :acc[b]]]).all()
        # rejected tree rows are not committed
        rejected = [j for j in range(N) if j not in path[b, :acc[b]]]
        for j in rejected:
            assert not any((row == tc[b, j]).all() for row in kept)


# ----------------------------------------------------------------------------- sensitivity
def accept_own_prediction(parents, tokens, target_next, root_next):
    """Planted mistake: a child is compared with its own prediction."""
    par, tok, nxt = (np.asarray(x) for x in (parents, tokens, target_next))
    B, N = par.shape
    out = []
    for b in range(B):
        cur, want, p = -1, int(root_next[b]), []
        while True:
            c = next((j for j in range(cur + 1, N) if par[b, j] == cur and tok[b, j] == want), -1)
            if c < 0:
                break
            p.append(c)
            cur = c
            nxt_c = next((j for j in range(cur + 1, N) if par[b, j] == cur), -1)
            want = int(nxt[b, nxt_c]) if nxt_c >= 0 else -1
        out.append(p)
    return out


def test_planted_mistakes_fail_a_pin():
    case = fixture_cases()[0]
    par = np.array([case["parents"]])
    tok = np.array([case["tokens"]])
    nxt = np.array([case["target_next"]])
    wrong = accept_own_prediction(par, tok, nxt, np.array([case["root_next"]]))
    assert wrong[0] != case["path"]
    # bonus from the parent of the last accepted node
    path, acc, _ = accept.tree_accept(par, tok, nxt, np.array([case["root_next"]]))
    last = int(path[0, acc[0] - 1])
    wrong_bonus = int(nxt[0, par[0, last]]) if par[0, last] >= 0 else case["root_next"]
    assert wrong_bonus != case["bonus"]
