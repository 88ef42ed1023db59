"""Best-first draft-tree construction: plain CPU reference -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may
import this module; the product library never loads it and shares no code with it.  Its
pins are listed in the header of ``tests/test_tree_build_pins.py``.

What the pages fix (cited by title and section):
* The engine has a GPU best-first tree builder that replaced a per-request CPU heapq
  ("Validating the Native Engine", section "The Broader Context").
* The drafter returns, for each depth up to a limit and each of top-k slots, a log
  probability and a token id, sorted so that the best-first search picks the best path
  ("The Capstone Validation", section "What the Test Actually Validated").
* A drafter that puts the target's token first at every depth with log probability 0 and
  distractors at decreasing log probabilities makes the builder select that path ("The
  Capstone Validation", same section); with budget 7 the tree is that chain.

The search, as the heap algorithm it replaces runs it: a node is a rank path
(k_1, ..., k_d), scored by the sum of its per-depth log probabilities.  The frontier starts
with the depth-1 rank-0 path.  Each step pops the best-scoring path (ties: the earliest
pushed); it becomes the next node, its parent being the node of its prefix (-1 at depth 1).
Then its next sibling (same prefix, rank + 1, if below K) and its first child (rank 0 at
the next depth, if below D) are pushed, in that order.  N steps give N nodes, parents
before children.  Scores are fp32: a path's score is its prefix's score plus one fp32 log
probability (one rounding per step), the same arithmetic on both sides of the parity test.
"""
from __future__ import annotations

import heapq

import numpy as np


def best_first_tree(logp, cand, N: int):
    """logp [B, D, K] float32 (each row sorted descending), cand [B, D, K] int32 token ids.

    Returns (parents [B, N], tokens [B, N], depth [B, N] (1-based), rank [B, N]) as int32;
    a request whose frontier empties before N nodes (K^1 + ... + K^D < N) gets -2 in the
    rest of its rows.
    """
    lp = np.asarray(logp, dtype=np.float32)
    cd = np.asarray(cand, dtype=np.int64)
    B, D, K = lp.shape
    parents = np.full((B, N), -2, np.int32)
    tokens = np.full((B, N), -2, np.int32)
    depth = np.full((B, N), -2, np.int32)
    rank = np.full((B, N), -2, np.int32)
    for b in range(B):
        node_score = []
        push_no = 0
        # entries: (-score, push order, prefix node, depth index, rank); score kept as float32
        heap = [(-lp[b, 0, 0], push_no, -1, 0, 0)]
        push_no += 1
        for i in range(N):
            if not heap:
                break
            neg, _, prefix, d, k = heapq.heappop(heap)
            score = np.float32(-neg)
            parents[b, i] = prefix
            tokens[b, i] = cd[b, d, k]
            depth[b, i] = d + 1
            rank[b, i] = k
            node_score.append(score)
            if k + 1 < K:
                base = node_score[prefix] if prefix >= 0 else np.float32(0.0)
                s = np.float32(base + lp[b, d, k + 1])
                heapq.heappush(heap, (-s, push_no, prefix, d, k + 1))
                push_no += 1
            if d + 1 < D:
                s = np.float32(score + lp[b, d + 1, 0])
                heapq.heappush(heap, (-s, push_no, i, d + 1, 0))
                push_no += 1
    return parents, tokens, depth, rank
