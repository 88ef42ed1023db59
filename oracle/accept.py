"""Greedy tree-accept and post-verify KV compaction: plain CPU references -- TEST
INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may
import this module; the product library never loads it and shares no code with it.  The
pins of both functions are listed in the header of ``tests/test_accept_pins.py``.

What the pages fix (cited by title and section):
* The engine closes each verify pass with a greedy tree-accept kernel and a KV cache with
  post-verify compaction ("Validating the Native Engine", section "The Broader Context").
* The speculative loop: the drafted candidates form a tree, the target verifies them in one
  batched pass, accepted tokens are committed and rejected ones discarded, and the target's
  prediction at the final accepted node is a bonus token ("The Capstone Validation",
  sections "Context and Motivation" and "What the Test Actually Validated").
* With a drafter that always proposes the target's greedy continuation, a block of 8
  (budget 7) commits 8 tokens per verify step: 24 tokens in 3 steps (same page, sections
  "What the Test Actually Validated" and "Conclusion").

Readings taken where the pages are silent:
* Greedy acceptance walks the tree from the committed context: a node is accepted when its
  token equals the target's greedy token at its parent's position (at the context's last
  position for a depth-1 node, ``root_next``), and the walk continues from it.  Siblings of a
  well-formed tree carry distinct tokens, so at most one child matches; for malformed input
  the lowest-index matching child is taken.  A child is looked for only among higher node
  indices (parents come before children), which also bounds the walk.
* The bonus token is the target's greedy token after the last accepted node (``root_next``
  when nothing is accepted).
* Compaction commits, per request, the accepted nodes' latent rows in path order right after
  the request's committed rows; the packed per-request cache is rebuilt with the new lengths
  (requests stay packed in request order).
"""
from __future__ import annotations

import numpy as np


def tree_accept(parents, tokens, target_next, root_next):
    """Greedy walk per request.

    parents [B, N] int (parent < child, -1 at depth 1), tokens [B, N] drafted token ids,
    target_next [B, N] the target's greedy token after each node, root_next [B] the target's
    greedy token after the committed context.

    Returns (path [B, N] int32, accepted node ids in root-to-leaf order, padded with -1;
    accept_len [B] int32; bonus [B] int32).
    """
    par = np.asarray(parents, dtype=np.int64)
    tok = np.asarray(tokens, dtype=np.int64)
    nxt = np.asarray(target_next, dtype=np.int64)
    root = np.asarray(root_next, dtype=np.int64)
    B, N = par.shape
    path = np.full((B, N), -1, dtype=np.int32)
    acc = np.zeros(B, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    for b in range(B):
        cur, want, k = -1, int(root[b]), 0
        while True:
            child = -1
            for j in range(cur + 1, N):
                if par[b, j] == cur and tok[b, j] == want:
                    child = j
                    break
            if child < 0:
                break
            path[b, k] = child
            k += 1
            cur, want = child, int(nxt[b, child])
        acc[b] = k
        bonus[b] = want
    return path, acc, bonus


def kv_compact(ckv, krope, cache_lens, tree_ckv, tree_krope, path, accept_len):
    """Rebuild the packed cache with each request's accepted rows appended.

    ckv [T, d_c], krope [T, d_r]: committed rows packed per request in request order;
    tree_ckv [B, N, d_c], tree_krope [B, N, d_r]; path / accept_len as from tree_accept.

    Returns (new_ckv [T', d_c], new_krope [T', d_r], new_lens [B] int32) with
    T' = T + sum(accept_len).
    """
    ckv, krope = np.asarray(ckv), np.asarray(krope)
    tc, tr = np.asarray(tree_ckv), np.asarray(tree_krope)
    lens = np.asarray(cache_lens, dtype=np.int64)
    acc = np.asarray(accept_len, dtype=np.int64)
    pth = np.asarray(path, dtype=np.int64)
    B = lens.shape[0]
    parts_c, parts_r = [], []
    off = 0
    for b in range(B):
        L = int(lens[b])
        parts_c.append(ckv[off:off + L])
        parts_r.append(krope[off:off + L])
        nodes = pth[b, :int(acc[b])]
        parts_c.append(tc[b, nodes])
        parts_r.append(tr[b, nodes])
        off += L
    new_lens = (lens + acc).astype(np.int32)
    return np.concatenate(parts_c, axis=0), np.concatenate(parts_r, axis=0), new_lens
