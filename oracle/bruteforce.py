"""Second, independent formulation of the verify attention -- TEST INFRASTRUCTURE ONLY.

No bitmask is used: for node i the path is collected by walking the parent array, the
key rows of the committed cache and of that path are concatenated, and ordinary
unmasked softmax attention runs over them in fp64 numpy.  This is the reading of
"The Capstone Validation", section "Context and Motivation" (the batched tree pass
must verify each continuation exactly as if it had been decoded alone) written as
literally as possible.  Only small inputs are meant to pass through it.
"""
from __future__ import annotations

import numpy as np


def path_of(parents_b, i: int):
    """Nodes on the root-to-node path of node i (i included), or None if a parent is invalid."""
    path, j = [], i
    while j != -1:
        path.append(j)
        p = int(parents_b[j])
        if p < -1 or p >= j:
            return None
        j = p
    return path[::-1]


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):                      # torch tensor (bf16 widens exactly)
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, np.float64)


def attention(q_lat, q_rope, ckv, krope, tree_ckv, tree_krope, parents, cache_lens, scale):
    ql, qr = _f64(q_lat), _f64(q_rope)
    B, N, H, dc = ql.shape
    ck, kr = _f64(ckv), _f64(krope)
    tc, tr = _f64(tree_ckv), _f64(tree_krope)
    s = float(np.float32(scale))
    out = np.zeros((B, N, H, dc))
    off = 0
    for b in range(B):
        L = int(cache_lens[b])
        for i in range(N):
            path = path_of(parents[b], i)
            if path is None:
                path = []
            keys_lat = np.concatenate([ck[off:off + L], tc[b, path]], axis=0)
            keys_rope = np.concatenate([kr[off:off + L], tr[b, path]], axis=0)
            if keys_lat.shape[0] == 0:
                continue
            for h in range(H):
                logits = s * (keys_lat @ ql[b, i, h] + keys_rope @ qr[b, i, h])
                w = np.exp(logits - logits.max())
                out[b, i, h] = (w / w.sum()) @ keys_lat
        off += L
    return out


def masks_from_paths(parents) -> np.ndarray:
    """Bitmasks built from explicit paths (python ints), for checking the mask walk."""
    par = np.asarray(parents)
    B, N = par.shape
    W = (N + 63) // 64
    m = np.zeros((B, N, W), dtype=np.uint64)
    for b in range(B):
        for i in range(N):
            path = path_of(par[b], i)
            if path is None:
                continue
            for j in path:
                m[b, i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return m
