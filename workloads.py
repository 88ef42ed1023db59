"""Seeded synthetic inputs for the tree-verify MLA-absorb attention path.

This module only *generates* inputs: parent arrays, committed-cache lengths, absorbed
queries and latent KV rows.  It contains none of the verify arithmetic (no masks, no
scores, no softmax), so both the fp64 oracle and the HIP path may consume it.

Workload shapes follow the draft-tree verification described on "The Capstone
Validation: Writing the DDTree Speculative Decode Test" (section "Context and
Motivation": a drafter proposes candidates arranged in a tree and the target verifies
them in one batched pass; section "What the Test Actually Validated": the drafter
returns, per depth, log-probabilities sorted for a best-first tree builder) and the
MLA model named on "Validating the Native Engine" (section "The Broader Context":
a DeepSeekV3-style model with Multi-head Latent Attention).

Every random draw comes from ``numpy.random.default_rng([config_id, request, stream,
seed])`` so that any single request can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
import heapq
import math
from typing import Dict, List, Optional

import numpy as np
import torch

# stream ids for default_rng([cfg, b, stream, seed])
S_TREE, S_LEN, S_QLAT, S_QROPE, S_CKV, S_KROPE, S_TCKV, S_TKROPE, S_OUTLIER = range(9)


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape and distribution of one synthetic verify batch."""
    name: str
    cfg_id: int
    batch: int
    nodes: int
    heads: int
    d_latent: int
    d_rope: int
    dtype: str                  # "bf16" or "f32"
    cache_len: Optional[int]    # fixed committed length, or None for ragged
    ragged: Optional[tuple] = None   # (lo, hi) inclusive, uniform integers
    tree: str = "bestfirst"     # "bestfirst" | "random" | "chain" | "star"
    depth: int = 8              # best-first: maximum depth
    topk: int = 8               # best-first: candidates per depth
    outlier_p: float = 0.0      # probability that an element is multiplied by outlier_mul
    outlier_mul: float = 20.0

    @property
    def scale(self) -> float:
        # softmax scale = 1/sqrt(qk_nope + rope) of the un-absorbed model head
        # (48 = 32 + 16 for the tiny model, 192 = 128 + 64 for the DeepSeekV3/Kimi head)
        return float(np.float32(1.0 / math.sqrt(48.0 if self.d_latent == 64 else 192.0)))


SPECS: Dict[str, Spec] = {
    # tiny fp32 model: random parent array, parent[i] uniform in [-1, i-1]
    "tiny": Spec("tiny", 1, 1, 8, 4, 64, 16, "f32", 32, tree="random"),
    # Kimi/DeepSeekV3 shape, one request, best-first tree of 64 nodes
    "kimi": Spec("kimi", 2, 1, 64, 64, 512, 64, "bf16", 4096, depth=8, topk=8),
    # linear chain of 16 nodes over a long committed cache
    "chain": Spec("chain", 3, 1, 16, 64, 512, 64, "bf16", 32768, tree="chain"),
    # ragged batch of 32 requests with cache lengths uniform in [1024, 16384]
    "ragged": Spec("ragged", 4, 32, 64, 64, 512, 64, "bf16", None, ragged=(1024, 16384),
                   depth=8, topk=8),
    # wide trees: 256 nodes (4 mask words per node), 1% outliers scaled x20
    "wide": Spec("wide", 5, 8, 256, 64, 512, 64, "bf16", 8192, depth=16, topk=16,
                 outlier_p=0.01),
    # supplements: one-node decode over the long cache; the pages' own verify block
    # (budget 7 = block size 8 minus the bonus token)
    "decode": Spec("decode", 6, 1, 1, 64, 512, 64, "bf16", 32768, tree="chain"),
    "block8": Spec("block8", 7, 1, 7, 64, 512, 64, "bf16", 4096, depth=7, topk=8),
    # prefill-shaped chains: a causal chunk of 256 tokens (the most nodes one call takes) over a
    # 4096- and a 32768-token committed cache
    "prefill4k": Spec("prefill4k", 8, 1, 256, 64, 512, 64, "bf16", 4096, tree="chain"),
    "prefill": Spec("prefill", 9, 1, 256, 64, 512, 64, "bf16", 32768, tree="chain"),
}


@dataclasses.dataclass
class Inputs:
    """One verify batch, as CPU torch tensors (bf16 or f32 values; int32 indices)."""
    spec: Spec
    parents: torch.Tensor        # [B, N] int32, -1 = attached to the committed cache
    cache_lens: torch.Tensor     # [B] int32
    q_lat: torch.Tensor          # [B, N, H, d_c]
    q_rope: torch.Tensor         # [B, N, H, d_r]
    kv_cache: torch.Tensor       # [T, d_c + d_r]; latent part then rope part, packed per request
    tree_kv: torch.Tensor        # [B, N, d_c + d_r]
    scale: float                 # an exactly representable fp32 value

    @property
    def ckv(self) -> torch.Tensor:
        return self.kv_cache[:, : self.spec.d_latent]

    @property
    def krope(self) -> torch.Tensor:
        return self.kv_cache[:, self.spec.d_latent:]

    @property
    def tree_ckv(self) -> torch.Tensor:
        return self.tree_kv[:, :, : self.spec.d_latent]

    @property
    def tree_krope(self) -> torch.Tensor:
        return self.tree_kv[:, :, self.spec.d_latent:]

    @property
    def total_len(self) -> int:
        return int(self.cache_lens.sum())


def _rng(spec: Spec, b: int, stream: int, seed: int) -> np.random.Generator:
    return np.random.default_rng([spec.cfg_id, b, stream, seed])


def _normal(spec: Spec, b: int, stream: int, seed: int, shape) -> np.ndarray:
    g = _rng(spec, b, stream, seed)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if spec.outlier_p > 0:
        go = _rng(spec, b, S_OUTLIER * 16 + stream, seed)
        hit = go.random(size=shape, dtype=np.float32) < spec.outlier_p
        x = np.where(hit, x * np.float32(spec.outlier_mul), x)
    return x


def _to_dtype(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    # round-to-nearest-even to bf16, so both paths consume identical bits
    return t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)


def drafter_logprobs(g: np.random.Generator, depth: int, topk: int) -> np.ndarray:
    """Per-depth candidate log-probs, each row sorted in descending order.

    The drafter interface returns one top-k list per depth; logits are N(0, 2^2)."""
    z = g.normal(0.0, 2.0, size=(depth, topk))
    z = z - z.max(axis=1, keepdims=True)
    lp = z - np.log(np.exp(z).sum(axis=1, keepdims=True))
    return -np.sort(-lp, axis=1)


def bestfirst_parents(logp: np.ndarray, budget: int) -> List[int]:
    """Pick the `budget` highest-scoring rank paths best-first; return their parents.

    A node is a path of per-depth ranks (k_1..k_d) scored by the sum of its log-probs.
    Popping order is the node numbering, so a parent is always numbered before its
    children.  Ties break by push order."""
    depth, topk = logp.shape
    heap = [(-logp[0, 0], 0, (0,), -1)]    # (-score, push_no, path, parent index)
    push_no = 1
    parents: List[int] = []
    while heap and len(parents) < budget:
        neg, _, path, par = heapq.heappop(heap)
        me = len(parents)
        parents.append(par)
        d, k = len(path), path[-1]
        if k + 1 < topk:          # next sibling: same prefix, next rank
            sib = path[:-1] + (k + 1,)
            heapq.heappush(heap, (neg + logp[d - 1, k] - logp[d - 1, k + 1], push_no, sib, par))
            push_no += 1
        if d < depth:             # first child: one level deeper, rank 0
            heapq.heappush(heap, (neg - logp[d, 0], push_no, path + (0,), me))
            push_no += 1
    if len(parents) < budget:
        raise ValueError("budget exceeds the number of distinct paths")
    return parents


def make_parents(spec: Spec, seed: int = 0) -> np.ndarray:
    B, N = spec.batch, spec.nodes
    out = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        g = _rng(spec, b, S_TREE, seed)
        if spec.tree == "chain":
            out[b] = np.arange(-1, N - 1, dtype=np.int32)
        elif spec.tree == "star":
            out[b] = -1
        elif spec.tree == "random":
            out[b] = [g.integers(-1, i) for i in range(N)]
        else:
            out[b] = bestfirst_parents(drafter_logprobs(g, spec.depth, spec.topk), N)
    return out


def make_cache_lens(spec: Spec, seed: int = 0) -> np.ndarray:
    if spec.ragged is None:
        return np.full(spec.batch, spec.cache_len, dtype=np.int32)
    lo, hi = spec.ragged
    return np.array([_rng(spec, b, S_LEN, seed).integers(lo, hi, endpoint=True)
                     for b in range(spec.batch)], dtype=np.int32)


def make_inputs(spec, seed: int = 0, cache_lens: Optional[np.ndarray] = None,
                parents: Optional[np.ndarray] = None) -> Inputs:
    """Build one seeded batch.  `spec` is a Spec or a key of SPECS."""
    if isinstance(spec, str):
        spec = SPECS[spec]
    B, N, H, dc, dr = spec.batch, spec.nodes, spec.heads, spec.d_latent, spec.d_rope
    lens = make_cache_lens(spec, seed) if cache_lens is None else np.asarray(cache_lens, np.int32)
    par = make_parents(spec, seed) if parents is None else np.asarray(parents, np.int32)
    q_lat = np.stack([_normal(spec, b, S_QLAT, seed, (N, H, dc)) for b in range(B)])
    q_rope = np.stack([_normal(spec, b, S_QROPE, seed, (N, H, dr)) for b in range(B)])
    kv_rows = []
    for b in range(B):
        L = int(lens[b])
        kv_rows.append(np.concatenate([_normal(spec, b, S_CKV, seed, (L, dc)),
                                       _normal(spec, b, S_KROPE, seed, (L, dr))], axis=1))
    kv = np.concatenate(kv_rows, axis=0) if kv_rows else np.zeros((0, dc + dr), np.float32)
    tkv = np.stack([np.concatenate([_normal(spec, b, S_TCKV, seed, (N, dc)),
                                    _normal(spec, b, S_TKROPE, seed, (N, dr))], axis=1)
                    for b in range(B)])
    return Inputs(spec=spec,
                  parents=torch.from_numpy(par.copy()),
                  cache_lens=torch.from_numpy(lens.copy()),
                  q_lat=_to_dtype(q_lat, spec.dtype),
                  q_rope=_to_dtype(q_rope, spec.dtype),
                  kv_cache=_to_dtype(kv, spec.dtype),
                  tree_kv=_to_dtype(tkv, spec.dtype),
                  scale=spec.scale)


def subset_requests(inp: Inputs, reqs: List[int]) -> Inputs:
    """The same requests, regenerated alone (identical values), in the given order."""
    spec = inp.spec
    offs = np.concatenate([[0], np.cumsum(inp.cache_lens.numpy().astype(np.int64))])
    kv = torch.cat([inp.kv_cache[offs[b]:offs[b + 1]] for b in reqs], dim=0)
    sub = dataclasses.replace(spec, batch=len(reqs))
    return Inputs(spec=sub, parents=inp.parents[reqs].clone(), cache_lens=inp.cache_lens[reqs].clone(),
                  q_lat=inp.q_lat[reqs].clone(), q_rope=inp.q_rope[reqs].clone(),
                  kv_cache=kv.contiguous(), tree_kv=inp.tree_kv[reqs].clone(), scale=inp.scale)


def with_spec(name: str, **kw) -> Spec:
    """A named spec with some fields replaced (small parity cases of the same recipe)."""
    return dataclasses.replace(SPECS[name], **kw)
