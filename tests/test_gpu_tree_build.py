"""GPU parity of the best-first tree builder (kdt_build_tree, through the C ABI) against the
CPU oracle (oracle/tree_build.py).  The builder's output is integer: parents, tokens, depths
and ranks must match bit for bit, ties included (both sides score paths in fp32, one rounding
per depth, and break equal scores by push order).  Every case prints its name before it runs."""
import json
import zlib
import os

import numpy as np
import pytest
import torch

import tree_verify_mla_02_amd as kdt
import workloads
from oracle import tree_build as ref
import oracle

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DEV = torch.device("cuda", 0)


def drafter(seed, B, D, K, quantum=None):
    """Per request and depth: K log probabilities sorted descending (logits N(0, 2^2)), and
    token ids.  With `quantum`, log probabilities are rounded to multiples of it, which makes
    equal path scores common (the tie-break is then exercised on every tree)."""
    rng = np.random.default_rng(seed)
    lp = np.stack([workloads.drafter_logprobs(rng, D, K) for _ in range(B)]).astype(np.float32)
    if quantum is not None:
        lp = (np.round(lp / quantum) * quantum).astype(np.float32)
        lp = -np.sort(-lp, axis=-1)
    cand = rng.integers(0, 160000, size=(B, D, K)).astype(np.int32)
    return np.ascontiguousarray(lp), np.ascontiguousarray(cand)


def run_gpu(lp, cand, N):
    outs = kdt.build_tree(torch.as_tensor(lp, device=DEV), torch.as_tensor(cand, device=DEV), N)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


def assert_tree_equal(lp, cand, N):
    got = run_gpu(lp, cand, N)
    want = ref.best_first_tree(lp, cand, N)
    for g, w, name in zip(got, want, ("parents", "tokens", "depth", "rank")):
        np.testing.assert_array_equal(g, w, err_msg=name)
    return got


def test_tree_handworked_fixture():
    cases = json.load(open(os.path.join(GOLDEN, "tree_build_handworked.json")))["cases"]
    for c in cases:
        print("case tree fixture", c["name"], flush=True)
        lp = np.array([c["logp"]], np.float32)
        cd = np.array([c["cand"]], np.int32)
        par, tok, dep, rk = run_gpu(lp, cd, c["N"])
        assert par[0].tolist() == c["parents"]
        assert tok[0].tolist() == c["tokens"]
        assert dep[0].tolist() == c["depth"]
        assert rk[0].tolist() == c["rank"]


@pytest.mark.parametrize("name,B,D,K,N", [
    ("kimi: 1 request, depth 8, top-8, 64 nodes", 1, 8, 8, 64),
    ("ragged: 32 requests, depth 8, top-8, 64 nodes", 32, 8, 8, 64),
    ("wide: 8 requests, depth 16, top-16, 256 nodes", 8, 16, 16, 256),
    ("block8: depth 7, top-8, 7 nodes", 4, 7, 8, 7),
    ("one node", 3, 5, 5, 1),
    ("depth 1: a star of K nodes", 2, 1, 64, 64),
    ("top-1: a chain", 2, 40, 1, 40),
    ("deep and narrow, 256 nodes", 2, 256, 2, 256),
    ("wide table, 256 nodes", 2, 8, 1024, 256),
])
def test_tree_matches_oracle(name, B, D, K, N):
    print("case tree", name, flush=True)
    lp, cand = drafter(zlib.crc32(name.encode()) % 1000, B, D, K)
    assert_tree_equal(lp, cand, N)


@pytest.mark.parametrize("quantum", [0.5, 0.25, 2.0])
def test_tree_ties_break_by_push_order(quantum):
    print(f"case tree ties, log probabilities in steps of {quantum}", flush=True)
    lp, cand = drafter(int(quantum * 100), 16, 6, 6, quantum=quantum)
    assert_tree_equal(lp, cand, 128)
    lp, cand = drafter(7, 4, 16, 16, quantum=quantum)
    assert_tree_equal(lp, cand, 256)


def test_tree_signed_zeros_and_minus_inf():
    print("case tree with -0.0, 0.0 and -inf log probabilities", flush=True)
    rng = np.random.default_rng(3)
    B, D, K = 6, 6, 5
    lp = np.zeros((B, D, K), np.float32)
    lp[:, :, 0] = np.where(rng.random((B, D)) < 0.5, -0.0, 0.0)
    lp[:, :, 1] = np.where(rng.random((B, D)) < 0.5, -0.0, 0.0)
    lp[:, :, 2] = -1.0
    lp[:, :, 3:] = -np.inf
    cand = rng.integers(0, 1000, size=(B, D, K)).astype(np.int32)
    assert_tree_equal(lp, cand, 200)


def test_tree_exhausted_frontier():
    print("case tree with fewer paths than nodes (rows filled with -2)", flush=True)
    lp, cand = drafter(11, 3, 3, 2, None)        # 2 + 4 + 8 = 14 paths
    par, tok, dep, rk = assert_tree_equal(lp, cand, 20)
    assert (par[:, 14:] == -2).all() and (par[:, :14] >= -1).all()


@pytest.mark.parametrize("seed", range(4))
def test_tree_random_shapes(seed):
    rng = np.random.default_rng(100 + seed)
    for _ in range(6):
        B = int(rng.integers(1, 9))
        D = int(rng.integers(1, 20))
        K = int(rng.integers(1, 20))
        N = int(rng.integers(1, 257))
        print(f"case tree random B={B} D={D} K={K} N={N}", flush=True)
        lp, cand = drafter(int(rng.integers(1 << 30)), B, D, K)
        assert_tree_equal(lp, cand, N)


def test_tree_feeds_the_visibility_masks():
    """The built parents go straight into the mask builder: masks equal the oracle's masks
    of the oracle's parents, bit for bit."""
    print("case tree -> visibility masks (wide shape)", flush=True)
    lp, cand = drafter(5, 8, 16, 16)
    par_d, _, _, _ = kdt.build_tree(torch.as_tensor(lp, device=DEV), torch.as_tensor(cand, device=DEV), 256)
    masks = kdt.build_visibility(par_d)
    torch.cuda.synchronize()
    par_ref = ref.best_first_tree(lp, cand, 256)[0]
    want, bad = oracle.visibility(par_ref)
    assert bad == 0
    np.testing.assert_array_equal(masks.cpu().numpy().view(np.uint64), want)


def test_tree_host_errors():
    print("case tree host-side errors", flush=True)
    lp = torch.zeros((1, 4, 4), dtype=torch.float32, device=DEV)
    cand = torch.zeros((1, 4, 4), dtype=torch.int32, device=DEV)
    with pytest.raises(kdt.KdtError):
        kdt.build_tree(lp, cand, 0)
    with pytest.raises(kdt.KdtError):
        kdt.build_tree(lp, cand, 257)
    big = torch.zeros((1, 2, 8193), dtype=torch.float32, device=DEV)
    with pytest.raises(kdt.KdtError):
        kdt.build_tree(big, torch.zeros_like(big, dtype=torch.int32), 8)
