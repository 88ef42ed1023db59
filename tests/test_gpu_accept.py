"""GPU parity of the greedy tree-accept and KV-compaction kernels (through the C ABI)
against the CPU oracle (oracle/accept.py).  Both are integer / copy work: results must match
bit for bit.  Every case prints its name before it runs."""
import json
import os

import numpy as np
import pytest
import torch

import tree_verify_mla_02_amd as kdt
import workloads
from oracle import accept as ref

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DEV = torch.device("cuda", 0)


def i32(x):
    return torch.as_tensor(np.ascontiguousarray(np.asarray(x, dtype=np.int32)), device=DEV)


def run_accept(par, tok, nxt, root):
    path, acc, bonus = kdt.tree_accept(i32(par), i32(tok), i32(nxt), i32(root))
    torch.cuda.synchronize()
    return path.cpu().numpy(), acc.cpu().numpy(), bonus.cpu().numpy()


def assert_accept_equal(par, tok, nxt, root):
    got = run_accept(par, tok, nxt, root)
    want = ref.tree_accept(par, tok, nxt, root)
    for g, w, name in zip(got, want, ("path", "accept_len", "bonus")):
        np.testing.assert_array_equal(g, w, err_msg=name)
    return got


def guided_predictions(rng, par, tok, hit=0.85):
    """Target predictions that follow a random root-to-leaf walk with probability `hit` at
    each step (so that long paths get accepted), anything else otherwise."""
    B, N = par.shape
    nxt = rng.integers(0, 1 << 20, size=(B, N))
    root = rng.integers(0, 1 << 20, size=B)
    for b in range(B):
        kids = [[j for j in range(N) if par[b, j] == i] for i in range(-1, N)]
        cur = -1
        while kids[cur + 1] and rng.random() < hit:
            j = int(rng.choice(kids[cur + 1]))
            if cur < 0:
                root[b] = tok[b, j]
            else:
                nxt[b, cur] = tok[b, j]
            cur = j
    return nxt, root


def test_accept_handworked_fixture():
    cases = json.load(open(os.path.join(GOLDEN, "accept_handworked.json")))["cases"]
    print("case accept handworked fixture", flush=True)
    par = np.array([c["parents"] + [-1] * (8 - len(c["parents"])) for c in cases])
    # pad short trees with extra depth-1 nodes whose token matches nothing
    tok = np.array([c["tokens"] + [-7] * (8 - len(c["tokens"])) for c in cases])
    nxt = np.array([c["target_next"] + [-9] * (8 - len(c["target_next"])) for c in cases])
    root = np.array([c["root_next"] for c in cases])
    path, acc, bonus = assert_accept_equal(par, tok, nxt, root)
    for b, c in enumerate(cases):
        assert path[b, :acc[b]].tolist() == c["path"] and int(bonus[b]) == c["bonus"]


@pytest.mark.parametrize("name", ["kimi", "ragged", "wide", "block8", "chain", "tiny", "decode"])
def test_accept_on_workload_trees(name):
    inp = workloads.make_inputs(name, seed=0)
    par = inp.parents.numpy()
    B, N = par.shape
    print(f"case accept {name}: B={B} N={N}", flush=True)
    rng = np.random.default_rng(11)
    # distinct sibling tokens (as a tree builder gives), guided predictions
    tok = rng.permutation(B * N * 4)[: B * N].reshape(B, N)
    nxt, root = guided_predictions(rng, par, tok)
    _, acc, _ = assert_accept_equal(par, tok, nxt, root)
    print(f"  accept lengths: max {int(acc.max())}, mean {float(acc.mean()):.2f}", flush=True)


@pytest.mark.parametrize("seed", range(6))
def test_accept_random_trees_with_repeated_tokens(seed):
    rng = np.random.default_rng(seed)
    B, N = 48, int(rng.integers(1, 257))
    print(f"case accept random repeated-token trees: seed {seed} B={B} N={N}", flush=True)
    par = np.stack([[-1] + [int(rng.integers(-1, i)) for i in range(1, N)] for _ in range(B)])
    tok = rng.integers(0, 3, size=(B, N))
    nxt = rng.integers(0, 3, size=(B, N))
    root = rng.integers(0, 3, size=B)
    assert_accept_equal(par, tok, nxt, root)


def test_accept_edges():
    print("case accept edges: N=1, a 256-node chain accepted whole, nothing accepted, malformed parents",
          flush=True)
    # N = 1
    assert_accept_equal(np.array([[-1], [-1]]), np.array([[4], [4]]), np.array([[8], [9]]), np.array([4, 5]))
    # a 256-node chain, every node accepted
    N = 256
    par = np.arange(-1, N - 1)[None]
    tok = np.arange(N)[None] + 100
    nxt = (np.arange(N)[None] + 101)
    path, acc, bonus = assert_accept_equal(par, tok, nxt, np.array([100]))
    assert int(acc[0]) == N and int(bonus[0]) == 100 + N
    # parents pointing forward or at themselves are never followed (the walk still ends)
    par = np.array([[-1, 5, 1, 3, -1, 0]])
    tok = np.array([[1, 2, 3, 4, 5, 6]])
    nxt = np.array([[2, 3, 4, 5, 6, 7]])
    assert_accept_equal(par, tok, nxt, np.array([1]))


# ------------------------------------------------------------------------------ compaction
def compact_case(rng, B, N, lens, dtype, acc=None):
    dc, dr = (512, 64) if dtype == torch.bfloat16 else (64, 16)
    D = dc + dr
    lens = np.asarray(lens, np.int64)
    T = int(lens.sum())
    kv = torch.randn(max(T, 1), D, generator=torch.Generator().manual_seed(int(rng.integers(1 << 30)))).to(dtype)
    tkv = torch.randn(B, N, D, generator=torch.Generator().manual_seed(int(rng.integers(1 << 30)))).to(dtype)
    if acc is None:
        acc = rng.integers(0, min(N, 9) + 1, size=B)
    path = np.full((B, N), -1, np.int64)
    for b in range(B):
        path[b, :acc[b]] = rng.choice(N, size=acc[b], replace=False)
    return kv, tkv, lens, np.asarray(acc), path, dc


def bits(t):
    """Integer view of a bf16 / fp32 tensor (the oracle copies rows; bits compare exactly)."""
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).numpy()


def desc_for(kv, tkv, B, N, dc, maxL, total):
    q_lat = torch.empty((B, N, 1, dc), dtype=kv.dtype, device=DEV)
    q_rope = torch.empty((B, N, 1, kv.shape[1] - dc), dtype=kv.dtype, device=DEV)
    return kdt.make_desc(q_lat, q_rope, kv[:, :dc], kv[:, dc:], tkv[:, :, :dc], tkv[:, :, dc:], maxL, total)


def run_compact(kv, tkv, lens, acc, path, dc, in_place=False, capacity=None, status=None):
    B, N = path.shape
    kv_d, tkv_d = kv.to(DEV), tkv.to(DEV)
    T = int(lens.sum())
    rows = T + int(acc.sum())
    if in_place:
        buf = torch.zeros((max(rows, 1), kv.shape[1]), dtype=kv.dtype, device=DEV)
        buf[:T] = kv_d[:T]
        src = out = buf
    else:
        src = kv_d
        out = torch.full((max(rows, 1) + 3, kv.shape[1]), 7, dtype=kv.dtype, device=DEV)
    desc = desc_for(src, tkv_d, B, N, dc, int(lens.max()) if B else 0, T)
    new_lens = torch.full((B,), -5, dtype=torch.int32, device=DEV)
    kdt.kv_compact(src[:, :dc], src[:, dc:], i32(lens), tkv_d[:, :, :dc], tkv_d[:, :, dc:], i32(path), i32(acc),
                   desc, out[:, :dc], out[:, dc:], new_lens=new_lens,
                   capacity_rows=capacity if capacity is not None else out.shape[0], dev_status=status)
    torch.cuda.synchronize()
    return out.cpu(), new_lens.cpu().numpy()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("lens", [[37], [0], [5, 0, 130, 64], [1024, 3, 77, 256, 1, 999, 64, 65]])
def test_compact_matches_oracle(dtype, lens):
    rng = np.random.default_rng(len(lens) * 7 + sum(lens))
    B, N = len(lens), 64
    print(f"case compact {dtype} lens={lens}", flush=True)
    kv, tkv, lens_a, acc, path, dc = compact_case(rng, B, N, lens, dtype)
    out, new_lens = run_compact(kv, tkv, lens_a, acc, path, dc)
    T = int(lens_a.sum())
    kb, tb = bits(kv[:T]), bits(tkv)
    wc, wr, wl = ref.kv_compact(kb[:, :dc], kb[:, dc:], lens_a, tb[:, :, :dc], tb[:, :, dc:], path, acc)
    rows = wc.shape[0]
    np.testing.assert_array_equal(new_lens, wl)
    got = bits(out)
    np.testing.assert_array_equal(got[:rows, :dc], wc)
    np.testing.assert_array_equal(got[:rows, dc:], wr)
    # rows past the new cache are untouched
    assert torch.equal(out[rows:], torch.full_like(out[rows:], 7))


def test_compact_in_place_single_request():
    rng = np.random.default_rng(4)
    print("case compact in place: B=1 L=4096 N=64", flush=True)
    kv, tkv, lens, acc, path, dc = compact_case(rng, 1, 64, [4096], torch.bfloat16, acc=np.array([8]))
    out, new_lens = run_compact(kv, tkv, lens, acc, path, dc, in_place=True)
    assert new_lens.tolist() == [4104]
    kb, tb = bits(kv), bits(tkv)
    wc, wr, _ = ref.kv_compact(kb[:, :dc], kb[:, dc:], lens, tb[:, :, :dc], tb[:, :, dc:], path, acc)
    got = bits(out)
    np.testing.assert_array_equal(got[:, :dc], wc)
    np.testing.assert_array_equal(got[:, dc:], wr)


def test_compact_after_accept_on_the_ragged_workload():
    """The two steps chained on the ragged batch's own lengths and trees."""
    inp = workloads.make_inputs("ragged", seed=0)
    par = inp.parents.numpy()
    B, N = par.shape
    print(f"case accept + compact, ragged: B={B} N={N} T={inp.total_len}", flush=True)
    rng = np.random.default_rng(2)
    tok = rng.permutation(B * N * 4)[: B * N].reshape(B, N)
    nxt, root = guided_predictions(rng, par, tok)
    path, acc, _ = run_accept(par, tok, nxt, root)
    lens = inp.cache_lens.numpy().astype(np.int64)
    dc = inp.spec.d_latent
    out, new_lens = run_compact(inp.kv_cache, inp.tree_kv, lens, acc.astype(np.int64), path.astype(np.int64), dc)
    np.testing.assert_array_equal(new_lens, lens + acc)
    # check every accepted row and the committed rows at each request's edges
    off_old = np.concatenate([[0], np.cumsum(lens)])
    off_new = np.concatenate([[0], np.cumsum(lens + acc)])
    kv16, tkv16, out16 = (t.view(torch.int16) for t in (inp.kv_cache, inp.tree_kv, out))
    for b in range(B):
        for r in (0, lens[b] - 1):
            if lens[b] > 0:
                assert torch.equal(out16[off_new[b] + r], kv16[off_old[b] + r])
        for k in range(acc[b]):
            assert torch.equal(out16[off_new[b] + lens[b] + k], tkv16[b, path[b, k]])


def test_compact_rejects_bad_device_inputs():
    rng = np.random.default_rng(9)
    print("case compact bad inputs: bad length, bad path entry, capacity too small", flush=True)
    kv, tkv, lens, acc, path, dc = compact_case(rng, 3, 16, [10, 20, 30], torch.bfloat16, acc=np.array([2, 3, 1]))
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    # accept_len above N: nothing written
    bad_acc = acc.copy()
    bad_acc[1] = 17
    out, new_lens = run_compact(kv, tkv, lens, bad_acc, path, dc, status=status)
    assert int(status.item()) == kdt._lib.KDT_DEV_BAD_ACCEPT
    assert (new_lens == -5).all() and torch.equal(out, torch.full_like(out, 7))
    # a path entry naming no node: only that request is left unwritten
    status.zero_()
    bad_path = path.copy()
    bad_path[2, 0] = 99
    out, new_lens = run_compact(kv, tkv, lens, acc, bad_path, dc, status=status)
    assert int(status.item()) == kdt._lib.KDT_DEV_BAD_ACCEPT
    assert new_lens.tolist()[:2] == [12, 23] and int(new_lens[2]) == -5
    # destination too small: nothing written
    status.zero_()
    out, new_lens = run_compact(kv, tkv, lens, acc, path, dc, capacity=int(lens.sum() + acc.sum()) - 1,
                                status=status)
    assert int(status.item()) == kdt._lib.KDT_DEV_BAD_ACCEPT
    assert (new_lens == -5).all() and torch.equal(out, torch.full_like(out, 7))
