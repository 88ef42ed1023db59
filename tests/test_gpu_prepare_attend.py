"""kdt_tree_verify_prepare_attend against the staged calls (prepare, then attend) it replaces,
each followed by combine.

For a one-request batch of bf16 512 + 64 inputs, on 64- or 128-row workgroups, the call works
out the plan unit of every grid slot and the visibility masks inside the attention launch (one
launch); every other batch runs the two stages.  Either way its results must be the staged results bit for bit: the masks, the
outputs, the whole workspace (plan header, offsets, lengths, unit list, split partials) and the
device status.  Both workspaces start zeroed, so bytes nobody writes compare equal too.  The
staged path itself is held to the oracle by the parity tests; one one-launch case is also
checked against the oracle here.  The masks are those of "Validating the Native Engine", section "The Broader
Context"; each output row is the attention of its own root-to-node path ("The Capstone
Validation", section "Context and Motivation")."""
import numpy as np
import pytest
import torch

import oracle
import tree_verify_mla_02_amd as kdt
import workloads
from gpu_helpers import TOL, report, to_device

pytestmark = pytest.mark.gpu

S = workloads.Spec
CASES = {
    "kimi": ("kimi", 3),
    "decode": ("decode", 3),
    "block8": ("block8", 3),
    # 256 nodes x 2 heads = 512 rows: four mask words, four tree tiles
    "n256": (S("fn256", 81, 1, 256, 2, 512, 64, "bf16", 5000, tree="random"), 1),
    # no committed keys: one split, only the tree
    "L0": (S("fL0", 82, 1, 5, 64, 512, 64, "bf16", 0, tree="random"), 1),
    # 40 row tiles, last split partly filled
    "rows2560": (S("f2560", 83, 1, 40, 64, 512, 64, "bf16", None, ragged=(2999, 2999), tree="random"), 1),
    # 8192 rows over 8192 keys: the largest request the 64-row geometry takes
    "rows8192": (S("f8192", 84, 1, 128, 64, 512, 64, "bf16", 8192, depth=12, topk=8), 1),
    # 48 heads: a wave's 32 rows span two nodes; 480 rows, so the last row half is past R
    "h48": (S("fh48", 86, 1, 10, 48, 512, 64, "bf16", 3000, tree="random"), 1),
    # 16 heads (< 32): every workgroup with tree keys builds all masks; a 32-node chain
    "h16chain": (S("fh16", 87, 1, 32, 16, 512, 64, "bf16", 2000, tree="chain"), 1),
    # deep paths on 64-row tiles: a 64-node chain (masks in registers) and a 128-node one (in LDS)
    "chain64": (S("fc64", 90, 1, 64, 64, 512, 64, "bf16", 4096, tree="chain"), 1),
    "chain128": (S("fc128", 91, 1, 128, 64, 512, 64, "bf16", 8192, tree="chain"), 1),
    # 128-row workgroups: the 16-node chain over 32768 keys (32 splits)
    "chain": ("chain", 3),
    # a 256-node causal chunk over 4096 keys: 128 row tiles, 2 splits, four mask words
    "prefill4k": ("prefill4k", 3),
    # 256 random-tree nodes x 4 heads over 20000 keys: 8 row tiles, 256-node masks
    "t128n256": (S("ft128", 88, 1, 256, 4, 512, 64, "bf16", 20000, tree="random"), 1),
    # 1000 rows (last row tile partly filled) over 9000 keys, 8 heads
    "t128rows1000": (S("ft1000", 89, 1, 125, 8, 512, 64, "bf16", 9000, tree="random"), 1),
}


def _inputs(name):
    spec, seed = CASES[name]
    return workloads.make_inputs(spec, seed=seed)


def _run(inp, dev, cache_lens, fused, max_len=None, total_len=None):
    """(masks, out, workspace bytes, status) of one call sequence on zeroed buffers."""
    maxL = int(inp.cache_lens.max()) if max_len is None else max_len
    desc = kdt.make_desc(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, maxL,
                         inp.total_len if total_len is None else total_len)
    ws = torch.zeros(kdt.workspace_size(desc), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.full(dev.q_lat.shape, float("nan"), dtype=torch.float32, device="cuda")
    B, N = dev.parents.shape
    masks = torch.full((B, N, (N + 63) // 64), -1, dtype=torch.int64, device="cuda")
    if fused:
        kdt.prepare_attend(dev.parents, cache_lens, dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv,
                           dev.tree_krope, inp.scale, out, desc, ws, masks_out=masks, dev_status=status)
    else:
        kdt.prepare(dev.parents, cache_lens, desc, ws, masks_out=masks, dev_status=status)
        kdt.attend(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, masks, inp.scale, out,
                   desc, ws)
    kdt.combine(out, desc, ws)
    torch.cuda.synchronize()
    return masks.cpu(), out.cpu(), ws.cpu(), int(status.item()), desc


def _same(a, b, what):
    assert a[0].shape == b[0].shape and torch.equal(a[0], b[0]), f"{what}: masks differ"
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32)), f"{what}: outputs differ"
    diff = (a[2] != b[2]).nonzero()
    assert diff.numel() == 0, f"{what}: workspace differs at {diff[:8].flatten().tolist()}"
    assert a[3] == b[3], f"{what}: status {a[3]} vs {b[3]}"


@pytest.mark.parametrize("name", list(CASES))
def test_fused_equals_staged(name):
    inp = _inputs(name)
    dev = to_device(inp)
    staged = _run(inp, dev, dev.cache_lens, fused=False)
    assert kdt.prepare_attend_launches(staged[4]) == 1, f"{name} should take the one-launch path"
    print(f"case {name}: splits {kdt.num_splits(staged[4])}", flush=True)
    fused = _run(inp, dev, dev.cache_lens, fused=True)
    _same(fused, staged, name)
    assert fused[3] == 0
    for _ in range(2):                          # repeated calls on reused buffers give the same bits
        again = _run(inp, dev, dev.cache_lens, fused=True)
        _same(again, fused, name + " (repeat)")


def test_fused_against_oracle_kimi():
    inp = _inputs("kimi")
    dev = to_device(inp)
    masks, out, _, status, _ = _run(inp, dev, dev.cache_lens, fused=True)
    ref_masks, ref_out, _ = oracle.run(inp)
    assert status == 0
    assert np.array_equal(masks.numpy().view(np.uint64), ref_masks)
    dc = inp.spec.d_latent
    err = float(np.abs(out.double().numpy().reshape(-1, dc) - ref_out.reshape(-1, dc)).max())
    report("kimi-fused", err, TOL["bf16"])
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("base,L", [("kimi", L) for L in (0, 1, 63, 64, 65, 1000, 1024, 1025, 4095)] +
                         [("chain", L) for L in (0, 1, 1023, 1025, 20000, 32767)] +
                         # trees with places in the split range: split 0 = the tree's 128 (256) keys
                         # then committed keys [0, 4032) ([0, 1920)), split 1 the rest
                         [("chain128", L) for L in (0, 1, 4031, 4032, 4033, 8191)] +
                         [("prefill4k", L) for L in (0, 1919, 1920, 1921, 4095)])
def test_fused_shorter_cache(base, L):
    """cache_lens[0] below the bound the geometry was made for: fewer splits, partial splits."""
    inp = _inputs(base)
    dev = to_device(inp)
    maxL = int(inp.cache_lens.max())
    lens = torch.tensor([L], dtype=torch.int32, device="cuda")
    staged = _run(inp, dev, lens, fused=False, max_len=maxL)
    fused = _run(inp, dev, lens, fused=True, max_len=maxL)
    _same(fused, staged, f"{base} L={L}")


@pytest.mark.parametrize("base,lens", [("kimi", [4096, 100, 0, 4095, 1025, 4096]),
                                       ("chain", [32768, 300, 0, 20000, 32767]),
                                       ("chain128", [8192, 4032, 0, 4033, 8192])])
def test_fused_one_workspace_changing_lengths(base, lens):
    """One workspace and one output buffer serve calls with changing cache_lens[0] (fewer splits,
    no cache, back to the full length): every call equals a fresh staged call bit for bit, so
    nothing a previous call left in the workspace (unit slots, partials of splits it had) leaks."""
    inp = _inputs(base)
    dev = to_device(inp)
    maxL = int(inp.cache_lens.max())
    desc = kdt.make_desc(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, maxL,
                         inp.total_len)
    ws = torch.zeros(kdt.workspace_size(desc), dtype=torch.uint8, device="cuda")
    out = torch.empty(dev.q_lat.shape, dtype=torch.float32, device="cuda")
    B, N = dev.parents.shape
    masks = torch.empty((B, N, (N + 63) // 64), dtype=torch.int64, device="cuda")
    for L in lens:
        lt = torch.tensor([L], dtype=torch.int32, device="cuda")
        out.fill_(float("nan"))
        kdt.prepare_attend(dev.parents, lt, dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope,
                           inp.scale, out, desc, ws, masks_out=masks)
        kdt.combine(out, desc, ws)
        torch.cuda.synchronize()
        staged = _run(inp, dev, lt, fused=False, max_len=maxL)
        assert torch.equal(masks.cpu(), staged[0]), f"{base} L={L}: masks differ"
        assert torch.equal(out.cpu().view(torch.int32), staged[1].view(torch.int32)), f"{base} L={L}: outputs differ"
        print(f"PASS {base} L={L}: reused workspace equals a fresh staged call", flush=True)


@pytest.mark.parametrize("base,L", [("kimi", 4097), ("kimi", -1), ("chain", 32769), ("chain", -1)])
def test_fused_rejected_cache_len(base, L):
    """A length outside [0, max_cache_len]: KDT_DEV_CACHE_LEN, outputs untouched, masks still
    written -- as the staged calls do."""
    inp = _inputs(base)
    dev = to_device(inp)
    maxL = int(inp.cache_lens.max())
    lens = torch.tensor([L], dtype=torch.int32, device="cuda")
    staged = _run(inp, dev, lens, fused=False, max_len=maxL)
    fused = _run(inp, dev, lens, fused=True, max_len=maxL)
    _same(fused, staged, f"{base} L={L}")
    assert fused[3] == 2                         # KDT_DEV_CACHE_LEN
    assert torch.isnan(fused[1]).all()


def test_fused_total_len_bound():
    """cache_lens[0] above total_cache_len is rejected like a length above max_cache_len."""
    inp = _inputs("block8")
    dev = to_device(inp)
    staged = _run(inp, dev, dev.cache_lens, fused=False, max_len=4096, total_len=4000)
    fused = _run(inp, dev, dev.cache_lens, fused=True, max_len=4096, total_len=4000)
    _same(fused, staged, "total bound")
    assert fused[3] == 2


@pytest.mark.parametrize("base", ["kimi", "chain"])
def test_fused_bad_parent(base):
    """A parent link outside [-1, j-1]: the rows whose path meets it get zero masks and
    KDT_DEV_BAD_PARENT, as the staged masks do."""
    inp = _inputs(base)
    parents = inp.parents.clone()
    parents[0, 9] = 12                          # not below 9
    parents[0, 14 if base == "chain" else 30] = -7
    inp = workloads.Inputs(inp.spec, parents, inp.cache_lens, inp.q_lat, inp.q_rope, inp.kv_cache, inp.tree_kv,
                           inp.scale)
    dev = to_device(inp)
    staged = _run(inp, dev, dev.cache_lens, fused=False)
    fused = _run(inp, dev, dev.cache_lens, fused=True)
    _same(fused, staged, "bad parent")
    assert fused[3] == 1                         # KDT_DEV_BAD_PARENT
    assert (fused[0][0, 9] == 0).all() and (fused[0][0, 14 if base == "chain" else 30] == 0).all()
    if base == "chain":                         # every later node of the chain passes through 9
        assert (fused[0][0, 9:] == 0).all()


@pytest.mark.parametrize("name", ["t64_ragged", "two_chains", "tiny"])
def test_fused_other_shapes_run_the_stages(name):
    """Batches the one-launch path does not take (several requests on either tile size, fp32)
    give the staged results through the same call (two launches)."""
    spec = {"t64_ragged": S("t64r", 72, 3, 40, 64, 512, 64, "bf16", None, ragged=(0, 3000)),
            "two_chains": S("chs2", 85, 2, 16, 64, 512, 64, "bf16", 20000, tree="chain"),
            "tiny": "tiny"}[name]
    inp = workloads.make_inputs(spec, seed=4)
    dev = to_device(inp)
    staged = _run(inp, dev, dev.cache_lens, fused=False)
    assert kdt.prepare_attend_launches(staged[4]) == 2
    fused = _run(inp, dev, dev.cache_lens, fused=True)
    _same(fused, staged, name)


@pytest.mark.parametrize("base", ["kimi", "chain"])
def test_fused_in_graph(base):
    """prepare_attend + combine captured in a graph and replayed, with eager work between replays."""
    inp = _inputs(base)
    dev = to_device(inp)
    eager = _run(inp, dev, dev.cache_lens, fused=True)
    desc = eager[4]
    ws = torch.zeros(kdt.workspace_size(desc), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.zeros(dev.q_lat.shape, dtype=torch.float32, device="cuda")
    masks = torch.zeros_like(eager[0], device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            kdt.prepare_attend(dev.parents, dev.cache_lens, dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv,
                               dev.tree_krope, inp.scale, out, desc, ws, masks_out=masks, dev_status=status)
            kdt.combine(out, desc, ws)
    torch.cuda.synchronize()
    for k in range(3):
        out.fill_(float("nan"))
        masks.fill_(-1)
        scratch = torch.randn(1 << 20, device="cuda") * 2.0
        graph.replay()
        torch.cuda.synchronize()
        print(f"replay {k}: scratch {float(scratch.sum()):.3f}", flush=True)
        assert torch.equal(out.cpu().view(torch.int32), eager[1].view(torch.int32)), f"replay {k}: outputs differ"
        assert torch.equal(masks.cpu(), eager[0]), f"replay {k}: masks differ"
    assert int(status.item()) == 0
