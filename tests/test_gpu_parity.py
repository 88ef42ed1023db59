"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Masks must match bit for bit.  Outputs must match within max-abs 2e-3 for bf16 inputs
(fp32 accumulate) and 1e-5 for fp32 inputs.  Every case prints a PASS/FAIL line with its
error.  Every case compares every output row.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import tree_verify_mla_02_amd as kdt
import workloads
from gpu_helpers import TOL, report, run_gpu, to_device

pytestmark = pytest.mark.gpu


def check(name, inp, rows=None, staged=False, dev=None):
    print(f"case {name}: B={inp.spec.batch} N={inp.spec.nodes} H={inp.spec.heads} "
          f"d=({inp.spec.d_latent},{inp.spec.d_rope}) {inp.spec.dtype} T={inp.total_len}", flush=True)
    masks, out, status = run_gpu(inp, dev=dev, staged=staged)
    ref_masks, bad = oracle.visibility(inp.parents.numpy())
    np.testing.assert_array_equal(masks, ref_masks)
    assert status == (kdt._lib.KDT_DEV_BAD_PARENT if bad else 0)
    dc = inp.spec.d_latent
    got = out.reshape(-1, dc).cpu().double().numpy()
    ref = oracle.run(inp, rows=rows)[1].reshape(-1, dc)
    if rows is not None:
        got = got[rows]
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    tol = TOL[inp.spec.dtype]
    report(name, err, tol)
    assert err <= tol
    return out


# ------------------------------------------------------------------ the workload configs
@pytest.mark.parametrize("name", ["tiny", "kimi", "chain", "ragged", "wide", "decode", "block8"])
def test_config_all_rows(name):
    """Every output row of every workload config against the oracle (ragged and wide take about
    half a minute of oracle time on 16 host threads)."""
    check(name, workloads.make_inputs(name, seed=0))


def test_kimi_second_seed_staged():
    inp = workloads.make_inputs("kimi", seed=1)
    check("kimi-seed1-staged", inp, staged=True)


# ------------------------------------------------------------------ small multi-tile cases (all rows)
SMALL = {
    # ragged tails everywhere: an empty cache, partial key tiles, a partial row tile
    "ragged3": (workloads.Spec("ragged3", 40, 3, 20, 8, 512, 64, "bf16", None, ragged=(0, 300), tree="random"),
                [0, 100, 257]),
    # two mask words; H=3 so 32-row wave slices straddle nodes
    "nodes65": (workloads.Spec("nodes65", 41, 2, 65, 3, 512, 64, "bf16", None, ragged=(1, 2000), tree="random"),
                [64, 1000]),
    # 256 nodes = four mask words, best-first tree
    "nodes256": (workloads.Spec("nodes256", 42, 1, 256, 2, 512, 64, "bf16", 300, depth=16, topk=16), None),
    # one request, few rows, long cache: split over many workgroups + combine, partial last split
    "split": (workloads.Spec("split", 43, 1, 8, 16, 512, 64, "bf16", 3000, tree="random"), None),
    "split_outliers": (workloads.Spec("split_o", 44, 2, 16, 8, 512, 64, "bf16", None, ragged=(500, 2500),
                                      outlier_p=0.01, depth=16, topk=16), None),
    "bf16_small_dims": (workloads.Spec("bsd", 45, 2, 9, 5, 64, 16, "bf16", None, ragged=(3, 80), tree="random"),
                        [77, 3]),
    "f32_ragged": (workloads.Spec("f32r", 46, 3, 30, 4, 64, 16, "f32", None, ragged=(0, 200), tree="random"),
                   [0, 65, 200]),
    "f32_split": (workloads.Spec("f32s", 47, 1, 8, 4, 64, 16, "f32", 5000, tree="random"), None),
    "star": (workloads.Spec("star", 48, 2, 12, 8, 512, 64, "bf16", 130, tree="star"), None),
    "chain_short": (workloads.Spec("chs", 49, 1, 16, 64, 512, 64, "bf16", 1000, tree="chain"), None),
    # at most 64 rows per request (the decode-shape kernel): one node x 64 heads over ragged
    # lengths, an empty cache and tails of one key; 40 rows (a partial second row half); a
    # 60-node tree of one head (tree keys in both 32-key halves of the tile); outliers; and
    # enough requests that keys are not split (outputs written by the attention kernel itself)
    "dec_ragged": (workloads.Spec("dec_r", 60, 5, 1, 64, 512, 64, "bf16", None, ragged=(0, 3000), tree="chain"),
                   [0, 1, 65, 1000, 2999]),
    "dec_rows40": (workloads.Spec("dec_40", 61, 2, 5, 8, 512, 64, "bf16", None, ragged=(1, 1500), tree="random"),
                   [1, 1500]),
    "dec_tree60": (workloads.Spec("dec_t60", 62, 1, 60, 1, 512, 64, "bf16", 700, depth=8, topk=8), None),
    "dec_outliers": (workloads.Spec("dec_o", 63, 2, 1, 64, 512, 64, "bf16", 5000, tree="chain", outlier_p=0.01),
                     None),
    "dec_unsplit": (workloads.Spec("dec_u", 64, 600, 1, 64, 512, 64, "bf16", None, ragged=(1, 200), tree="chain"),
                    None),
    # small requests in a batch that fills the GPU: 128-row workgroups, no split
    "batch300": (workloads.Spec("b300", 65, 300, 2, 64, 512, 64, "bf16", None, ragged=(1, 300), tree="random"), None),
    # 1000 rows over short caches: 64-row workgroups (16 row tiles, the last partial), two mask
    # words, a split
    "rows1000": (workloads.Spec("r1000", 66, 2, 125, 8, 512, 64, "bf16", None, ragged=(700, 2600), depth=10, topk=6),
                 None),
    # the same rows over a long cache: 128-row workgroups with a partial last tile
    "rows1000_long": (workloads.Spec("r1000l", 67, 1, 125, 8, 512, 64, "bf16", 9000, depth=10, topk=6), None),
    # mid-size trees over short ragged caches (64-row workgroups beyond 512 rows): 2560 rows a
    # request, an empty cache and a one-key tail; 888 rows (a partial 64-row tile, H = 24 so
    # 32-row slices straddle nodes), outliers
    "t64_ragged": (workloads.Spec("t64r", 72, 3, 40, 64, 512, 64, "bf16", None, ragged=(0, 3000), depth=8, topk=8),
                   [0, 1, 2999]),
    "t64_rows888": (workloads.Spec("t64p", 73, 2, 37, 24, 512, 64, "bf16", None, ragged=(100, 5000), tree="random",
                                   outlier_p=0.01), [5000, 777]),
    # 128 heads (the DeepSeek-V3 count): over a short cache a 64-row tile is half of a node's
    # heads; over a long one a 128-row tile is one node
    "h128_t64": (workloads.Spec("h128a", 68, 1, 32, 128, 512, 64, "bf16", 3000, depth=6, topk=8), None),
    "h128_t128": (workloads.Spec("h128b", 69, 1, 32, 128, 512, 64, "bf16", 10000, depth=6, topk=8), None),
    # the 64-row kernel's 16x16x32 S^T chain (key splits of at least 1024 keys): the Kimi shape
    # with outliers, so that softmax references move; and 2048 rows over 8192 keys (8 splits)
    "kimi_outliers": (workloads.Spec("kimi_o", 74, 1, 64, 64, 512, 64, "bf16", 4096, outlier_p=0.01), None),
    "qk16_s8": (workloads.Spec("q16s8", 75, 1, 32, 64, 512, 64, "bf16", 8192, tree="random", outlier_p=0.005),
                None),
    # the same chain with a partial last row tile (4000 rows) and a two-tile tree whose keys have
    # places in the split range (125 nodes: 5 splits of 1216 keys)
    "qk16_partial": (workloads.Spec("q16p", 76, 1, 125, 32, 512, 64, "bf16", 6000, tree="random"), None),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_all_rows(name):
    spec, lens = SMALL[name]
    inp = workloads.make_inputs(spec, seed=0, cache_lens=None if lens is None else np.array(lens, np.int32))
    check(name, inp)


@pytest.mark.parametrize("name", ["split", "nodes256", "chain_short", "dec_tree60", "rows1000_long", "h128_t64",
                                  "h128_t128", "kimi_outliers", "qk16_partial"])
def test_small_one_launch(name):
    """The one-request cases through kdt_tree_verify_prepare_attend (masks, plan and attention in
    one launch), every row against the oracle."""
    spec, lens = SMALL[name]
    inp = workloads.make_inputs(spec, seed=0, cache_lens=None if lens is None else np.array(lens, np.int32))
    check(name + " (one launch)", inp, staged="one")


def test_chain_equals_causal_prefill_on_gpu():
    """A chain tree over a cache is causal prefill over cache ++ chain (torch SDPA, fp64)."""
    spec = workloads.Spec("chsdpa", 50, 1, 16, 4, 512, 64, "bf16", 700, tree="chain")
    inp = workloads.make_inputs(spec, seed=0)
    _, out, _ = run_gpu(inp)
    L, N = 700, 16
    k = torch.cat([inp.kv_cache, inp.tree_kv[0]]).double()
    q = torch.cat([inp.q_lat[0], inp.q_rope[0]], -1).double().permute(1, 0, 2)   # [H, N, D]
    causal = torch.arange(L + N)[None, :] <= (L + torch.arange(N))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        q[None], k[None, None].expand(1, 4, -1, -1), k[None, None, :, :512].expand(1, 4, -1, -1),
        attn_mask=causal, scale=inp.scale)[0].permute(1, 0, 2)
    err = float((out[0].cpu().double() - ref).abs().max())
    report("chain==causal-prefill", err, TOL["bf16"])
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("name", ["tiny", "kimi", "block8", "wide"])
def test_prepare_equals_separate_calls(name):
    """kdt_tree_verify_prepare (masks + plan in one launch) gives the same masks, status and
    outputs, bit for bit, as kdt_build_visibility + kdt_tree_verify_plan; and passes parity."""
    inp = workloads.make_inputs(name, seed=3)
    if name == "wide":
        inp = workloads.subset_requests(inp, [0, 5])
    dev = to_device(inp)
    m1, o1, s1 = run_gpu(inp, dev=dev, staged=True)
    m2, o2, s2 = run_gpu(inp, dev=dev, staged="prepare")
    np.testing.assert_array_equal(m1, m2)
    assert s1 == s2
    assert torch.equal(o1, o2)
    check(f"{name}-prepare", inp, staged="prepare", dev=dev)


def test_prepare_flags_bad_parents_and_lengths():
    spec = workloads.Spec("prepbad", 53, 2, 8, 4, 512, 64, "bf16", 100, tree="random")
    par = workloads.make_parents(spec, 0)
    par[1, 4] = 4          # its own parent
    inp = workloads.make_inputs(spec, seed=0, parents=par)
    masks, _, status = run_gpu(inp, staged="prepare")
    assert status & kdt._lib.KDT_DEV_BAD_PARENT
    ref_masks, bad = oracle.visibility(inp.parents.numpy())
    assert bad > 0
    np.testing.assert_array_equal(masks, ref_masks)


# ------------------------------------------------------------------ edge cases and properties
def test_invalid_parents_flag_and_zero_rows():
    spec = workloads.Spec("badpar", 51, 2, 8, 4, 512, 64, "bf16", 100, tree="random")
    par = workloads.make_parents(spec, 0)
    par[0, 3] = 5          # parent after child
    par[1, 6] = -7         # below -1
    inp = workloads.make_inputs(spec, seed=0, parents=par)
    masks, _, status = run_gpu(inp)
    assert status & kdt._lib.KDT_DEV_BAD_PARENT
    check("invalid-parents", inp)      # oracle zeroes the same rows


def test_invalid_cache_lens_leave_out_untouched():
    spec = workloads.Spec("badlen", 52, 2, 8, 4, 512, 64, "bf16", 100, tree="random")
    inp = workloads.make_inputs(spec, seed=0)
    dev = to_device(inp)
    masks = kdt.build_visibility(dev.parents)
    for lens, maxL in (([100, 101], 100), ([-1, 100], 100), ([100, 100], 100)):
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        out = torch.full(dev.q_lat.shape, 7.0, dtype=torch.float32, device="cuda")
        total = 150 if lens == [100, 100] else 200        # the last case overflows the packed rows
        kdt.tree_verify_attn(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, masks,
                             torch.tensor(lens, dtype=torch.int32, device="cuda"), inp.scale, out=out,
                             dev_status=status, max_cache_len=maxL, total_cache_len=total)
        torch.cuda.synchronize()
        assert int(status.item()) & kdt._lib.KDT_DEV_CACHE_LEN, lens
        assert bool((out == 7.0).all()), lens
    print("PASS invalid-cache-lens: flagged, out untouched", flush=True)


def test_invisible_nodes_do_not_matter():
    """Perturbing the tree rows of siblings / descendants / cousins of node i leaves out[i] bit-identical."""
    spec = workloads.Spec("invis", 53, 1, 40, 8, 512, 64, "bf16", 300, depth=6, topk=4)
    inp = workloads.make_inputs(spec, seed=0)
    masks, base, _ = run_gpu(inp)
    par = inp.parents.numpy()[0]
    rng = np.random.default_rng(0)
    for i in rng.choice(40, size=6, replace=False):
        anc, j = set(), int(i)
        while j != -1:
            anc.add(j)
            j = int(par[j])
        others = [j for j in range(40) if j not in anc]
        pert = dataclasses.replace(inp, tree_kv=inp.tree_kv.clone())
        pert.tree_kv[0, others] = (torch.randn(len(others), 576) * 3).to(torch.bfloat16)
        _, out2, _ = run_gpu(pert)
        assert torch.equal(out2[0, i], base[0, i]), i
    print("PASS invisibility: outputs bit-identical under perturbation of invisible nodes", flush=True)


def test_deterministic_and_permutation_exact():
    inp = workloads.make_inputs(dataclasses.replace(workloads.SPECS["ragged"], batch=6), seed=2)
    _, a, _ = run_gpu(inp)
    _, b, _ = run_gpu(inp)
    assert torch.equal(a, b)
    perm = [3, 0, 5, 1, 4, 2]
    _, c, _ = run_gpu(workloads.subset_requests(inp, perm))
    assert torch.equal(c, a[perm])
    print("PASS determinism + request permutation: bit-identical", flush=True)


def test_request_alone_matches_batch():
    inp = workloads.make_inputs(dataclasses.replace(workloads.SPECS["ragged"], batch=4), seed=3)
    _, full, _ = run_gpu(inp)
    for b in range(4):
        _, solo, _ = run_gpu(workloads.subset_requests(inp, [b]))
        err = float((solo[0] - full[b]).abs().max())
        assert err <= TOL["bf16"], (b, err)
    print("PASS request independence", flush=True)


def test_abi_errors_on_device():
    inp = workloads.make_inputs("tiny", seed=0)
    dev = to_device(inp)
    masks = kdt.build_visibility(dev.parents)
    desc = kdt.make_desc(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, 32)
    ws = kdt.alloc_workspace(desc)
    out = torch.empty(dev.q_lat.shape, dtype=torch.float32, device="cuda")
    with pytest.raises(kdt.KdtError) as e:                      # workspace too small
        kdt.plan(dev.cache_lens, desc, ws[:16], None)
    assert e.value.code == kdt._lib.KDT_ERR_WORKSPACE
    with pytest.raises(kdt.KdtError) as e:                      # misaligned pointer
        kdt.attend(dev.q_lat.view(-1)[1:].view(-1)[: dev.q_lat.numel() - 1], dev.q_rope, dev.ckv, dev.krope,
                   dev.tree_ckv, dev.tree_krope, masks, inp.scale, out, desc, ws)
    assert e.value.code == kdt._lib.KDT_ERR_MISALIGNED
    bad = kdt.make_desc(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, 32)
    bad.d_latent = 128
    with pytest.raises(kdt.KdtError) as e:
        kdt.workspace_size(bad)
    assert e.value.code == kdt._lib.KDT_ERR_UNSUPPORTED
    with pytest.raises(kdt.KdtError) as e:
        kdt.build_visibility(torch.zeros((1, 257), dtype=torch.int32, device="cuda"))
    assert e.value.code == kdt._lib.KDT_ERR_UNSUPPORTED
    print("PASS ABI error paths", flush=True)


@pytest.mark.parametrize("seed", range(4))
def test_random_small_requests(seed):
    """Random small batches (at most 512 rows per request, so they take 64-row workgroups when the
    batch does not fill the GPU, 128-row ones otherwise): random trees, heads, ragged lengths
    with empty caches and one-key tails, all rows against the oracle."""
    rng = np.random.default_rng(1000 + seed)
    for case in range(4):
        B = int(rng.integers(1, 7))
        H = int(rng.choice([1, 3, 8, 16, 64]))
        N = int(rng.integers(1, max(2, min(256, 512 // H)) + 1))
        lo = int(rng.integers(0, 2))
        hi = int(rng.integers(lo, 2500))
        spec = workloads.Spec(f"rnd{seed}_{case}", 90 + seed, B, N, H, 512, 64, "bf16", None, ragged=(lo, hi),
                              tree="random", outlier_p=0.01 if case == 3 else 0.0)
        inp = workloads.make_inputs(spec, seed=case)
        check(f"random small request seed {seed} case {case}", inp)


@pytest.mark.parametrize("name", ["h128_t64", "rows1000_long", "ragged3"])
def test_strided_inputs_equal_contiguous(name):
    """Queries, cache and tree rows as views of 640-wide rows (latent, rope, then padding): the row
    strides of the descriptor differ from the widths, and every call equals the contiguous one bit
    for bit (64- and 128-row tiles, one and three requests; staged and one-launch calls)."""
    spec, lens = SMALL[name]
    inp = workloads.make_inputs(spec, seed=0, cache_lens=None if lens is None else np.array(lens, np.int32))
    dc, dr = spec.d_latent, spec.d_rope
    W = 640
    dev = to_device(inp)
    q = torch.zeros(dev.q_lat.shape[:-1] + (W,), dtype=dev.q_lat.dtype, device="cuda")
    q[..., :dc] = dev.q_lat
    q[..., dc:dc + dr] = dev.q_rope
    kv = torch.zeros((dev.kv.shape[0], W), dtype=dev.kv.dtype, device="cuda")
    kv[:, :dc + dr] = dev.kv
    tkv = torch.zeros(dev.tree_kv.shape[:-1] + (W,), dtype=dev.tree_kv.dtype, device="cuda")
    tkv[..., :dc + dr] = dev.tree_kv
    maxL = int(inp.cache_lens.max())
    masks = kdt.build_visibility(dev.parents)
    base = kdt.tree_verify_attn(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, masks,
                                dev.cache_lens, inp.scale, max_cache_len=maxL, total_cache_len=inp.total_len)
    views = (q[..., :dc], q[..., dc:dc + dr], kv[:, :dc], kv[:, dc:dc + dr], tkv[..., :dc], tkv[..., dc:dc + dr])
    got = kdt.tree_verify_attn(*views, masks, dev.cache_lens, inp.scale, max_cache_len=maxL,
                               total_cache_len=inp.total_len)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), base.view(torch.int32)), f"{name}: strided staged call differs"
    if spec.batch == 1:
        desc = kdt.make_desc(*views, maxL, inp.total_len)
        assert desc.q_lat_stride == W and desc.ckv_stride == W and desc.tree_ckv_stride == W
        ws = kdt.alloc_workspace(desc)
        one = torch.empty(dev.q_lat.shape, dtype=torch.float32, device="cuda")
        kdt.prepare_attend(dev.parents, dev.cache_lens, *views, inp.scale, one, desc, ws)
        kdt.combine(one, desc, ws)
        torch.cuda.synchronize()
        assert torch.equal(one.view(torch.int32), base.view(torch.int32)), f"{name}: strided one-launch call differs"
    print(f"PASS strided inputs [{name}] bit-identical to contiguous", flush=True)

