"""GPU edge cases of the attention kernels, through the C ABI, against closed forms and the fp64
oracle.  Each property is run on every attention kernel the library builds:

  k128   bf16, d = 512 + 64, 1024 rows over 9000 keys: the 128-row kernel, keys split
  k64    bf16, d = 512 + 64, 128 rows per request: the 64-row kernel, keys split
  k64w   bf16, d = 512 + 64, 1024 rows over 1500 keys: the 64-row kernel, 16 row tiles
  bf16s  bf16, d = 64 + 16: the 128-row kernel at small dims
  f32    fp32, d = 64 + 16: the fp32 instantiation (fp32 split partials)

The properties are those a tree node's output must have as ordinary attention over its committed
cache and its root-to-node path ("The Capstone Validation", section "Context and Motivation":
every drafted continuation is verified in one pass as if decoded alone):
  * scale 0: every visible key weighs the same, so the output is the mean of the visible latent
    rows (closed form); a negative scale is an ordinary scale of the other sign (oracle);
  * one key whose score exceeds every other visible score by more than 100: the output is that
    key's latent row (closed form);
  * adding the same amount to every score of a row (a constant rope coordinate on every key and
    a large query coordinate against it) changes nothing, although the shifted scores overflow
    fp32 exponentials; a steep score ramp makes the kernels move their softmax reference, and
    rescale their accumulators, several times per key split;
  * permuting the heads of a node permutes its outputs, bit for bit; relabelling the nodes in
    another parents-first order permutes the outputs (within the tolerance: the tree keys are then
    summed in another order).
Also: batches past the plan's LDS capacity (more than 1024 requests, more than 2048 groups), fp32
requests with outputs of magnitude 1-4 over long caches (split partials in fp32), and causal
prefill of chains of 256 nodes and of longer sequences in 256-node chunks.
The bf16 512 + 64 cases, all one-request batches, also run through the one-launch call
(kdt_tree_verify_prepare_attend), whose outputs must equal the staged calls' bit for bit.
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

KERNELS = {
    # over 8192 keys: 128-row tiles (shorter caches take 64-row ones up to 8192 rows)
    "k128": workloads.Spec("e128", 70, 1, 16, 64, 512, 64, "bf16", 9000, tree="random"),
    "k64": workloads.Spec("e64", 71, 1, 2, 64, 512, 64, "bf16", 1300, tree="chain"),
    "k64w": workloads.Spec("e64w", 75, 1, 16, 64, 512, 64, "bf16", 1500, tree="random"),
    # a two-tile tree: its 128 keys have places in the split range (14 splits of 384 keys)
    "k64p": workloads.Spec("e64p", 77, 1, 128, 8, 512, 64, "bf16", 5000, tree="random"),
    "bf16s": workloads.Spec("es", 72, 2, 9, 8, 64, 16, "bf16", 700, tree="random"),
    "f32": workloads.Spec("ef", 73, 2, 8, 4, 64, 16, "f32", 700, tree="random"),
}


def test_k128_takes_128_row_tiles():
    """k128 must run the 128-row kernel: for 1024 rows over 9000 keys 128-row tiles make 29 splits
    of 320 keys (64-row tiles would make 16)."""
    inp = workloads.make_inputs(KERNELS["k128"], seed=0)
    dev = to_device(inp)
    desc = kdt.make_desc(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, 9000, inp.total_len)
    assert kdt.num_splits(desc) == 29


def test_two_tile_tree_has_places_in_the_split_range():
    """k64p's 128-node tree takes 128 places in the range the splits cut: 5128 virtual keys in 14
    splits of 384 (split 0: the tree tiles and committed keys 0..255).  Without places the 5000
    committed keys would make 16 splits of 320."""
    inp = workloads.make_inputs(KERNELS["k64p"], seed=0)
    dev = to_device(inp)
    desc = kdt.make_desc(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, 5000, inp.total_len)
    assert kdt.num_splits(desc) == 14


@pytest.mark.parametrize("L", [255, 256, 257, 4480, 4999])
def test_two_tile_tree_split_boundaries_vs_oracle(L):
    """Cache lengths at the edges of split 0's committed keys (256) and of the last split, under the
    geometry made for 5000 keys: every row against the oracle, and the one-launch call equal to the
    staged calls."""
    inp = workloads.make_inputs(KERNELS["k64p"], seed=9, cache_lens=np.array([L], dtype=np.int32))
    _gpu_vs_oracle(f"k64p L={L} vs oracle", inp, max_len=5000)


def _plain_f32(inp, masks):
    """The attention definition in plain fp32 PyTorch on the CPU: one request and node at a time,
    softmax over the cache rows and the visible tree rows."""
    B, N = inp.parents.shape
    dc = inp.spec.d_latent
    out = np.zeros((B, N, inp.spec.heads, dc))
    offs = np.concatenate([[0], np.cumsum(inp.cache_lens.numpy())])
    for b in range(B):
        cache = torch.cat([inp.ckv[offs[b]:offs[b + 1]].float(), inp.krope[offs[b]:offs[b + 1]].float()], 1)
        for i in range(N):
            vis = [j for j in range(N) if (int(masks[b, i, j // 64]) >> (j % 64)) & 1]
            k = torch.cat([cache, torch.cat([inp.tree_ckv[b, vis].float(), inp.tree_krope[b, vis].float()], 1)])
            q = torch.cat([inp.q_lat[b, i].float(), inp.q_rope[b, i].float()], 1)
            out[b, i] = (torch.softmax((q @ k.T) * inp.scale, dim=1) @ k[:, :dc]).numpy()
    return out


@pytest.mark.parametrize("case", [(1, 31, 4, 100), (3, 64, 16, 875)])
def test_f32_with_outliers_is_as_accurate_as_f32(case):
    """fp32 inputs with x20 outliers (outputs up to about 80, scores spread over hundreds): fp32
    arithmetic cannot hold the 1e-5 bound of unit-scale inputs here (a 1-ulp score error alone
    moves a weight by about 5e-6 relative), so the kernel is held to 4x the error of the plain fp32
    definition against the fp64 oracle, and never to less than 1e-5."""
    B, N, H, L = case
    spec = workloads.Spec(f"f32o{N}", 78, B, N, H, 64, 16, "f32", None if B > 1 else L,
                          ragged=(0, L) if B > 1 else None, outlier_p=0.01, depth=8, topk=8)
    inp = workloads.make_inputs(spec, seed=1)
    masks, out, status = run_gpu(inp)
    assert status == 0
    ref = oracle.run(inp)[1]
    got = out.cpu().double().numpy()
    err = float(np.abs(got - ref).max())
    f32_err = float(np.abs(_plain_f32(inp, masks) - ref).max())
    bound = max(TOL["f32"], 4 * f32_err)
    report(f"f32 outliers {case} (plain fp32: {f32_err:.2e})", err, bound)
    assert np.isfinite(got).all() and err <= bound


def _cast(x: np.ndarray, like: torch.Tensor) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(like.dtype)


def _paths(parents: np.ndarray):
    """Root-to-node path (as a set of node ids) of every node, by walking parent links."""
    B, N = parents.shape
    out = []
    for b in range(B):
        rows = []
        for i in range(N):
            p, j = set(), i
            while j != -1:
                p.add(j)
                j = int(parents[b, j])
            rows.append(sorted(p))
        out.append(rows)
    return out


def _gpu_vs_oracle(name, inp, tol=None, max_len=None):
    """Every row of the GPU output against the oracle; returns (gpu out, oracle out) as fp64.
    A one-request bf16 512 + 64 batch also runs through the one-launch call, which must give the
    staged calls' bits.  max_len: the cache-length bound of the geometry (default: the longest
    request)."""
    _, out, status = run_gpu(inp, max_len=max_len)
    assert status == 0
    got = out.cpu().double().numpy()
    ref = oracle.run(inp)[1]
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max())
    tol = TOL[inp.spec.dtype] if tol is None else tol
    report(name, err, tol)
    assert err <= tol
    sp = inp.spec
    if sp.batch == 1 and sp.dtype == "bf16" and sp.d_latent == 512:
        dev = to_device(inp)
        _, staged, _ = run_gpu(inp, dev, staged="prepare", max_len=max_len)
        _, one, st1 = run_gpu(inp, dev, staged="one", max_len=max_len)
        assert st1 == 0
        assert torch.equal(one.view(torch.int32), staged.view(torch.int32)), f"{name}: one launch differs"
        print(f"PASS {name}: one launch bit-identical to the staged calls", flush=True)
    return got, ref


@pytest.mark.parametrize("kern", list(KERNELS))
def test_scale_zero_is_mean_of_visible_latents(kern):
    spec = KERNELS[kern]
    inp = dataclasses.replace(workloads.make_inputs(spec, seed=0), scale=0.0)
    got, _ = _gpu_vs_oracle(f"scale 0 vs oracle [{kern}]", inp)
    # closed form: the arithmetic mean of the visible latent rows
    lens = inp.cache_lens.numpy().astype(np.int64)
    offs = np.concatenate([[0], np.cumsum(lens)])
    ckv = inp.ckv.double().numpy()
    tckv = inp.tree_ckv.double().numpy()
    paths = _paths(inp.parents.numpy())
    err = 0.0
    for b in range(spec.batch):
        csum, n0 = ckv[offs[b]:offs[b + 1]].sum(0), lens[b]
        for i in range(spec.nodes):
            mean = (csum + tckv[b, paths[b][i]].sum(0)) / (n0 + len(paths[b][i]))
            err = max(err, float(np.abs(got[b, i] - mean[None, :]).max()))
    report(f"scale 0 vs mean of visible latents [{kern}]", err, TOL[spec.dtype])
    assert err <= TOL[spec.dtype]


@pytest.mark.parametrize("kern", list(KERNELS))
def test_negative_scale(kern):
    inp = workloads.make_inputs(KERNELS[kern], seed=1)
    inp = dataclasses.replace(inp, scale=-inp.scale * 1.5)
    _gpu_vs_oracle(f"negative scale [{kern}]", inp)


def _dominant(inp, where: str, margin: float = 130.0):
    """Inputs where one key of every request (a cache key, or tree node 0 of a chain) scores about
    `margin` above every other key: rope coordinate 0 is 1 on that key and 0 elsewhere, and every
    query's rope coordinate 0 is margin / scale."""
    sp = inp.spec
    kv, tkv, qr = inp.kv_cache.clone(), inp.tree_kv.clone(), inp.q_rope.clone()
    dc = sp.d_latent
    kv[:, dc] = 0
    tkv[:, :, dc] = 0
    lens = inp.cache_lens.numpy().astype(np.int64)
    offs = np.concatenate([[0], np.cumsum(lens)])
    dom = []
    for b in range(sp.batch):
        if where == "tree":
            tkv[b, 0, dc] = 1
            dom.append(tkv[b, 0, :dc].double().numpy())
        else:
            L = int(lens[b])
            t = {"first": 0, "middle": L // 2 + 7, "last": L - 1}[where]
            kv[offs[b] + t, dc] = 1
            dom.append(kv[offs[b] + t, :dc].double().numpy())
    qr[..., 0] = margin / inp.scale
    return dataclasses.replace(inp, kv_cache=kv, tree_kv=tkv, q_rope=qr), dom


@pytest.mark.parametrize("kern", list(KERNELS))
@pytest.mark.parametrize("where", ["first", "middle", "last", "tree"])
def test_one_dominant_key(kern, where):
    spec = KERNELS[kern]
    if where == "tree":
        spec = dataclasses.replace(spec, tree="chain")      # node 0 is on every node's path
    inp, dom = _dominant(workloads.make_inputs(spec, seed=2), where)
    got, _ = _gpu_vs_oracle(f"dominant {where} key vs oracle [{kern}]", inp)
    err = max(float(np.abs(got[b] - dom[b]).max()) for b in range(spec.batch))
    report(f"dominant {where} key vs its latent row [{kern}]", err, TOL[spec.dtype])
    assert err <= TOL[spec.dtype]


@pytest.mark.parametrize("kern", list(KERNELS))
def test_common_shift_of_100_changes_nothing(kern):
    """krope[.][0] = 1 on every key; adding 100/scale to every query's rope coordinate 0 adds 100
    to every score of the row (e^100 overflows fp32).  The GPU output on the shifted inputs must
    match the oracle on the unshifted ones."""
    inp = workloads.make_inputs(KERNELS[kern], seed=3)
    dc = inp.spec.d_latent
    kv, tkv = inp.kv_cache.clone(), inp.tree_kv.clone()
    kv[:, dc] = 1
    tkv[:, :, dc] = 1
    base = dataclasses.replace(inp, kv_cache=kv, tree_kv=tkv)
    qr = base.q_rope.clone()
    qr[..., 0] = qr[..., 0].float() + 100.0 / inp.scale
    shifted = dataclasses.replace(base, q_rope=qr)
    _, out, status = run_gpu(shifted)
    assert status == 0
    ref = oracle.run(base)[1]
    err = float(np.abs(out.cpu().double().numpy() - ref).max())
    report(f"+100 common shift vs unshifted oracle [{kern}]", err, TOL[inp.spec.dtype])
    assert err <= TOL[inp.spec.dtype]


@pytest.mark.parametrize("kern", list(KERNELS))
def test_score_ramp_moves_the_reference(kern):
    """Rope coordinate 1 of cache key t is a sawtooth ramp * ((t mod 256) - 128) (the top of a
    tooth on the tree keys), every query's is 1: within each 256-key split the scores climb by
    ~50 (base 2) per 64-key tile, so the softmax reference -- which moves, for the whole wave,
    once a block max passes it by 2^32, to the running max + 2^32 -- moves twice per split after
    its first setting, and the accumulators are rescaled each time.  The teeth keep the scores
    within about +-100 (base 2), and the latent rows are scaled by 1/4, so that fp32 rounding of
    the scores stays below the fp32 tolerance."""
    inp = workloads.make_inputs(KERNELS[kern], seed=4)
    sp = inp.spec
    dc = sp.d_latent
    ramp = 50.0 / (64 * inp.scale * np.log2(np.e))
    kv, tkv, qr = inp.kv_cache.clone(), inp.tree_kv.clone(), inp.q_rope.clone()
    kv[:, :dc] = (kv[:, :dc].float() * 0.25).to(kv.dtype)
    tkv[:, :, :dc] = (tkv[:, :, :dc].float() * 0.25).to(tkv.dtype)
    lens = inp.cache_lens.numpy().astype(np.int64)
    offs = np.concatenate([[0], np.cumsum(lens)])
    for b in range(sp.batch):
        t = np.arange(lens[b], dtype=np.float32)
        kv[offs[b]:offs[b + 1], dc + 1] = _cast(ramp * (t % 256 - 128), kv)
        tkv[b, :, dc + 1] = float(ramp * 127)
    qr[..., 1] = 1.0
    _gpu_vs_oracle(f"score ramp, reference moves [{kern}]",
                   dataclasses.replace(inp, kv_cache=kv, tree_kv=tkv, q_rope=qr))


@pytest.mark.parametrize("kern", list(KERNELS))
def test_head_permutation_is_exact(kern):
    inp = workloads.make_inputs(KERNELS[kern], seed=5)
    H = inp.spec.heads
    perm = torch.from_numpy(np.random.default_rng(5).permutation(H))
    _, base, _ = run_gpu(inp)
    permuted = dataclasses.replace(inp, q_lat=inp.q_lat[:, :, perm].contiguous(),
                                   q_rope=inp.q_rope[:, :, perm].contiguous())
    _, out, _ = run_gpu(permuted)
    assert torch.equal(out, base[:, :, perm.cuda()])
    print(f"PASS head permutation bit-identical [{kern}]", flush=True)


@pytest.mark.parametrize("kern", ["k128", "k64", "k64w", "f32"])
def test_node_relabel_permutes_outputs(kern):
    """Another parents-first numbering of the same tree (children of a node in reverse order,
    found by a depth-first walk) permutes the outputs."""
    inp = workloads.make_inputs(dataclasses.replace(KERNELS[kern], tree="random"), seed=6)
    par = inp.parents.numpy()
    B, N = par.shape
    new_of = np.zeros((B, N), np.int64)
    new_par = np.zeros((B, N), np.int32)
    for b in range(B):
        kids = {}
        for j in range(N):
            kids.setdefault(int(par[b, j]), []).append(j)
        order, stack = [], list(kids.get(-1, []))
        while stack:
            j = stack.pop()
            order.append(j)
            stack.extend(kids.get(j, []))
        new_of[b, order] = np.arange(N)
        for old in range(N):
            p = int(par[b, old])
            new_par[b, new_of[b, old]] = -1 if p < 0 else new_of[b, p]
        assert (new_par[b] < np.arange(N)).all()
    old_of = np.argsort(new_of, axis=1)
    idx = torch.from_numpy(old_of)
    take = lambda t: torch.stack([t[b, idx[b]] for b in range(B)]).contiguous()   # noqa: E731
    relab = dataclasses.replace(inp, parents=torch.from_numpy(new_par), q_lat=take(inp.q_lat),
                                q_rope=take(inp.q_rope), tree_kv=take(inp.tree_kv))
    _, base, _ = run_gpu(inp)
    _, out, _ = run_gpu(relab)
    back = torch.stack([out[b, torch.from_numpy(new_of[b]).cuda()] for b in range(B)])
    err = float((back - base).abs().max())
    report(f"node relabel permutes outputs [{kern}]", err, TOL[inp.spec.dtype])
    assert err <= TOL[inp.spec.dtype]


# ------------------------------------------------------------------ plan capacity
@pytest.mark.parametrize("batch,nodes,heads", [(1100, 1, 8), (2100, 1, 8), (1100, 2, 64)])
def test_batches_past_plan_lds(batch, nodes, heads):
    """More than 1024 requests (lengths and offsets no longer fit the plan's LDS) and more than
    2048 groups (the work order is request order): every row against the oracle."""
    spec = workloads.Spec(f"big{batch}", 74, batch, nodes, heads, 512, 64, "bf16", None, ragged=(0, 60),
                          tree="chain")
    inp = workloads.make_inputs(spec, seed=0)
    _gpu_vs_oracle(f"{batch} requests x {nodes * heads} rows (plan past its LDS)", inp)


# ------------------------------------------------------------------ fp32 with large outputs
@pytest.mark.parametrize("L", [1024, 5000])
def test_f32_split_large_outputs(L):
    """fp32 inputs, one request over a long cache (keys split over workgroups, partials in fp32),
    latent rows scaled x2 so that outputs reach magnitudes 1-4: every row within 1e-5."""
    spec = workloads.Spec(f"f32big{L}", 75, 1, 8, 4, 64, 16, "f32", L, tree="random")
    inp = workloads.make_inputs(spec, seed=0)
    dc = spec.d_latent
    kv, tkv = inp.kv_cache.clone(), inp.tree_kv.clone()
    kv[:, :dc] *= 2
    tkv[:, :, :dc] *= 2
    inp = dataclasses.replace(inp, kv_cache=kv, tree_kv=tkv)
    dev = to_device(inp)
    desc = kdt.make_desc(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, L)
    assert kdt.num_splits(desc) > 1
    _, ref = _gpu_vs_oracle(f"fp32 L={L}, outputs up to |x| ~ 4", inp)
    assert np.abs(ref).max() >= 1.0


# ------------------------------------------------------------------ prefill-shaped chains
@pytest.mark.parametrize("name", ["prefill4k", "prefill"])
def test_prefill_chain_all_rows(name):
    """A 256-node chain (a causal chunk of 256 tokens) over 4096 and 32768 committed tokens: every
    row against the oracle."""
    _gpu_vs_oracle(name, workloads.make_inputs(name, seed=0))


def _causal_reference(kv_all, q_all, scale, L0, H):
    """Causal attention of query rows [L0, L0 + n) over kv_all[: L0 + n] (torch SDPA, fp64, CPU)."""
    n = q_all.shape[0]
    k = kv_all[: L0 + n].double()
    q = q_all.double().permute(1, 0, 2)                                          # [H, n, D]
    mask = torch.arange(L0 + n)[None, :] <= (L0 + torch.arange(n))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        q[None], k[None, None].expand(1, H, -1, -1), k[None, None, :, :512].expand(1, H, -1, -1),
        attn_mask=mask, scale=scale)[0]
    return ref.permute(1, 0, 2)                                                  # [n, H, 512]


def test_prefill_chain_equals_causal_sdpa():
    """The 256-node chain over 4096 committed tokens is causal prefill of those 256 tokens."""
    inp = workloads.make_inputs("prefill4k", seed=0)
    _, out, _ = run_gpu(inp)
    H = inp.spec.heads
    kv_all = torch.cat([inp.kv_cache, inp.tree_kv[0]])
    q_all = torch.cat([inp.q_lat[0], inp.q_rope[0]], -1)
    ref = _causal_reference(kv_all, q_all, inp.scale, inp.spec.cache_len, H)
    err = float((out[0].cpu().double() - ref).abs().max())
    report("256-node chain == causal prefill (SDPA)", err, TOL["bf16"])
    assert err <= TOL["bf16"]


def test_long_prefill_in_256_node_chunks():
    """Causal prefill of 600 tokens after a 1000-token cache, as successive calls of at most 256
    chain nodes each (every chunk's tokens are committed to the cache before the next chunk), equals
    causal attention over the whole sequence."""
    H, L0, n = 16, 1000, 600
    spec = workloads.Spec("chunked", 76, 1, n, H, 512, 64, "bf16", L0, tree="chain")
    g = np.random.default_rng(76)
    kv_all = torch.from_numpy(g.standard_normal((L0 + n, 576), dtype=np.float32)).to(torch.bfloat16)
    q_all = torch.from_numpy(g.standard_normal((n, H, 576), dtype=np.float32)).to(torch.bfloat16)
    outs, done = [], 0
    while done < n:
        c = min(256, n - done)
        L = L0 + done
        chunk = workloads.Inputs(
            spec=dataclasses.replace(spec, nodes=c, cache_len=L),
            parents=torch.arange(-1, c - 1, dtype=torch.int32)[None],
            cache_lens=torch.tensor([L], dtype=torch.int32),
            q_lat=q_all[done:done + c, :, :512][None].contiguous(),
            q_rope=q_all[done:done + c, :, 512:][None].contiguous(),
            kv_cache=kv_all[:L].contiguous(), tree_kv=kv_all[L:L + c][None].contiguous(), scale=spec.scale)
        _, out, status = run_gpu(chunk)
        assert status == 0
        outs.append(out[0].cpu().double())
        done += c
    ref = _causal_reference(kv_all, q_all, spec.scale, L0, H)
    err = float((torch.cat(outs) - ref).abs().max())
    report("600-token prefill in 256-node chunks == causal attention", err, TOL["bf16"])
    assert err <= TOL["bf16"]
