"""Pins of the fp64 oracle against facts it does not compute itself (CPU only).

What pins what:
  visibility  -- hand-derived fixture (tests/golden/visibility_handworked.txt), closed forms
                 (chain -> lower-triangular, star -> identity), structural invariants on random
                 and best-first trees, exhaustive agreement with an explicit path walk over
                 every parent array with N <= 6.
  attention   -- hand-derived fixture (tests/golden/attention_handworked.json); a chain tree
                 equals causal prefill and a single node equals one decode step, both through
                 torch's scaled_dot_product_attention in fp64; a star equals independent
                 decodes; scale 0 gives the mean of the visible latents; a dominant key gives
                 its own latent; a common score shift changes nothing; permuting heads permutes
                 outputs; the MLA absorption identity against materialised per-head K/V; and
                 exhaustive agreement with the path-walk formulation (oracle/bruteforce.py).
  sensitivity -- planted mistakes (a dropped rope term, a missing self bit, a cache offset off
                 by one, a transposed operand) each fail at least one pin.

The rule behind all of them: a node of the draft tree is verified exactly as an ordinary
decode over the committed cache plus its own root-to-node path ("The Capstone Validation",
section "Context and Motivation"); prefill and decode are the two ordinary attention passes
of "Validating the Native Engine", section "What the Message Actually Says".
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import bruteforce
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- helpers
def read_visibility_fixture():
    cases, cur = [], None
    for line in open(os.path.join(GOLDEN, "visibility_handworked.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        tok = line.split()
        if tok[0] == "case":
            cur = {"name": tok[1], "masks": {}}
            cases.append(cur)
        elif tok[0] == "parents":
            cur["parents"] = [int(t) for t in tok[1:]]
        elif tok[0] == "bad":
            cur["bad"] = int(tok[1])
        elif tok[0] == "mask":
            cur["masks"][int(tok[1])] = [int(t, 16) for t in tok[2:]]
    return cases


def tiny_inputs(N, L, H=2, dc=8, dr=4, seed=0, parents=None, dtype="f32", B=1, lens=None):
    spec = workloads.Spec("pin", 90 + N, B, N, H, dc, dr, dtype, L, tree="random")
    par = None if parents is None else np.asarray(parents, np.int32).reshape(B, N)
    return workloads.make_inputs(spec, seed=seed, parents=par, cache_lens=lens)


def run_oracle(inp, **kw):
    masks, out, bad = oracle.run(inp, **kw)
    return out


def sdpa_rows(q_lat, q_rope, keys_lat, keys_rope, scale, mask=None):
    """Ordinary attention via torch (fp64): q [M, *], keys [K, *] -> [M, dc]."""
    q = torch.cat([torch.as_tensor(q_lat), torch.as_tensor(q_rope)], -1).double()[None, None]
    k = torch.cat([torch.as_tensor(keys_lat), torch.as_tensor(keys_rope)], -1).double()[None, None]
    v = torch.as_tensor(keys_lat).double()[None, None]
    m = None if mask is None else torch.as_tensor(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=float(scale))
    return o[0, 0].numpy()


# ----------------------------------------------------------------------------- visibility pins
@pytest.mark.parametrize("case", read_visibility_fixture(), ids=lambda c: c["name"])
def test_visibility_handworked(case):
    par = np.array([case["parents"]], np.int32)
    masks, bad = oracle.visibility(par)
    assert bad == case["bad"]
    W = masks.shape[2]
    for i, words in case["masks"].items():
        want = words + [0] * (W - len(words))
        assert [int(w) for w in masks[0, i]] == want, (i, [hex(int(w)) for w in masks[0, i]])


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 128, 200, 256])
def test_visibility_closed_forms(N):
    chain = np.arange(-1, N - 1, dtype=np.int32)[None]
    star = np.full((1, N), -1, np.int32)
    mc, bc = oracle.visibility(chain)
    ms, bs = oracle.visibility(star)
    assert bc == 0 and bs == 0
    for i in range(N):
        full = (1 << (i + 1)) - 1               # chain: bits 0..i
        one = 1 << i                            # star: bit i only
        for w in range(mc.shape[2]):
            assert int(mc[0, i, w]) == (full >> (64 * w)) & (2**64 - 1)
            assert int(ms[0, i, w]) == (one >> (64 * w)) & (2**64 - 1)


def _mask_int(row):
    return sum(int(w) << (64 * k) for k, w in enumerate(row))


@pytest.mark.parametrize("name,seed", [("kimi", 0), ("kimi", 1), ("wide", 0), ("tiny", 3),
                                       ("block8", 0), ("ragged", 0)])
def test_visibility_invariants(name, seed):
    spec = workloads.SPECS[name]
    par = workloads.make_parents(spec, seed)
    masks, bad = oracle.visibility(par)
    assert bad == 0
    B, N = par.shape
    for b in range(B):
        depth = {}
        for i in range(N):
            m = _mask_int(masks[b, i])
            p = int(par[b, i])
            assert (m >> i) & 1                                  # self bit
            assert m >> (i + 1) == 0                            # nothing at or after i+1
            assert m == ((_mask_int(masks[b, p]) if p >= 0 else 0) | (1 << i))
            depth[i] = 1 + (depth[p] if p >= 0 else 0)
            assert bin(m).count("1") == depth[i]
    # padding bits beyond N stay zero
    W = masks.shape[2]
    assert all(_mask_int(masks[b, i]) < (1 << N) for b in range(B) for i in range(N)) and W == (N + 63) // 64


def all_parent_arrays(N):
    return itertools.product(*[range(-1, i) for i in range(N)])


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 6])
def test_visibility_exhaustive(N):
    pars = np.array(list(all_parent_arrays(N)), np.int32)
    masks, bad = oracle.visibility(pars)
    assert bad == 0
    np.testing.assert_array_equal(masks, bruteforce.masks_from_paths(pars))


def test_visibility_invalid_rows_match_path_walk():
    rng = np.random.default_rng(7)
    pars = rng.integers(-3, 9, size=(64, 8)).astype(np.int32)
    masks, bad = oracle.visibility(pars)
    ref = bruteforce.masks_from_paths(pars)
    np.testing.assert_array_equal(masks, ref)
    invalid = sum(bruteforce.path_of(pars[b], i) is None for b in range(64) for i in range(8))
    assert bad == invalid and invalid > 0


# ----------------------------------------------------------------------------- attention pins
def test_attention_handworked():
    g = json.load(open(os.path.join(GOLDEN, "attention_handworked.json")))
    N = len(g["parents"])
    f = lambda x: torch.tensor(x, dtype=torch.float32)
    q_lat = f(g["q_lat"]).reshape(1, N, 1, -1)
    q_rope = f(g["q_rope"]).reshape(1, N, 1, -1)
    masks, bad = oracle.visibility(np.array([g["parents"]], np.int32))
    out = oracle.attention(q_lat, q_rope, f(g["cache_ckv"]), f(g["cache_krope"]),
                           f(g["tree_ckv"])[None], f(g["tree_krope"])[None], masks,
                           np.array([len(g["cache_ckv"])], np.int32), g["scale"])
    np.testing.assert_allclose(out[0, :, 0], np.array(g["expected"]), atol=g["tolerance"], rtol=0)


@pytest.mark.parametrize("L,N", [(0, 5), (7, 1), (33, 16), (130, 9)])
def test_chain_equals_causal_prefill(L, N):
    inp = tiny_inputs(N, L, parents=np.arange(-1, N - 1))
    out = run_oracle(inp)
    keys_lat = torch.cat([inp.ckv, inp.tree_ckv[0]]).double()
    keys_rope = torch.cat([inp.krope, inp.tree_krope[0]]).double()
    # node i sees keys 0 .. L+i: the causal mask of a prefill over cache ++ chain
    causal = torch.arange(L + N)[None, :] <= (L + torch.arange(N))[:, None]
    for h in range(inp.spec.heads):
        ref = sdpa_rows(inp.q_lat[0, :, h], inp.q_rope[0, :, h], keys_lat, keys_rope, inp.scale, causal)
        np.testing.assert_allclose(out[0, :, h], ref, atol=1e-12, rtol=0)


def test_chain_config_rows_equal_causal_prefill():
    """The long-context chain workload (16 nodes over 32768 cache rows), a sample of rows."""
    inp = workloads.make_inputs("chain", seed=0)
    spec, L = inp.spec, int(inp.cache_lens[0])
    rows = [(i * spec.heads + h) for i, h in [(0, 0), (5, 17), (15, 63)]]
    out = run_oracle(inp, rows=rows)
    keys_lat = torch.cat([inp.ckv, inp.tree_ckv[0]]).double()
    keys_rope = torch.cat([inp.krope, inp.tree_krope[0]]).double()
    for k, r in enumerate(rows):
        i, h = divmod(r, spec.heads)
        ref = sdpa_rows(inp.q_lat[0, i, h][None], inp.q_rope[0, i, h][None],
                        keys_lat[: L + i + 1], keys_rope[: L + i + 1], inp.scale)
        np.testing.assert_allclose(out[k], ref[0], atol=1e-11, rtol=0)


@pytest.mark.parametrize("L", [0, 1, 64, 257])
def test_single_node_equals_decode(L):
    inp = tiny_inputs(1, L, parents=[-1])
    out = run_oracle(inp)
    keys_lat = torch.cat([inp.ckv, inp.tree_ckv[0]]).double()
    keys_rope = torch.cat([inp.krope, inp.tree_krope[0]]).double()
    ref = sdpa_rows(inp.q_lat[0, 0], inp.q_rope[0, 0], keys_lat, keys_rope, inp.scale)
    np.testing.assert_allclose(out[0, 0], ref, atol=1e-12, rtol=0)


def test_star_equals_independent_decodes():
    N, L = 6, 20
    inp = tiny_inputs(N, L, parents=[-1] * N)
    out = run_oracle(inp)
    for i in range(N):
        keys_lat = torch.cat([inp.ckv, inp.tree_ckv[0, i:i + 1]]).double()
        keys_rope = torch.cat([inp.krope, inp.tree_krope[0, i:i + 1]]).double()
        ref = sdpa_rows(inp.q_lat[0, i], inp.q_rope[0, i], keys_lat, keys_rope, inp.scale)
        np.testing.assert_allclose(out[0, i], ref, atol=1e-12, rtol=0)


def test_scale_zero_is_mean_of_visible_latents():
    par = [-1, 0, 0, 1, -1, 4, 3]
    inp = tiny_inputs(7, 11, parents=par)
    inp.scale = 0.0
    out = run_oracle(inp)
    lat = inp.ckv.double().numpy()
    tl = inp.tree_ckv[0].double().numpy()
    for i in range(7):
        anc, j = [], i
        while j != -1:
            anc.append(j)
            j = par[j]
        want = np.concatenate([lat, tl[anc]]).mean(axis=0)
        for h in range(inp.spec.heads):
            np.testing.assert_allclose(out[0, i, h], want, atol=1e-13, rtol=0)


def test_dominant_key_gives_its_latent():
    N, L = 4, 9
    inp = tiny_inputs(N, L, parents=[-1, 0, 1, 1])
    # make the rope part of tree node 1 line up with every query's rope part at a huge score
    big = 1e3
    inp.tree_kv[0, 1, inp.spec.d_latent:] = 0
    inp.tree_kv[0, 1, inp.spec.d_latent] = 1.0
    inp.q_rope[..., 0] = big / inp.scale
    out = run_oracle(inp)
    for i in (1, 2, 3):       # node 1 is on the path of nodes 1, 2, 3
        for h in range(inp.spec.heads):
            np.testing.assert_allclose(out[0, i, h], inp.tree_ckv[0, 1].double().numpy(), atol=1e-12)


def test_common_shift_changes_nothing():
    inp = tiny_inputs(5, 13, parents=[-1, 0, 1, 0, 3])
    base = run_oracle(inp)
    dc = inp.spec.d_latent
    inp.kv_cache[:, dc] = 1.0
    inp.tree_kv[:, :, dc] = 1.0
    ref = run_oracle(inp)          # same keys, rope coordinate 0 now 1 everywhere
    inp2 = tiny_inputs(5, 13, parents=[-1, 0, 1, 0, 3])
    inp2.kv_cache[:, dc] = 1.0
    inp2.tree_kv[:, :, dc] = 1.0
    inp2.q_rope[..., 0] += 100.0 / inp2.scale    # every score of a row shifts by +100
    shifted = run_oracle(inp2)
    np.testing.assert_allclose(shifted, ref, atol=1e-9, rtol=0)
    assert np.abs(base - ref).max() > 1e-3        # the edit itself did change the outputs


def test_head_permutation_equivariance():
    inp = tiny_inputs(5, 10, H=4, parents=[-1, 0, 0, 2, -1])
    out = run_oracle(inp)
    perm = [2, 0, 3, 1]
    inp.q_lat = inp.q_lat[:, :, perm].contiguous()
    inp.q_rope = inp.q_rope[:, :, perm].contiguous()
    outp = run_oracle(inp)
    np.testing.assert_array_equal(outp, out[:, :, perm])


def test_mla_absorption_identity():
    """Absorbed attention equals ordinary multi-head attention with per-head K/V up-projections."""
    rng = np.random.default_rng(11)
    H, dc, dr, dn, dv, N, L = 3, 8, 4, 5, 6, 4, 10
    par = [-1, 0, 1, 0]
    c_cache, r_cache = rng.standard_normal((L, dc)), rng.standard_normal((L, dr))
    c_tree, r_tree = rng.standard_normal((N, dc)), rng.standard_normal((N, dr))
    W_uk = rng.standard_normal((H, dn, dc))     # k_nope = W_uk c
    W_uv = rng.standard_normal((H, dv, dc))     # v = W_uv c
    q_nope = rng.standard_normal((N, H, dn))
    q_pe = rng.standard_normal((N, H, dr))
    scale = float(np.float32(1 / np.sqrt(dn + dr)))
    q_lat = np.einsum("nhd,hdc->nhc", q_nope, W_uk)            # absorbed query
    masks, _ = oracle.visibility(np.array([par], np.int32))
    absorbed = oracle.attention(q_lat[None], q_pe[None], c_cache, r_cache, c_tree[None], r_tree[None],
                                masks, np.array([L], np.int32), scale)[0]
    for i in range(N):
        path, j = [], i
        while j != -1:
            path.append(j)
            j = par[j]
        C = np.concatenate([c_cache, c_tree[path]])
        R = np.concatenate([r_cache, r_tree[path]])
        for h in range(H):
            k = np.concatenate([C @ W_uk[h].T, R], axis=1)
            v = C @ W_uv[h].T
            q = np.concatenate([q_nope[i, h], q_pe[i, h]])[None]
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.tensor(q)[None], torch.tensor(k)[None], torch.tensor(v)[None], scale=scale)[0, 0]
            np.testing.assert_allclose(W_uv[h] @ absorbed[i, h], ref.numpy(), atol=1e-10, rtol=0)


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5])
def test_exhaustive_trees_match_path_walk(N):
    L = 6
    for k, par in enumerate(all_parent_arrays(N)):
        inp = tiny_inputs(N, L, H=2, dc=4, dr=2, seed=k, parents=par)
        out = run_oracle(inp)
        ref = bruteforce.attention(inp.q_lat, inp.q_rope, inp.ckv, inp.krope, inp.tree_ckv,
                                   inp.tree_krope, inp.parents.numpy(), inp.cache_lens.numpy(), inp.scale)
        np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)


def test_ragged_batch_matches_path_walk_and_row_subsets():
    spec = workloads.Spec("pinr", 98, 4, 6, 2, 8, 4, "bf16", None, ragged=(0, 40), tree="random")
    inp = workloads.make_inputs(spec, seed=3)
    masks, out, bad = oracle.run(inp)
    ref = bruteforce.attention(inp.q_lat, inp.q_rope, inp.ckv, inp.krope, inp.tree_ckv,
                               inp.tree_krope, inp.parents.numpy(), inp.cache_lens.numpy(), inp.scale)
    np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)
    rows = [0, 7, 13, 47, 5]
    sub = oracle.run(inp, rows=rows)[1]
    np.testing.assert_array_equal(sub, out.reshape(-1, spec.d_latent)[rows])


# ----------------------------------------------------------------------------- sensitivity
def _pins_pass(attn_fn):
    """Run a handful of the pins above against an attention implementation."""
    ok = True
    g = json.load(open(os.path.join(GOLDEN, "attention_handworked.json")))
    f = lambda x: torch.tensor(x, dtype=torch.float32)
    N = len(g["parents"])
    par = np.array([g["parents"]], np.int32)
    out = attn_fn(f(g["q_lat"]).reshape(1, N, 1, -1), f(g["q_rope"]).reshape(1, N, 1, -1),
                  f(g["cache_ckv"]), f(g["cache_krope"]), f(g["tree_ckv"])[None],
                  f(g["tree_krope"])[None], par, np.array([2], np.int32), g["scale"])
    ok &= np.allclose(out[0, :, 0], g["expected"], atol=1e-6, rtol=0)
    N, L = 5, 9
    inp = tiny_inputs(N, L, parents=np.arange(-1, N - 1))
    out = attn_fn(inp.q_lat, inp.q_rope, inp.ckv, inp.krope, inp.tree_ckv, inp.tree_krope,
                  inp.parents.numpy(), inp.cache_lens.numpy(), inp.scale)
    keys_lat = torch.cat([inp.ckv, inp.tree_ckv[0]]).double()
    keys_rope = torch.cat([inp.krope, inp.tree_krope[0]]).double()
    causal = torch.arange(L + N)[None, :] <= (L + torch.arange(N))[:, None]
    for h in range(inp.spec.heads):
        ref = sdpa_rows(inp.q_lat[0, :, h], inp.q_rope[0, :, h], keys_lat, keys_rope, inp.scale, causal)
        ok &= np.allclose(out[0, :, h], ref, atol=1e-10, rtol=0)
    return bool(ok)


def _oracle_fn(q_lat, q_rope, ckv, krope, tckv, tkrope, parents, lens, scale):
    masks, _ = oracle.visibility(parents)
    return oracle.attention(q_lat, q_rope, ckv, krope, tckv, tkrope, masks, lens, scale)


def test_pins_accept_the_oracle():
    assert _pins_pass(_oracle_fn)


@pytest.mark.parametrize("mutant", ["drop_rope", "no_self_bit", "cache_off_by_one", "transposed_q", "drop_ancestors"])
def test_pins_reject_planted_mistakes(mutant):
    def fn(q_lat, q_rope, ckv, krope, tckv, tkrope, parents, lens, scale):
        masks, _ = oracle.visibility(parents)
        q_lat, q_rope = torch.as_tensor(q_lat), torch.as_tensor(q_rope)
        ckv, krope = torch.as_tensor(ckv), torch.as_tensor(krope)
        if mutant == "drop_rope":
            q_rope = torch.zeros_like(q_rope)
        elif mutant == "no_self_bit":
            N = masks.shape[1]
            for i in range(N):
                masks[:, i, i // 64] &= ~np.uint64(1 << (i % 64))
        elif mutant == "cache_off_by_one":
            ckv, krope = ckv[1:], krope[1:]
            lens = np.maximum(np.asarray(lens) - 1, 0).astype(np.int32)
        elif mutant == "transposed_q":
            q_lat = q_lat.flip(-1).contiguous()
        elif mutant == "drop_ancestors":
            N = masks.shape[1]
            for i in range(N):
                masks[:, i, :] = 0
                masks[:, i, i // 64] = np.uint64(1 << (i % 64))
        return oracle.attention(q_lat, q_rope, ckv, krope, tckv, tkrope, masks, lens, scale)
    assert not _pins_pass(fn)
