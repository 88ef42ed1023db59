"""One plan serving many attention calls, and the staged calls captured in a graph.

The plan (kdt_tree_verify_plan / _prepare) is made once per verify step and reused for every
layer, since the cache lengths and the tree do not change between layers ("The Capstone
Validation", section "Context and Motivation": one batched pass of the target over the drafted
tree).  Every attend + combine after one plan must give the same bits, split (Kimi: 8 splits
and the combine kernel) or not (a batch that fills the GPU).  The same calls captured in a
graph and replayed, with eager work between replays, must equal the eager result each time."""
import numpy as np
import pytest
import torch

import oracle
import tree_verify_mla_02_amd as kdt
import workloads
from gpu_helpers import TOL, report, to_device

pytestmark = pytest.mark.gpu


def _desc(inp, dev):
    return kdt.make_desc(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope,
                         int(inp.cache_lens.max()), inp.total_len)


def _check_rows(name, inp, out):
    dc = inp.spec.d_latent
    got = out.reshape(-1, dc).cpu().double().numpy()
    ref = oracle.run(inp)[1].reshape(-1, dc)
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max())
    tol = TOL[inp.spec.dtype]
    report(name, err, tol)
    assert err <= tol


def _inputs(name):
    if name == "batch300":
        spec = workloads.Spec("b300r", 71, 300, 2, 64, 512, 64, "bf16", None, ragged=(1, 300), tree="random")
        return workloads.make_inputs(spec, seed=0)
    return workloads.make_inputs(name, seed=2)


@pytest.mark.parametrize("name", ["kimi", "decode", "batch300"])
def test_one_plan_many_attends(name):
    inp = _inputs(name)
    dev = to_device(inp)
    desc = _desc(inp, dev)
    print(f"case {name}: splits {kdt.num_splits(desc)}", flush=True)
    ws = kdt.alloc_workspace(desc)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    masks = kdt.prepare(dev.parents, dev.cache_lens, desc, ws, dev_status=status)
    outs = []
    for _ in range(3):
        out = torch.full(dev.q_lat.shape, float("nan"), dtype=torch.float32, device="cuda")
        kdt.attend(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, masks, inp.scale, out,
                   desc, ws)
        kdt.combine(out, desc, ws)
        torch.cuda.synchronize()
        outs.append(out.cpu())
    assert int(status.item()) == 0
    for k in (1, 2):
        assert torch.equal(outs[k], outs[0]), f"attend {k} differs from attend 0"
    _check_rows(f"{name}-plan-reuse", inp, outs[0].cuda())


@pytest.mark.parametrize("name", ["kimi", "decode"])
def test_staged_calls_in_graph(name):
    """prepare outside, attend + combine captured once and replayed three times."""
    inp = _inputs(name)
    dev = to_device(inp)
    desc = _desc(inp, dev)
    ws = kdt.alloc_workspace(desc)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    masks = kdt.prepare(dev.parents, dev.cache_lens, desc, ws, dev_status=status)
    eager = torch.empty(dev.q_lat.shape, dtype=torch.float32, device="cuda")
    kdt.attend(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, masks, inp.scale, eager,
               desc, ws)
    kdt.combine(eager, desc, ws)
    torch.cuda.synchronize()
    out = torch.zeros_like(eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            kdt.attend(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, masks, inp.scale,
                       out, desc, ws)
            kdt.combine(out, desc, ws)
    torch.cuda.synchronize()
    for k in range(3):
        out.fill_(float("nan"))
        scratch = torch.randn(1 << 20, device="cuda") * 2.0        # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        print(f"{name} replay {k}: scratch {float(scratch.sum()):.3f}", flush=True)
        assert torch.equal(out, eager), f"replay {k} differs from the eager calls"
    assert int(status.item()) == 0
    _check_rows(f"{name}-graph", inp, eager)
