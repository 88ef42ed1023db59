"""The allocation-free verify entry point (kdt_tree_verify_attn_noalloc, include/kdt_noalloc.h),
through the C ABI: on two calls in a row -- a 64-node tree over 4096 tokens (keys split eight
ways, 48 MiB of the static scratch array), then a smaller batch on the same array -- its outputs
equal those of kdt_tree_verify_attn with a caller workspace bit for bit, and match the fp64
oracle within the bf16 tolerance.  A batch whose workspace exceeds the array is rejected before
anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import tree_verify_mla_02_amd as kdt
import workloads
from gpu_helpers import TOL, report, to_device

pytestmark = pytest.mark.gpu


def _compare(name, inp):
    dev = to_device(inp)
    maxL, total = int(inp.cache_lens.max()), inp.total_len
    masks = kdt.build_visibility(dev.parents)
    ref = kdt.tree_verify_attn(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, masks,
                               dev.cache_lens, inp.scale, max_cache_len=maxL, total_cache_len=total)
    out = torch.full_like(ref, float("nan"))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    kdt.tree_verify_attn_noalloc(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, masks,
                                 dev.cache_lens, inp.scale, max_cache_len=maxL, total_cache_len=total, out=out,
                                 dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(out, ref), name
    err = float(np.abs(out.cpu().double().numpy() - oracle.run(inp)[1]).max())
    report(f"no-alloc entry point, {name}", err, TOL[inp.spec.dtype])
    assert err <= TOL[inp.spec.dtype]


def test_noalloc_equals_workspace_entry_point_on_two_calls():
    _compare("kimi (48 MiB of scratch)", workloads.make_inputs("kimi", seed=0))
    small = workloads.Spec("na_small", 80, 2, 8, 16, 512, 64, "bf16", None, ragged=(100, 3000), tree="random")
    _compare("2 small requests after it", workloads.make_inputs(small, seed=0))


def test_noalloc_rejects_a_batch_larger_than_its_scratch():
    inp = workloads.make_inputs(workloads.Spec("na_big", 81, 1, 254, 64, 512, 64, "bf16", 64, tree="chain"), seed=0)
    dev = to_device(inp)
    masks = kdt.build_visibility(dev.parents)
    out = torch.full(dev.q_lat.shape, 7.0, dtype=torch.float32, device="cuda")
    # the bounds describe a 1M-token cache: three splits of 254 x 64 rows of partials, 71.8 MiB
    desc = kdt.make_desc(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, 1 << 20, 1 << 20)
    assert kdt.workspace_size(desc) > (64 << 20)
    with pytest.raises(kdt.KdtError) as e:
        kdt.tree_verify_attn_noalloc(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, masks,
                                     dev.cache_lens, inp.scale, max_cache_len=1 << 20, out=out, desc=desc)
    assert e.value.code == kdt._lib.KDT_ERR_WORKSPACE
    assert "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    print("PASS no-alloc entry point rejects a batch larger than its scratch", flush=True)
