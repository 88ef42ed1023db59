"""Shared helpers of the GPU tests: move a workloads.Inputs batch to the device and run the
C-ABI path on it."""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import torch

import tree_verify_mla_02_amd as kdt
import workloads

TOL = {"bf16": 2e-3, "f32": 1e-5}     # max-abs bounds on the fp32 outputs


@dataclasses.dataclass
class DevInputs:
    parents: torch.Tensor
    cache_lens: torch.Tensor
    q_lat: torch.Tensor
    q_rope: torch.Tensor
    kv: torch.Tensor
    tree_kv: torch.Tensor
    dc: int

    @property
    def ckv(self):
        return self.kv[:, : self.dc]

    @property
    def krope(self):
        return self.kv[:, self.dc:]

    @property
    def tree_ckv(self):
        return self.tree_kv[:, :, : self.dc]

    @property
    def tree_krope(self):
        return self.tree_kv[:, :, self.dc:]


def to_device(inp: workloads.Inputs) -> DevInputs:
    kv = inp.kv_cache
    if kv.shape[0] == 0:                        # keep a valid (aligned) allocation
        kv = torch.zeros((1, kv.shape[1]), dtype=kv.dtype)
    return DevInputs(parents=inp.parents.cuda(), cache_lens=inp.cache_lens.cuda(), q_lat=inp.q_lat.cuda(),
                     q_rope=inp.q_rope.cuda(), kv=kv.cuda(), tree_kv=inp.tree_kv.cuda(), dc=inp.spec.d_latent)


def run_gpu(inp: workloads.Inputs, dev: DevInputs = None, staged=False, max_len=None):
    """Masks [B,N,W] (numpy uint64) and outputs [B,N,H,d_c] (torch fp32, on device).

    staged: False = kdt_build_visibility + kdt_tree_verify_attn; True = visibility, plan,
    attend, combine as separate calls; "prepare" = kdt_tree_verify_prepare (masks and plan
    in one launch), attend, combine; "one" = kdt_tree_verify_prepare_attend (masks, plan and
    attention in one launch where the batch allows), combine.  max_len: the cache-length bound
    the geometry is made for (default: the longest request)."""
    dev = dev or to_device(inp)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    maxL = int(inp.cache_lens.max()) if inp.cache_lens.numel() else 0
    maxL = maxL if max_len is None else max_len
    total = inp.total_len
    if staged == "one":
        desc = kdt.make_desc(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, maxL, total)
        ws = kdt.alloc_workspace(desc)
        out = torch.empty(dev.q_lat.shape, dtype=torch.float32, device="cuda")
        masks = kdt.prepare_attend(dev.parents, dev.cache_lens, dev.q_lat, dev.q_rope, dev.ckv, dev.krope,
                                   dev.tree_ckv, dev.tree_krope, inp.scale, out, desc, ws, dev_status=status)
        kdt.combine(out, desc, ws)
        torch.cuda.synchronize()
        return masks.cpu().numpy().view(np.uint64), out, int(status.item())
    if staged == "prepare":
        desc = kdt.make_desc(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, maxL, total)
        ws = kdt.alloc_workspace(desc)
        out = torch.empty(dev.q_lat.shape, dtype=torch.float32, device="cuda")
        masks = kdt.prepare(dev.parents, dev.cache_lens, desc, ws, dev_status=status)
        kdt.attend(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, masks, inp.scale, out,
                   desc, ws)
        kdt.combine(out, desc, ws)
        torch.cuda.synchronize()
        return masks.cpu().numpy().view(np.uint64), out, int(status.item())
    masks = kdt.build_visibility(dev.parents, dev_status=status)
    if not staged:
        out = kdt.tree_verify_attn(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, masks,
                                   dev.cache_lens, inp.scale, dev_status=status, max_cache_len=maxL,
                                   total_cache_len=total)
    else:
        desc = kdt.make_desc(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, maxL, total)
        ws = kdt.alloc_workspace(desc)
        out = torch.empty(dev.q_lat.shape, dtype=torch.float32, device="cuda")
        kdt.plan(dev.cache_lens, desc, ws, dev_status=status)
        kdt.attend(dev.q_lat, dev.q_rope, dev.ckv, dev.krope, dev.tree_ckv, dev.tree_krope, masks, inp.scale, out,
                   desc, ws)
        kdt.combine(out, desc, ws)
    torch.cuda.synchronize()
    return masks.cpu().numpy().view(np.uint64), out, int(status.item())


def report(name: str, err: float, tol: float):
    line = f"{'PASS' if err <= tol else 'FAIL'} {name}: max-abs {err:.3e} (tol {tol:.0e})"
    print(line, flush=True)
    sys.stdout.flush()
    return line
