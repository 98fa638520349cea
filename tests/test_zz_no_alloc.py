"""moe_permute_noalloc (the permutation with its scratch in a fixed device
array of the library instead of a caller workspace) against moe_permute on
the same inputs: every routing buffer and the gathered rows bit for bit, on
two calls in a row, the second with a smaller batch (the array keeps the
first call's contents)."""
import numpy as np
import pytest
import torch

import sparse_mixture_experts_gating_amd as moe
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (T, E, k, capacity_factor, group): both past the one-workgroup path, so the
# count / scan / scatter kernels run on the scratch; the second is smaller and
# drops assignments at a per-group capacity.
CALLS = [(8192, 256, 8, 0.0, 0), (3000, 64, 6, 1.0, 1024)]


def _run(T, E, k, cf, group, noalloc):
    spec = workloads.MIXTRAL_PREFILL_BF16.replace(name="noalloc", T=T, d=256, E=E, k=k, F=64,
                                                  capacity_factor=cf, capacity_group=group)
    cfg = moe.config_from_spec(spec)
    idx = workloads.random_topk_idx(T, E, k, seed=900 + T + E, skew=1.1)
    x = workloads.make_inputs(spec, device=DEV, experts=False)["x"]
    r = moe.alloc_routing(cfg, DEV)
    r["topk_idx"].copy_(idx.reshape(-1).to(DEV))
    x_perm = torch.full((T * k, spec.d), -7.0, dtype=torch.bfloat16, device=DEV)
    if noalloc:
        moe.moe_permute_noalloc(cfg, x, moe.make_routing(r), x_perm)
    else:
        ws = moe.alloc_workspace(cfg, moe.STAGE_PERMUTE, DEV)
        moe.moe_permute(cfg, x, moe.make_routing(r), x_perm, ws)
    torch.cuda.synchronize()
    return r, x_perm


def test_permute_noalloc_equals_permute_on_two_calls():
    for T, E, k, cf, group in CALLS:
        print(f"[noalloc] T={T} E={E} k={k} cf={cf} group={group}", flush=True)
        want, want_x = _run(T, E, k, cf, group, noalloc=False)
        got, got_x = _run(T, E, k, cf, group, noalloc=True)
        for key in ("counts", "offsets", "slot_row"):
            assert torch.equal(got[key], want[key]), key
        n = int(want["offsets"][-1])
        assert torch.equal(got["row_token"][:n], want["row_token"][:n])
        assert torch.equal(got_x, want_x)
        if cf > 0:
            assert n < T * k  # the capacity dropped assignments
