"""Full-size parity: every workload at its real shape, run through moe_forward
exactly as the benchmark launches it.

Routing-locked mode (the bit-exact contract): the oracle's gating runs on the
float32 logits the GPU wrote, and the GPU's selections, weights, counts,
offsets, row map and slot map must equal the oracle's bit for bit on every
token.  The outputs of sampled tokens, which the oracle computes one by one
from those same logits, must then be within tolerance with no token left out.

Independent mode: the oracle also computes its own logits for every token.
Tokens whose selection differs between the two ("flips") are counted and
reported; each must be a near tie (the oracle's selection-boundary gap within
4x the largest logit difference).

Inputs are generated on the GPU with seeded generators; the oracle receives
host copies of the same tensors.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import DEV, TOL, rel_err, run_forward, token_choice_flips

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().to("cpu").float().numpy() if t.dtype != torch.int32 else t.detach().cpu().numpy()


def _sample(T, n):
    return np.unique(np.concatenate([[0, T - 1], np.linspace(0, T - 1, n).astype(np.int64)]))


def _spec_capacity(spec):
    if spec.gating == "expert_choice":
        return oracle.capacity(spec.capacity_factor, spec.T, spec.E)
    if spec.gating == "switch" or spec.capacity_factor > 0:
        group = spec.capacity_group or spec.T
        return oracle.capacity_topk(spec.capacity_factor, group, spec.k, spec.E, spec.min_capacity)
    return 0


def _check_routing_locked(spec, routing):
    """GPU routing buffers against the oracle's gating and permutation of the
    GPU's own logits, bit for bit.  Returns the oracle's routing."""
    T, E = spec.T, spec.E
    lg = _np(routing["logits"]).reshape(T, E)
    cap = _spec_capacity(spec)
    counts, offsets = _np(routing["counts"]), _np(routing["offsets"])
    if spec.gating == "expert_choice":
        ec_idx, ec_score = oracle.route_expert_choice(lg, cap)
        assert np.array_equal(_np(routing["topk_idx"]).reshape(E, cap), ec_idx)
        np.testing.assert_allclose(_np(routing["topk_w"]).reshape(E, cap), ec_score, rtol=1e-5, atol=1e-30)
        assert np.array_equal(counts, np.full(E, cap))
        assert np.array_equal(offsets, np.arange(E + 1) * cap)
        assert np.array_equal(_np(routing["row_token"]), ec_idx.reshape(-1))
        sr = np.full((T, E), -1, np.int64)
        for e in range(E):
            sr[ec_idx[e], e] = e * cap + np.arange(cap)
        assert np.array_equal(_np(routing["slot_row"]).reshape(T, E), sr)
        return dict(logits=lg, ec_idx=ec_idx, capacity=cap, counts=counts)
    idx, w = oracle.route_topk(lg, spec.k, spec.gating)
    assert np.array_equal(_np(routing["topk_idx"]).reshape(T, spec.k), idx)
    np.testing.assert_allclose(_np(routing["topk_w"]).reshape(T, spec.k), w, rtol=2e-6, atol=1e-30)
    perm = oracle.permute(idx, E, cap, spec.capacity_group if cap else 0)
    n = perm["kept"]
    assert np.array_equal(counts, perm["counts"])
    assert np.array_equal(offsets, perm["offsets"])
    assert np.array_equal(_np(routing["row_token"])[:n], perm["row_token"])
    assert np.array_equal(_np(routing["slot_row"]).reshape(T, spec.k), perm["slot_row"])
    return dict(logits=lg, topk_idx=idx, capacity=cap, counts=counts, kept=n)


def _independent_flips(spec, inp, locked):
    """Tokens (token choice) or expert selections (expert choice) that differ
    when the oracle routes from its own logits; every one must be a near tie."""
    T, E = spec.T, spec.E
    or_lg = oracle.logits(inp["x"], inp["wg"], inp["bg"])
    gpu_lg = locked["logits"]
    dl = float(np.abs(gpu_lg.astype(np.float64) - or_lg).max())
    rep = dict(max_abs_logit_diff=dl)
    if spec.gating == "expert_choice":
        C = locked["capacity"]
        or_idx, _ = oracle.route_expert_choice(or_lg, C)
        experts, tokens = 0, set()
        for e in range(E):
            gs, os_ = set(locked["ec_idx"][e].tolist()), set(or_idx[e].tolist())
            if gs != os_:
                col = np.sort(or_lg[:, e].astype(np.float64))[::-1]
                assert col[C - 1] - col[C] <= 4 * dl + 1e-30, f"expert {e}: selection differs beyond a near tie"
                experts += 1
                tokens |= gs ^ os_
        rep.update(flipped_experts=experts, flipped_tokens=len(tokens))
        return rep
    or_idx, _ = oracle.route_topk(or_lg, spec.k, spec.gating)
    flips, near, _ = token_choice_flips(locked["topk_idx"], or_idx, gpu_lg, or_lg, spec.k)
    assert near.all(), f"routing flips that are not near ties: {flips[~near][:10]}"
    rep.update(flipped_tokens=len(flips))
    if locked["capacity"]:
        # a flip can shift the positions (and keep status) of later tokens of
        # the same (capacity group, expert): count the tokens whose kept set differs
        group = spec.capacity_group if locked["capacity"] else 0
        or_perm = oracle.permute(or_idx, E, locked["capacity"], group)
        gpu_perm = oracle.permute(locked["topk_idx"], E, locked["capacity"], group)
        kept_g = np.where(gpu_perm["slot_row"] >= 0, locked["topk_idx"], -1)
        kept_o = np.where(or_perm["slot_row"] >= 0, or_idx, -1)
        rep.update(flip_affected_tokens=int((np.sort(kept_g, 1) != np.sort(kept_o, 1)).any(1).sum()),
                   dropped_assignments=int(T * spec.k - gpu_perm["kept"]))
    return rep


@pytest.mark.parametrize("spec", workloads.FULL, ids=lambda s: s.name)
def test_full_size_routing_locked_and_independent(spec):
    inp = workloads.make_inputs(spec, device=DEV)
    y, routing = run_forward(spec, inp)
    locked = _check_routing_locked(spec, routing)
    # outputs of sampled tokens, routed by the GPU's logits: no token excluded
    toks = _sample(spec.T, 16 if spec.T > 16 else spec.T)
    ref = oracle.forward_tokens(spec, inp, toks, lg=locked["logits"])
    err = rel_err(_np(y)[toks], ref["y64"])
    assert err <= TOL[spec.dtype], f"max rel err {err}"
    rep = _independent_flips(spec, inp, locked)
    counts = locked["counts"]
    print(f"[parity] {spec.name}: routing-locked bit-exact on {spec.T} tokens; sampled {len(toks)} tokens "
          f"max rel err {err:.3e}; independent routing {rep}; load max/avg "
          f"{counts.max() / max(counts.mean(), 1e-30):.2f}, empty experts {(counts == 0).sum()}", flush=True)


def test_forward_with_x_of_two_gib():
    """x of exactly 2 GiB (T = 131072, d = 8192): one 32-bit buffer offset no
    longer spans it, so the forward pass gathers the routed rows with the
    gather kernel before the first GEMM instead of inside it; 64-bit row
    offsets throughout.  Routing locked to the GPU's logits (bit-exact on every
    token), sampled tokens against the oracle."""
    spec = workloads.MIXTRAL_PREFILL_BF16.replace(name="x_two_gib", T=131072, d=8192, E=4, k=1, F=64)
    assert spec.T * spec.d * 2 == 1 << 31
    inp = workloads.make_inputs(spec, device=DEV)
    y, routing = run_forward(spec, inp)
    locked = _check_routing_locked(spec, routing)
    assert (locked["counts"] > 0).all()
    toks = _sample(spec.T, 12)
    ref = oracle.forward_tokens(spec, inp, toks, lg=locked["logits"])
    ys = _np(y[torch.from_numpy(toks).to(DEV)])
    err = rel_err(ys, ref["y64"])
    print(f"[parity] x_two_gib: sampled {len(toks)} tokens, max rel err {err:.3e}", flush=True)
    assert err <= TOL[spec.dtype]
    del inp, y, routing
    torch.cuda.empty_cache()
