"""Full-size parity: every workload at its real shape, run through moe_forward
exactly as the benchmark launches it, checked on sampled tokens that the
oracle computes one by one (plus routing-wide properties that hold at any size).

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
    s = np.unique(np.concatenate([[0, T - 1], np.linspace(0, T - 1, n).astype(np.int64)]))
    return s


@pytest.mark.parametrize("spec", workloads.FULL, ids=lambda s: s.name)
def test_full_size_sampled_tokens(spec):
    inp = workloads.make_inputs(spec, device=DEV)
    y, routing = run_forward(spec, inp)
    T, E = spec.T, spec.E
    counts = _np(routing["counts"])
    offsets = _np(routing["offsets"])
    # properties that hold at any size
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    if spec.gating == "expert_choice":
        C = oracle.capacity(spec.capacity_factor, T, E)
        assert (counts == C).all()
        ec = _np(routing["topk_idx"]).reshape(E, C)
        assert all(len(set(r.tolist())) == C for r in ec)
    elif spec.gating == "switch":
        C = oracle.capacity(spec.capacity_factor, spec.capacity_group, E)
        idx = _np(routing["topk_idx"]).reshape(T)
        G = spec.capacity_group
        want = sum(min(int((idx[g0:g0 + G] == e).sum()), C) for g0 in range(0, T, G) for e in range(E))
        assert counts.sum() == want
    else:
        assert counts.sum() == T * spec.k
        w = _np(routing["topk_w"]).reshape(T, spec.k).astype(np.float64)
        assert np.allclose(w.sum(1), 1.0, atol=1e-5)
    # sampled tokens against the oracle
    toks = _sample(T, 12 if T > 16 else T)
    ref = oracle.forward_tokens(spec, inp, toks)
    gpu_lg = _np(routing["logits"])
    ok = np.ones(len(toks), bool)
    if spec.gating == "expert_choice":
        or_lg = oracle.logits(inp["x"], inp["wg"], inp["bg"])
        dl = float(np.abs(gpu_lg.astype(np.float64) - or_lg).max())
        for e in range(E):
            gs, os_ = set(ec[e].tolist()), set(ref["ec_idx"][e].tolist())
            if gs != os_:
                col = np.sort(or_lg[:, e].astype(np.float64))[::-1]
                assert col[C - 1] - col[C] <= 4 * dl + 1e-30
                ok &= ~np.isin(toks, list(gs ^ os_))
    elif spec.gating == "switch":
        or_lg = oracle.logits(inp["x"], inp["wg"], inp["bg"])
        or_idx, _ = oracle.route_topk(or_lg, 1, "switch")
        flips, near, _ = token_choice_flips(idx, or_idx, gpu_lg, or_lg, 1)
        assert near.all()
        touched = {(t // G, idx[t]) for t in flips} | {(t // G, or_idx[t, 0]) for t in flips}
        for i, t in enumerate(toks):
            if (t // G, idx[t]) in touched or (t // G, or_idx[t, 0]) in touched:
                ok[i] = False
    else:
        flips, near, _ = token_choice_flips(_np(routing["topk_idx"]).reshape(T, spec.k)[toks], ref["topk_idx"],
                                            gpu_lg[toks], ref["logits_sel"], spec.k)
        assert near.all()
        ok[flips] = False
    assert ok.sum() >= len(toks) - 2
    err = rel_err(_np(y)[toks][ok], ref["y64"][ok])
    print(f"{spec.name}: sampled {ok.sum()} tokens, max rel err {err:.3e}, flips excluded {(~ok).sum()}")
    assert err <= TOL[spec.dtype]


def test_forward_with_x_of_two_gib():
    """x of exactly 2 GiB (T = 131072, d = 8192): one 32-bit buffer offset no
    longer spans it, so the forward pass gathers the routed rows with the
    gather kernel before the first GEMM instead of inside it; 64-bit row
    offsets throughout.  Sampled tokens against the oracle."""
    spec = workloads.MIXTRAL_PREFILL_BF16.replace(name="x_two_gib", T=131072, d=8192, E=4, k=1, F=64)
    assert spec.T * spec.d * 2 == 1 << 31
    inp = workloads.make_inputs(spec, device=DEV)
    y, routing = run_forward(spec, inp)
    counts = _np(routing["counts"])
    assert counts.sum() == spec.T and (counts > 0).all()
    toks = _sample(spec.T, 12)
    ref = oracle.forward_tokens(spec, inp, toks)
    flips, near, _ = token_choice_flips(_np(routing["topk_idx"]).reshape(spec.T, 1)[toks], ref["topk_idx"],
                                        _np(routing["logits"]).reshape(spec.T, spec.E)[toks], ref["logits_sel"], 1)
    assert near.all()
    ok = np.ones(len(toks), bool)
    ok[flips] = False
    ys = _np(y[torch.from_numpy(toks).to(DEV)])
    err = rel_err(ys[ok], ref["y64"][ok])
    print(f"x_two_gib: sampled {ok.sum()} tokens, max rel err {err:.3e}")
    assert err <= TOL[spec.dtype]
    del inp, y, routing
    torch.cuda.empty_cache()
